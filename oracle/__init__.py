"""CPU oracle for DHSA chunk-routed sparse causal prefill, for this project's online
chunk-boundary rule, for decode against the kept structure and for routing under a token
budget (test infrastructure only).

Only tests/, ``__graft_entry__.smoke()`` and bench.py's ``cpu_baseline`` leg
import this package.  It shares no code with the HIP path.
"""
from .dhsa_oracle import (attend, chunk_scores, chunk_sequence, chunk_summaries,  # noqa: F401
                          dense_attention, group_chunk_scores, kept_token_mask, prefill, route,
                          route_grouped, route_plan, select_key_chunks, token_importance,
                          validate_layout)
from .chunking_oracle import adjacent_similarity, chunk_boundaries  # noqa: F401,E402
from .decode_oracle import decode_sequence  # noqa: F401,E402
from .budget_oracle import route_plan_tokens, route_tokens, select_key_chunks_tokens  # noqa: F401,E402
