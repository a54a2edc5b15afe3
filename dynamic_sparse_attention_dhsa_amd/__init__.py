"""MI355X-native DHSA chunk-routed sparse causal prefill.

The compute path is the HIP library built from ``csrc/`` for gfx950.  The
functions re-exported here (from ``binding``) only marshal torch tensors into
the C ABI declared in ``include/dhsa.h``.
"""
from .binding import (DecodeState, DhsaError, Layout, RoutePlan, adjacent_similarity, chunk_boundaries,  # noqa: F401
                      SeqLayout, TokenPlan, chunk_summarize, load_library, online_chunks, prefill, route,
                      route_tokens, sparse_prefill)
