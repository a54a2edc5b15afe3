"""MI355X-native DHSA chunk-routed sparse causal prefill.

The compute path is the HIP library built from ``csrc/`` for gfx950.  The
functions re-exported here (from ``binding``) only marshal torch tensors into
the C ABI declared in ``include/dhsa.h``.
"""
from .binding import (DhsaError, Layout, RoutePlan, chunk_summarize, load_library,  # noqa: F401
                      prefill, route, sparse_prefill)
