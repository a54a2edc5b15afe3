"""MI355X-native DHSA chunk-routed sparse causal prefill.

The compute path is the HIP library built from ``csrc/`` (gfx950).  The
Python functions in ``binding`` only marshal torch tensors into the C ABI
declared in ``include/dhsa.h``.
"""
