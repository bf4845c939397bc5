"""Sparse multi-head latent attention (MLA) forward for AMD MI355X (gfx950).

The compute path is libsmla.so (hand-written HIP kernels behind the C ABI in
include/smla.h); ``smla`` is its thin ctypes binding and ``inputs`` draws the
seeded synthetic workloads.
"""
from .smla import (KV_BF16, KV_FP8_GROUP128, KV_FP8_PER_TENSOR, SmlaError, cache_write,  # noqa: F401
                   convert_indices, decode_fwd, decode_num_splits, decode_workspace_size, load,
                   prefill_fwd, version)
