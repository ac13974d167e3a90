"""Block-sparse attention with top-k block selection for AMD MI355X (gfx950).

The kernels live in libbsattn.so (C ABI, include/bsattn.h); `bsattn` is its binding.
Importing the package does not load the library; the first call does, and raises if
it is not built.
"""
from .bsattn import (CAUSAL, GROUP_SELECT, POOL_MAX, BsattnError,  # noqa: F401
                     backward, block_sparse_attention, decode, decode_pool, forward, key_blocks,
                     lib,
                     select, select_workspace_bytes, topk_count)
