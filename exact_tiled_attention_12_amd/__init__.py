"""Exact tiled attention (fused forward + recomputing backward) for MI355X / gfx950.

The compute lives in libattn.so (HIP kernels behind the C ABI in
include/attn.h); this package holds its ctypes binding, the autograd wrapper, the build step, the
workload shapes, the seeded input generator and the FLOP accounting.
"""
from .attn import (attn_bwd, attn_bwd_blocksparse, attn_bwd_noalloc, attn_bwd_dkdv, attn_bwd_dq, attn_bwd_dq_d, attn_bwd_main,  # noqa: F401
                   attn_bwd_preprocess, attn_bwd_workspace_bytes, attn_fwd, attn_fwd_blocksparse, attn_fwd_fp8, lib,
                   prepare, AttnError, LIB_PATH, MASK_BLOCK)
from .autograd import FlashAttentionFn, flash_attention  # noqa: F401
