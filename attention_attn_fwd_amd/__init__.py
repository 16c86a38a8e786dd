"""MI355X-native causal GQA attention forward.

The compute path is libattn_fwd.so (hand-written HIP kernels for gfx950 behind
a C ABI, include/attn_fwd.h); this package only marshals arguments to it.
Importing the package does not load the library; the first call does, and
raises if the library is not built (there is no CPU fallback).
"""
from ._binding import (  # noqa: F401
    ATTN_ERR_HIP, ATTN_ERR_INVALID_ARG, ATTN_ERR_OOM, ATTN_ERR_SCRATCH_LIMIT, ATTN_ERR_UNSUPPORTED, ATTN_FWD_FP16,
    ATTN_FWD_FP32, ATTN_FWD_NONCAUSAL, ATTN_OK, EXPORTS, LIB_PATH, PATH_DECODE, PATH_NONE, PATH_PREFILL, AttnError,
    attn_bwd, attn_fwd, attn_fwd_ex, attn_fwd_f32, attn_fwd_noalloc, attn_fwd_paged, attn_fwd_plan,
    attn_fwd_release_scratch, attn_fwd_strerror, backward, forward, forward_paged, load, strerror,
)
