"""libmiattn: fused exact attention for AMD MI355X (gfx950).

The compute lives in the HIP library ``libmiattn.so`` (C ABI, declared in
include/miattn.h); this package is its thin ctypes binding plus the build
script.  Functions carry the C names and take device tensors:

    attn_fwd, attn_bwd, attn_bwd_workspace_bytes,
    attn_bwd_preprocess, attn_bwd_dkdv, attn_bwd_dq, attn_bwd_dq_preprocess,
    attn_fwd_gqa, attn_bwd_gqa,
    attn_fwd_window, attn_bwd_window,
    attn_fwd_block_sparse, attn_bwd_block_sparse, attn_bwd_block_sparse_workspace_bytes,
    attn_decode, attn_decode_workspace_bytes,
    attn_quantize_fp8_rows, attn_quantize_fp8_vt, attn_fwd_fp8,
    attn_fwd_f32, attn_bwd_f32, attn_bwd_f32_workspace_bytes,
    attn_fwd_varlen, attn_bwd_varlen, attn_bwd_varlen_workspace_bytes

plus check_cu_seqlens (host-side validation of packed offsets).
"""
from ._lib import (  # noqa: F401
    LIB_PATH,
    MiattnError,
    attn_bwd,
    attn_bwd_dkdv,
    attn_bwd_dq,
    attn_bwd_dq_preprocess,
    attn_bwd_f32,
    attn_bwd_f32_workspace_bytes,
    attn_bwd_gqa,
    attn_bwd_noalloc,
    attn_bwd_noalloc_max_rows,
    attn_bwd_block_sparse,
    attn_bwd_block_sparse_workspace_bytes,
    attn_bwd_window,
    attn_bwd_preprocess,
    attn_bwd_varlen,
    attn_bwd_varlen_workspace_bytes,
    attn_bwd_workspace_bytes,
    attn_decode,
    attn_decode_workspace_bytes,
    attn_fwd,
    attn_fwd_f32,
    attn_fwd_fp8,
    attn_fwd_block_sparse,
    attn_fwd_gqa,
    attn_fwd_window,
    attn_fwd_varlen,
    attn_quantize_fp8_rows,
    attn_quantize_fp8_vt,
    check_cu_seqlens,
    load,
    miattn_status_string,
    miattn_version,
)
