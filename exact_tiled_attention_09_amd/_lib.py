"""ctypes binding of libmiattn (argument marshalling only).

Every function here has the name of a C entry point in include/miattn.h,
takes torch tensors that already live on the GPU, passes their data pointers
and sizes to the library, and raises MiattnError on a nonzero status.  No
arithmetic of the method happens in Python, and there is no fallback: if the
shared library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmiattn.so")

MIATTN_OK = 0
MIATTN_ERR_INVALID_ARG = -1
MIATTN_ERR_UNSUPPORTED = -2
MIATTN_ERR_HIP = -3

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_S = ctypes.c_size_t

# name -> (restype, argtypes)
SIGNATURES = {
    "miattn_version": (_I, []),
    "miattn_status_string": (ctypes.c_char_p, [_I]),
    "attn_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P]),
    "attn_bwd_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "attn_bwd_f32_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "attn_bwd": (_I, [_P] * 9 + [_I, _I, _I, _I, _F, _I, _P, _S, _P]),
    "attn_bwd_preprocess": (_I, [_P, _P, _I, _I, _I, _I, _P, _S, _P]),
    "attn_bwd_dkdv": (_I, [_P] * 7 + [_I, _I, _I, _I, _F, _I, _P, _S, _P]),
    "attn_bwd_dq": (_I, [_P] * 6 + [_I, _I, _I, _I, _F, _I, _P, _S, _P]),
    "attn_fwd_gqa": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_bwd_gqa": (_I, [_P] * 9 + [_I, _I, _I, _I, _I, _F, _I, _P, _S, _P]),
    "attn_fwd_window": (_I, [_P] * 5 + [_I] * 5 + [_F, _I, _I, _I, _P]),
    "attn_bwd_window": (_I, [_P] * 9 + [_I] * 5 + [_F, _I, _I, _I, _P, _S, _P]),
    "attn_fwd_block_sparse": (_I, [_P] * 5 + [_I] * 5 + [_F, _I, _P, _P, _I, _P]),
    "attn_bwd_block_sparse_workspace_bytes": (_S, [_I, _I, _I, _I, _I, _I]),
    "attn_bwd_block_sparse": (_I, [_P] * 9 + [_I] * 5 + [_F, _I, _P, _P, _I, _P, _S, _P]),
    "attn_decode_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "attn_decode": (_I, [_P] * 5 + [_I] * 5 + [_F, _P, _P, _S, _P]),
    "attn_quantize_fp8_rows": (_I, [_P, _P, _P, _I, _I, _I, _I, _P]),
    "attn_quantize_fp8_vt": (_I, [_P, _P, _P, _I, _I, _I, _I, _P]),
    "attn_fwd_fp8": (_I, [_P] * 8 + [_I] * 5 + [_F, _I, _P]),
    "attn_fwd_f32": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P]),
    "attn_bwd_f32": (_I, [_P] * 9 + [_I, _I, _I, _I, _F, _I, _P, _S, _P]),
    "attn_fwd_varlen": (_I, [_P] * 5 + [_P, _I, _I, _I, _I, _I, _F, _I, _P, _P]),
    "attn_bwd_varlen_workspace_bytes": (_S, [_I, _I, _I]),
    "attn_bwd_varlen": (_I, [_P] * 9 + [_P, _I, _I, _I, _I, _I, _F, _I, _P, _P, _S, _P]),
}


class MiattnError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libmiattn.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m exact_tiled_attention_09_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmiattn takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("libmiattn takes contiguous tensors only")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, status: int):
    if status != MIATTN_OK:
        raise MiattnError(fn, status, load().miattn_status_string(status).decode())


def _dense_dims(q):
    if q.dim() != 4:
        raise ValueError("dense tensors are [B, H, N, d]")
    B, H, N, d = q.shape
    return int(B), int(H), int(N), int(d)


def miattn_version() -> int:
    return load().miattn_version()


def miattn_status_string(status: int) -> str:
    return load().miattn_status_string(status).decode()


def attn_fwd(q, k, v, o, lse, scale: float, causal: bool, stream=None):
    B, H, N, d = _dense_dims(q)
    _check("attn_fwd", load().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                                       float(scale), int(bool(causal)), _stream(stream)))


def attn_bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(load().attn_bwd_workspace_bytes(B, H, N, d))


def attn_bwd(q, k, v, o, lse, dO, dq, dk, dv, scale: float, causal: bool, workspace, stream=None):
    B, H, N, d = _dense_dims(q)
    _check("attn_bwd", load().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq),
                                       _ptr(dk), _ptr(dv), B, H, N, d, float(scale), int(bool(causal)),
                                       _ptr(workspace), workspace.numel() * workspace.element_size(),
                                       _stream(stream)))


def attn_bwd_preprocess(o, dO, workspace, stream=None):
    B, H, N, d = _dense_dims(o)
    _check("attn_bwd_preprocess", load().attn_bwd_preprocess(_ptr(o), _ptr(dO), B, H, N, d, _ptr(workspace),
                                                             workspace.numel() * workspace.element_size(),
                                                             _stream(stream)))


def attn_bwd_dkdv(q, k, v, lse, dO, dk, dv, scale: float, causal: bool, workspace, stream=None):
    B, H, N, d = _dense_dims(q)
    _check("attn_bwd_dkdv", load().attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dO), _ptr(dk),
                                                 _ptr(dv), B, H, N, d, float(scale), int(bool(causal)),
                                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                                 _stream(stream)))


def attn_bwd_dq(q, k, v, lse, dO, dq, scale: float, causal: bool, workspace, stream=None):
    B, H, N, d = _dense_dims(q)
    _check("attn_bwd_dq", load().attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dO), _ptr(dq), B, H, N, d,
                                             float(scale), int(bool(causal)), _ptr(workspace),
                                             workspace.numel() * workspace.element_size(), _stream(stream)))


def _gqa_dims(q, k):
    B, H, N, d = _dense_dims(q)
    if k.dim() != 4 or int(k.shape[0]) != B or int(k.shape[2]) != N or int(k.shape[3]) != d:
        raise ValueError("grouped K/V are [B, H_kv, N, d] with the B, N, d of Q")
    return B, H, int(k.shape[1]), N, d


def attn_fwd_gqa(q, k, v, o, lse, scale: float, causal: bool, stream=None):
    B, H, Hkv, N, d = _gqa_dims(q, k)
    _check("attn_fwd_gqa", load().attn_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d,
                                               float(scale), int(bool(causal)), _stream(stream)))


def attn_bwd_gqa(q, k, v, o, lse, dO, dq, dk, dv, scale: float, causal: bool, workspace, stream=None):
    B, H, Hkv, N, d = _gqa_dims(q, k)
    _check("attn_bwd_gqa", load().attn_bwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
                                               _ptr(dq), _ptr(dk), _ptr(dv), B, H, Hkv, N, d, float(scale),
                                               int(bool(causal)), _ptr(workspace),
                                               workspace.numel() * workspace.element_size(), _stream(stream)))


def attn_fwd_window(q, k, v, o, lse, scale: float, causal: bool, window_left: int, window_right: int,
                    stream=None):
    B, H, Hkv, N, d = _gqa_dims(q, k)
    _check("attn_fwd_window", load().attn_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d,
                                                     float(scale), int(bool(causal)), int(window_left),
                                                     int(window_right), _stream(stream)))


def attn_bwd_window(q, k, v, o, lse, dO, dq, dk, dv, scale: float, causal: bool, window_left: int,
                    window_right: int, workspace, stream=None):
    B, H, Hkv, N, d = _gqa_dims(q, k)
    _check("attn_bwd_window", load().attn_bwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
                                                     _ptr(dq), _ptr(dk), _ptr(dv), B, H, Hkv, N, d, float(scale),
                                                     int(bool(causal)), int(window_left), int(window_right),
                                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                                     _stream(stream)))


def attn_fwd_block_sparse(q, k, v, o, lse, scale: float, causal: bool, row_ptr, col_idx, stream=None):
    """row_ptr, col_idx: int32 device tensors (the CSR block list)."""
    B, H, Hkv, N, d = _gqa_dims(q, k)
    _check("attn_fwd_block_sparse",
           load().attn_fwd_block_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d,
                                        float(scale), int(bool(causal)), _ptr(row_ptr), _ptr(col_idx),
                                        int(col_idx.numel()), _stream(stream)))


def attn_bwd_block_sparse_workspace_bytes(B: int, H: int, H_kv: int, N: int, d: int, nnz: int) -> int:
    return int(load().attn_bwd_block_sparse_workspace_bytes(B, H, H_kv, N, d, nnz))


def attn_bwd_block_sparse(q, k, v, o, lse, dO, dq, dk, dv, scale: float, causal: bool, row_ptr, col_idx,
                          workspace, stream=None):
    B, H, Hkv, N, d = _gqa_dims(q, k)
    _check("attn_bwd_block_sparse",
           load().attn_bwd_block_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq),
                                        _ptr(dk), _ptr(dv), B, H, Hkv, N, d, float(scale), int(bool(causal)),
                                        _ptr(row_ptr), _ptr(col_idx), int(col_idx.numel()), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream)))


def attn_decode_workspace_bytes(B: int, H: int, H_kv: int, N_kv: int, d: int) -> int:
    return int(load().attn_decode_workspace_bytes(B, H, H_kv, N_kv, d))


def attn_decode(q, k_cache, v_cache, o, lse, scale: float, cache_seqlens, workspace, stream=None):
    """q, o: [B, H, d]; k_cache, v_cache: [B, H_kv, N_kv, d]; lse: [B, H];
    cache_seqlens: int32 device tensor [B] or None."""
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q is [B, H, d] and the caches are [B, H_kv, N_kv, d]")
    B, H, d = (int(x) for x in q.shape)
    Hkv, N = int(k_cache.shape[1]), int(k_cache.shape[2])
    if int(k_cache.shape[0]) != B or int(k_cache.shape[3]) != d:
        raise ValueError("the caches must have the B and d of q")
    sl = None if cache_seqlens is None else _ptr(cache_seqlens)
    _check("attn_decode", load().attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), B, H, Hkv,
                                             N, d, float(scale), sl, _ptr(workspace),
                                             workspace.numel() * workspace.element_size(), _stream(stream)))


def attn_quantize_fp8_rows(x, x8, scales, stream=None):
    """x bf16 [B, H, N, d] -> x8 uint8 [B, H, N, d], scales fp32 [B, H, ceil(N/64)]."""
    B, H, N, d = _dense_dims(x)
    _check("attn_quantize_fp8_rows", load().attn_quantize_fp8_rows(_ptr(x), _ptr(x8), _ptr(scales), B, H, N, d,
                                                                   _stream(stream)))


def attn_quantize_fp8_vt(v, v8t, scales, stream=None):
    """v bf16 [B, H, N, d] -> v8t uint8 [B, H, ceil(N/64), d, 64], scales fp32 [B, H]."""
    B, H, N, d = _dense_dims(v)
    _check("attn_quantize_fp8_vt", load().attn_quantize_fp8_vt(_ptr(v), _ptr(v8t), _ptr(scales), B, H, N, d,
                                                               _stream(stream)))


def attn_fwd_fp8(q8, q_scale, k8, k_scale, v8t, v_scale, o, lse, scale: float, causal: bool, stream=None):
    B, H, N, d = _dense_dims(q8)
    Hkv = int(k8.shape[1])
    _check("attn_fwd_fp8", load().attn_fwd_fp8(_ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(v8t),
                                               _ptr(v_scale), _ptr(o), _ptr(lse), B, H, Hkv, N, d, float(scale),
                                               int(bool(causal)), _stream(stream)))


def attn_bwd_f32_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(load().attn_bwd_f32_workspace_bytes(B, H, N, d))


def attn_fwd_f32(q, k, v, o, lse, scale: float, causal: bool, stream=None):
    B, H, N, d = _dense_dims(q)
    _check("attn_fwd_f32", load().attn_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                                               float(scale), int(bool(causal)), _stream(stream)))


def attn_bwd_f32(q, k, v, o, lse, dO, dq, dk, dv, scale: float, causal: bool, workspace, stream=None):
    B, H, N, d = _dense_dims(q)
    _check("attn_bwd_f32", load().attn_bwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
                                               _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, float(scale),
                                               int(bool(causal)), _ptr(workspace),
                                               workspace.numel() * workspace.element_size(), _stream(stream)))


def _varlen_dims(q):
    if q.dim() != 3:
        raise ValueError("packed tensors are [T, H, d]")
    T, H, d = q.shape
    return int(T), int(H), int(d)


def attn_fwd_varlen(q, k, v, o, lse, cu_seqlens, max_seqlen: int, scale: float, causal: bool,
                    key_valid=None, stream=None):
    T, H, d = _varlen_dims(q)
    nseq = int(cu_seqlens.numel()) - 1
    _check("attn_fwd_varlen", load().attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                                     _ptr(cu_seqlens), nseq, int(max_seqlen), T, H, d,
                                                     float(scale), int(bool(causal)), _ptr(key_valid),
                                                     _stream(stream)))


def attn_bwd_varlen_workspace_bytes(total_tokens: int, H: int, d: int) -> int:
    return int(load().attn_bwd_varlen_workspace_bytes(total_tokens, H, d))


def attn_bwd_varlen(q, k, v, o, lse, dO, dq, dk, dv, cu_seqlens, max_seqlen: int, scale: float, causal: bool,
                    workspace, key_valid=None, stream=None):
    T, H, d = _varlen_dims(q)
    nseq = int(cu_seqlens.numel()) - 1
    _check("attn_bwd_varlen", load().attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
                                                     _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cu_seqlens), nseq,
                                                     int(max_seqlen), T, H, d, float(scale), int(bool(causal)),
                                                     _ptr(key_valid), _ptr(workspace),
                                                     workspace.numel() * workspace.element_size(),
                                                     _stream(stream)))
