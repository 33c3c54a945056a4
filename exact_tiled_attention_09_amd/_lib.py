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
MIATTN_ERR_TOO_LARGE = -4

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
    "attn_bwd_noalloc": (_I, [_P] * 9 + [_I, _I, _I, _I, _F, _I, _P]),
    "attn_bwd_noalloc_max_rows": (_S, []),
    "attn_bwd_preprocess": (_I, [_P, _P, _I, _I, _I, _I, _P, _S, _P]),
    "attn_bwd_dkdv": (_I, [_P] * 7 + [_I, _I, _I, _I, _F, _I, _P, _S, _P]),
    "attn_bwd_dq": (_I, [_P] * 6 + [_I, _I, _I, _I, _F, _I, _P, _S, _P]),
    "attn_bwd_dq_preprocess": (_I, [_P] * 7 + [_I, _I, _I, _I, _F, _I, _P, _S, _P]),
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


_DTYPES = {}


def _dtype(name: str):
    if not _DTYPES:
        import torch
        _DTYPES.update(bfloat16=torch.bfloat16, float32=torch.float32, int32=torch.int32, uint8=torch.uint8)
    return _DTYPES[name]


def _expect(fn: str, *specs):
    """Each spec is (name, tensor, shape tuple, dtype name): the library sees
    raw pointers, so a tensor of the wrong shape or dtype would make its
    kernels read or write past the buffer; refuse it here, before any launch.
    (torch.Size compares with a tuple in C and dtypes by identity: the check
    stays far below a kernel launch in host time.)"""
    for name, t, shape, dtype in specs:
        if t is None or t.shape != shape or t.dtype is not _dtype(dtype):
            if t is None:
                raise ValueError(f"{fn}: {name} is required")
            if t.shape != shape:
                raise ValueError(f"{fn}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
            raise ValueError(f"{fn}: {name} is {t.dtype}, expected torch.{dtype}")


def _dense_dims(q):
    if q.dim() != 4:
        raise ValueError("dense tensors are [B, H, N, d]")
    B, H, N, d = q.shape
    return int(B), int(H), int(N), int(d)


def miattn_version() -> int:
    return load().miattn_version()


def miattn_status_string(status: int) -> str:
    return load().miattn_status_string(status).decode()


def _dense_specs(fn, dtype, B, H, N, d, **tensors):
    shapes = {"lse": (B, H, N)}
    specs = []
    for name, t in tensors.items():
        specs.append((name, t, shapes.get(name, (B, H, N, d)), "float32" if name == "lse" else dtype))
    _expect(fn, *specs)


def attn_fwd(q, k, v, o, lse, scale: float, causal: bool, stream=None):
    B, H, N, d = _dense_dims(q)
    _dense_specs("attn_fwd", "bfloat16", B, H, N, d, q=q, k=k, v=v, o=o, lse=lse)
    _check("attn_fwd", load().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                                       float(scale), int(bool(causal)), _stream(stream)))


def attn_bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(load().attn_bwd_workspace_bytes(B, H, N, d))


def attn_bwd(q, k, v, o, lse, dO, dq, dk, dv, scale: float, causal: bool, workspace, stream=None):
    B, H, N, d = _dense_dims(q)
    _dense_specs("attn_bwd", "bfloat16", B, H, N, d, q=q, k=k, v=v, o=o, lse=lse, dO=dO, dq=dq, dk=dk, dv=dv)
    _check("attn_bwd", load().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq),
                                       _ptr(dk), _ptr(dv), B, H, N, d, float(scale), int(bool(causal)),
                                       _ptr(workspace), workspace.numel() * workspace.element_size(),
                                       _stream(stream)))


def attn_bwd_noalloc_max_rows() -> int:
    return int(load().attn_bwd_noalloc_max_rows())


def attn_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, scale: float, causal: bool, stream=None):
    """attn_bwd without a workspace: D lives in the library's own device
    scratch (B*H*N <= attn_bwd_noalloc_max_rows()); calls overlapping on one
    GPU race."""
    B, H, N, d = _dense_dims(q)
    _dense_specs("attn_bwd_noalloc", "bfloat16", B, H, N, d, q=q, k=k, v=v, o=o, lse=lse, dO=dO, dq=dq, dk=dk,
                 dv=dv)
    _check("attn_bwd_noalloc", load().attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
                                                       _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, float(scale),
                                                       int(bool(causal)), _stream(stream)))


def attn_bwd_preprocess(o, dO, workspace, stream=None):
    B, H, N, d = _dense_dims(o)
    _dense_specs("attn_bwd_preprocess", "bfloat16", B, H, N, d, o=o, dO=dO)
    _check("attn_bwd_preprocess", load().attn_bwd_preprocess(_ptr(o), _ptr(dO), B, H, N, d, _ptr(workspace),
                                                             workspace.numel() * workspace.element_size(),
                                                             _stream(stream)))


def attn_bwd_dkdv(q, k, v, lse, dO, dk, dv, scale: float, causal: bool, workspace, stream=None):
    B, H, N, d = _dense_dims(q)
    _dense_specs("attn_bwd_dkdv", "bfloat16", B, H, N, d, q=q, k=k, v=v, lse=lse, dO=dO, dk=dk, dv=dv)
    _check("attn_bwd_dkdv", load().attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dO), _ptr(dk),
                                                 _ptr(dv), B, H, N, d, float(scale), int(bool(causal)),
                                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                                 _stream(stream)))


def attn_bwd_dq(q, k, v, lse, dO, dq, scale: float, causal: bool, workspace, stream=None):
    B, H, N, d = _dense_dims(q)
    _dense_specs("attn_bwd_dq", "bfloat16", B, H, N, d, q=q, k=k, v=v, lse=lse, dO=dO, dq=dq)
    _check("attn_bwd_dq", load().attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dO), _ptr(dq), B, H, N, d,
                                             float(scale), int(bool(causal)), _ptr(workspace),
                                             workspace.numel() * workspace.element_size(), _stream(stream)))


def attn_bwd_dq_preprocess(q, k, v, o, lse, dO, dq, scale: float, causal: bool, workspace, stream=None):
    B, H, N, d = _dense_dims(q)
    _dense_specs("attn_bwd_dq_preprocess", "bfloat16", B, H, N, d, q=q, k=k, v=v, o=o, lse=lse, dO=dO, dq=dq)
    _check("attn_bwd_dq_preprocess",
           load().attn_bwd_dq_preprocess(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq), B, H, N,
                                         d, float(scale), int(bool(causal)), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(stream)))


def _gqa_dims(q, k):
    B, H, N, d = _dense_dims(q)
    if k.dim() != 4 or int(k.shape[0]) != B or int(k.shape[2]) != N or int(k.shape[3]) != d:
        raise ValueError("grouped K/V are [B, H_kv, N, d] with the B, N, d of Q")
    return B, H, int(k.shape[1]), N, d


def _gqa_specs(fn, B, H, Hkv, N, d, **tensors):
    kv_names = ("k", "v", "dk", "dv")
    specs = []
    for name, t in tensors.items():
        if name == "lse":
            specs.append((name, t, (B, H, N), "float32"))
        else:
            specs.append((name, t, (B, Hkv if name in kv_names else H, N, d), "bfloat16"))
    _expect(fn, *specs)


def _block_list_specs(fn, N, row_ptr, col_idx):
    nqb = (N + 127) // 128
    if col_idx is None or col_idx.dim() != 1:
        raise ValueError(f"{fn}: col_idx is a 1-D int32 tensor")
    _expect(fn, ("row_ptr", row_ptr, (nqb + 1,), "int32"), ("col_idx", col_idx, (int(col_idx.numel()),), "int32"))


def attn_fwd_gqa(q, k, v, o, lse, scale: float, causal: bool, stream=None):
    B, H, Hkv, N, d = _gqa_dims(q, k)
    _gqa_specs("attn_fwd_gqa", B, H, Hkv, N, d, q=q, k=k, v=v, o=o, lse=lse)
    _check("attn_fwd_gqa", load().attn_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d,
                                               float(scale), int(bool(causal)), _stream(stream)))


def attn_bwd_gqa(q, k, v, o, lse, dO, dq, dk, dv, scale: float, causal: bool, workspace, stream=None):
    B, H, Hkv, N, d = _gqa_dims(q, k)
    _gqa_specs("attn_bwd_gqa", B, H, Hkv, N, d, q=q, k=k, v=v, o=o, lse=lse, dO=dO, dq=dq, dk=dk, dv=dv)
    _check("attn_bwd_gqa", load().attn_bwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
                                               _ptr(dq), _ptr(dk), _ptr(dv), B, H, Hkv, N, d, float(scale),
                                               int(bool(causal)), _ptr(workspace),
                                               workspace.numel() * workspace.element_size(), _stream(stream)))


def attn_fwd_window(q, k, v, o, lse, scale: float, causal: bool, window_left: int, window_right: int,
                    stream=None):
    B, H, Hkv, N, d = _gqa_dims(q, k)
    _gqa_specs("attn_fwd_window", B, H, Hkv, N, d, q=q, k=k, v=v, o=o, lse=lse)
    _check("attn_fwd_window", load().attn_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d,
                                                     float(scale), int(bool(causal)), int(window_left),
                                                     int(window_right), _stream(stream)))


def attn_bwd_window(q, k, v, o, lse, dO, dq, dk, dv, scale: float, causal: bool, window_left: int,
                    window_right: int, workspace, stream=None):
    B, H, Hkv, N, d = _gqa_dims(q, k)
    _gqa_specs("attn_bwd_window", B, H, Hkv, N, d, q=q, k=k, v=v, o=o, lse=lse, dO=dO, dq=dq, dk=dk, dv=dv)
    _check("attn_bwd_window", load().attn_bwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
                                                     _ptr(dq), _ptr(dk), _ptr(dv), B, H, Hkv, N, d, float(scale),
                                                     int(bool(causal)), int(window_left), int(window_right),
                                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                                     _stream(stream)))


def attn_fwd_block_sparse(q, k, v, o, lse, scale: float, causal: bool, row_ptr, col_idx, stream=None):
    """row_ptr, col_idx: int32 device tensors (the CSR block list)."""
    B, H, Hkv, N, d = _gqa_dims(q, k)
    _gqa_specs("attn_fwd_block_sparse", B, H, Hkv, N, d, q=q, k=k, v=v, o=o, lse=lse)
    _block_list_specs("attn_fwd_block_sparse", N, row_ptr, col_idx)
    _check("attn_fwd_block_sparse",
           load().attn_fwd_block_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d,
                                        float(scale), int(bool(causal)), _ptr(row_ptr), _ptr(col_idx),
                                        int(col_idx.numel()), _stream(stream)))


def attn_bwd_block_sparse_workspace_bytes(B: int, H: int, H_kv: int, N: int, d: int, nnz: int) -> int:
    return int(load().attn_bwd_block_sparse_workspace_bytes(B, H, H_kv, N, d, nnz))


def attn_bwd_block_sparse(q, k, v, o, lse, dO, dq, dk, dv, scale: float, causal: bool, row_ptr, col_idx,
                          workspace, stream=None):
    B, H, Hkv, N, d = _gqa_dims(q, k)
    _gqa_specs("attn_bwd_block_sparse", B, H, Hkv, N, d, q=q, k=k, v=v, o=o, lse=lse, dO=dO, dq=dq, dk=dk, dv=dv)
    _block_list_specs("attn_bwd_block_sparse", N, row_ptr, col_idx)
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
    _expect("attn_decode", ("q", q, (B, H, d), "bfloat16"), ("k_cache", k_cache, (B, Hkv, N, d), "bfloat16"),
            ("v_cache", v_cache, (B, Hkv, N, d), "bfloat16"), ("o", o, (B, H, d), "bfloat16"),
            ("lse", lse, (B, H), "float32"))
    if cache_seqlens is not None:
        _expect("attn_decode", ("cache_seqlens", cache_seqlens, (B,), "int32"))
    sl = None if cache_seqlens is None else _ptr(cache_seqlens)
    _check("attn_decode", load().attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), B, H, Hkv,
                                             N, d, float(scale), sl, _ptr(workspace),
                                             workspace.numel() * workspace.element_size(), _stream(stream)))


def attn_quantize_fp8_rows(x, x8, scales, stream=None):
    """x bf16 [B, H, N, d] -> x8 uint8 [B, H, N, d], scales fp32 [B, H, ceil(N/64)]."""
    B, H, N, d = _dense_dims(x)
    _expect("attn_quantize_fp8_rows", ("x", x, (B, H, N, d), "bfloat16"), ("x8", x8, (B, H, N, d), "uint8"),
            ("scales", scales, (B, H, (N + 63) // 64), "float32"))
    _check("attn_quantize_fp8_rows", load().attn_quantize_fp8_rows(_ptr(x), _ptr(x8), _ptr(scales), B, H, N, d,
                                                                   _stream(stream)))


def attn_quantize_fp8_vt(v, v8t, scales, stream=None):
    """v bf16 [B, H, N, d] -> v8t uint8 [B, H, ceil(N/64), d, 64], scales fp32 [B, H]."""
    B, H, N, d = _dense_dims(v)
    _expect("attn_quantize_fp8_vt", ("v", v, (B, H, N, d), "bfloat16"),
            ("v8t", v8t, (B, H, (N + 63) // 64, d, 64), "uint8"), ("scales", scales, (B, H), "float32"))
    _check("attn_quantize_fp8_vt", load().attn_quantize_fp8_vt(_ptr(v), _ptr(v8t), _ptr(scales), B, H, N, d,
                                                               _stream(stream)))


def attn_fwd_fp8(q8, q_scale, k8, k_scale, v8t, v_scale, o, lse, scale: float, causal: bool, stream=None):
    B, H, N, d = _dense_dims(q8)
    Hkv = int(k8.shape[1]) if k8 is not None and k8.dim() == 4 else -1
    nb = (N + 63) // 64
    _expect("attn_fwd_fp8", ("q8", q8, (B, H, N, d), "uint8"), ("q_scale", q_scale, (B, H, nb), "float32"),
            ("k8", k8, (B, Hkv, N, d), "uint8"), ("k_scale", k_scale, (B, Hkv, nb), "float32"),
            ("v8t", v8t, (B, Hkv, nb, d, 64), "uint8"), ("v_scale", v_scale, (B, Hkv), "float32"),
            ("o", o, (B, H, N, d), "bfloat16"), ("lse", lse, (B, H, N), "float32"))
    _check("attn_fwd_fp8", load().attn_fwd_fp8(_ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(v8t),
                                               _ptr(v_scale), _ptr(o), _ptr(lse), B, H, Hkv, N, d, float(scale),
                                               int(bool(causal)), _stream(stream)))


def attn_bwd_f32_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(load().attn_bwd_f32_workspace_bytes(B, H, N, d))


def attn_fwd_f32(q, k, v, o, lse, scale: float, causal: bool, stream=None):
    B, H, N, d = _dense_dims(q)
    _dense_specs("attn_fwd_f32", "float32", B, H, N, d, q=q, k=k, v=v, o=o, lse=lse)
    _check("attn_fwd_f32", load().attn_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                                               float(scale), int(bool(causal)), _stream(stream)))


def attn_bwd_f32(q, k, v, o, lse, dO, dq, dk, dv, scale: float, causal: bool, workspace, stream=None):
    B, H, N, d = _dense_dims(q)
    _dense_specs("attn_bwd_f32", "float32", B, H, N, d, q=q, k=k, v=v, o=o, lse=lse, dO=dO, dq=dq, dk=dk, dv=dv)
    _check("attn_bwd_f32", load().attn_bwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
                                               _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, float(scale),
                                               int(bool(causal)), _ptr(workspace),
                                               workspace.numel() * workspace.element_size(), _stream(stream)))


def _varlen_dims(q):
    if q.dim() != 3:
        raise ValueError("packed tensors are [T, H, d]")
    T, H, d = q.shape
    return int(T), int(H), int(d)


def _varlen_specs(fn, T, H, d, cu_seqlens, key_valid, **tensors):
    if cu_seqlens is None or cu_seqlens.dim() != 1:
        raise ValueError(f"{fn}: cu_seqlens is a 1-D int32 tensor [nseq + 1]")
    specs = [("cu_seqlens", cu_seqlens, (int(cu_seqlens.numel()),), "int32")]
    for name, t in tensors.items():
        specs.append((name, t, (H, T) if name == "lse" else (T, H, d), "float32" if name == "lse" else "bfloat16"))
    if key_valid is not None:
        specs.append(("key_valid", key_valid, (T,), "uint8"))
    _expect(fn, *specs)


def check_cu_seqlens(cu_seqlens_host, total_tokens: int, max_seqlen: int, fn: str = "cu_seqlens") -> None:
    """Validate a host copy of the cumulative offsets before a packed call.

    The library reads cu_seqlens from device memory and cannot check it
    without a device-to-host copy; a caller that holds the offsets on the host
    passes them here (or as `cu_seqlens_host=` to the packed wrappers): they
    must start at 0, never decrease, end at total_tokens, and no sequence may
    be longer than max_seqlen."""
    cu = [int(x) for x in (cu_seqlens_host.tolist() if hasattr(cu_seqlens_host, "tolist") else cu_seqlens_host)]
    if len(cu) < 2:
        raise ValueError(f"{fn}: cu_seqlens needs at least two entries")
    if cu[0] != 0:
        raise ValueError(f"{fn}: cu_seqlens[0] is {cu[0]}, expected 0")
    if cu[-1] != total_tokens:
        raise ValueError(f"{fn}: cu_seqlens[-1] is {cu[-1]}, expected total_tokens = {total_tokens}")
    for i in range(len(cu) - 1):
        step = cu[i + 1] - cu[i]
        if step < 0:
            raise ValueError(f"{fn}: cu_seqlens decreases at entry {i + 1}")
        if step > max_seqlen:
            raise ValueError(f"{fn}: sequence {i} has {step} tokens, more than max_seqlen = {max_seqlen}")


def attn_fwd_varlen(q, k, v, o, lse, cu_seqlens, max_seqlen: int, scale: float, causal: bool,
                    key_valid=None, stream=None, cu_seqlens_host=None):
    T, H, d = _varlen_dims(q)
    _varlen_specs("attn_fwd_varlen", T, H, d, cu_seqlens, key_valid, q=q, k=k, v=v, o=o, lse=lse)
    if cu_seqlens_host is not None:
        if len(cu_seqlens_host) != int(cu_seqlens.numel()):
            raise ValueError("attn_fwd_varlen: cu_seqlens_host and cu_seqlens differ in length")
        check_cu_seqlens(cu_seqlens_host, T, int(max_seqlen), "attn_fwd_varlen")
    nseq = int(cu_seqlens.numel()) - 1
    _check("attn_fwd_varlen", load().attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                                     _ptr(cu_seqlens), nseq, int(max_seqlen), T, H, d,
                                                     float(scale), int(bool(causal)), _ptr(key_valid),
                                                     _stream(stream)))


def attn_bwd_varlen_workspace_bytes(total_tokens: int, H: int, d: int) -> int:
    return int(load().attn_bwd_varlen_workspace_bytes(total_tokens, H, d))


def attn_bwd_varlen(q, k, v, o, lse, dO, dq, dk, dv, cu_seqlens, max_seqlen: int, scale: float, causal: bool,
                    workspace, key_valid=None, stream=None, cu_seqlens_host=None):
    T, H, d = _varlen_dims(q)
    _varlen_specs("attn_bwd_varlen", T, H, d, cu_seqlens, key_valid, q=q, k=k, v=v, o=o, lse=lse, dO=dO, dq=dq,
                  dk=dk, dv=dv)
    if cu_seqlens_host is not None:
        if len(cu_seqlens_host) != int(cu_seqlens.numel()):
            raise ValueError("attn_bwd_varlen: cu_seqlens_host and cu_seqlens differ in length")
        check_cu_seqlens(cu_seqlens_host, T, int(max_seqlen), "attn_bwd_varlen")
    nseq = int(cu_seqlens.numel()) - 1
    _check("attn_bwd_varlen", load().attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
                                                     _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cu_seqlens), nseq,
                                                     int(max_seqlen), T, H, d, float(scale), int(bool(causal)),
                                                     _ptr(key_valid), _ptr(workspace),
                                                     workspace.numel() * workspace.element_size(),
                                                     _stream(stream)))
