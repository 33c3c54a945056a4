"""FP8 (E4M3) quantization and the reference for FP8 attention, in float64.

Test infrastructure only (see the package docstring).

[P4 §18.6.2] FlashAttention-3's FP8 forward: Q, K and V are converted to FP8
E4M3 (1 sign, 4 exponent, 3 mantissa bits; largest magnitude 448, smallest
normal 2^-6) with dynamic per-block scales computed for each load block of Q
and of K, s = max|X_block| / 448, X_fp8 = E4M3(X / s); S = Q K^T accumulates
in fp32, the softmax runs in fp32, and O is dequantized to bf16.

Readings where the pages leave the format open:
  * E4M3 is the OCP "E4M3FN" encoding: exponent bias 7, no infinities, the
    all-ones exponent and mantissa pattern is NaN, subnormals below 2^-6.
  * Conversion rounds to nearest, ties to even, keeping the sign of zero;
    magnitudes in (448, 464] round to 448 (464 is the midpoint to the next
    binade, which E4M3FN does not have).
  * Blocks are 64 consecutive rows of one (batch, head) for Q and K; the
    pages name per-block scales for Q and K only, so V gets one scale per
    (batch, head).  s and X / s are fp32 divisions (correctly rounded); an
    all-zero block gets s = 1.
  * The reference output is exact attention (this package's definition) on
    the dequantized tensors s * E4M3value.  The pages also round P to FP8 for
    the P V product but leave open how P is scaled first; what that rounding
    adds is bounded in ``fp8_output_bound`` for a caller-given power-of-two
    pre-scale of P (none by default), including P small enough to be an
    E4M3 subnormal after the scaling.
"""
from __future__ import annotations

import numpy as np

from .attention import gqa_forward, head_forward, visible_mask

__all__ = [
    "E4M3_MAX",
    "e4m3_values",
    "e4m3_encode",
    "quantize_rows",
    "quantize_heads",
    "dequantize_rows",
    "dequantize_heads",
    "fp8_reference",
    "fp8_reference_rows",
    "fp8_output_bound",
]

E4M3_MAX = 448.0
BLOCK = 64


def e4m3_values() -> np.ndarray:
    """Value of each of the 256 codes (NaN for the two NaN codes)."""
    v = np.empty(256)
    for c in range(256):
        sign, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            v[c] = np.nan
            continue
        mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
        v[c] = -mag if sign else mag
    return v


_VALUES = e4m3_values()
_POS_CODES = np.array([c for c in range(0x7F)], dtype=np.int64)   # 0x00 .. 0x7E, increasing values
_POS_VALUES = _VALUES[_POS_CODES]


def e4m3_encode(x) -> np.ndarray:
    """Round-to-nearest-even E4M3 codes (uint8) of fp32 values."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    if np.any(np.isnan(x)) or np.any(np.abs(x) > 464.0):
        raise ValueError("value outside the E4M3 range")
    mag = np.abs(x)
    hi = np.searchsorted(_POS_VALUES, mag, side="left")      # first value >= mag
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - mag
    exact = d_hi == 0
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(exact | pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(mag > E4M3_MAX, 0x7E, code)   # (448, 464]: nearest is 448
    sign = np.signbit(x).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def _scale(amax):
    """s = amax / 448 in fp32 (s = 1 for an all-zero block)."""
    amax = np.asarray(amax, dtype=np.float32)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def quantize_rows(x, block: int = BLOCK):
    """Q or K [B, H, N, d] -> codes [B, H, N, d] (uint8) and scales
    [B, H, ceil(N / block)] (fp32), one scale per block of rows."""
    x = np.asarray(x, dtype=np.float32)
    B, H, N, d = x.shape
    nb = -(-N // block)
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty((B, H, nb), dtype=np.float32)
    for t in range(nb):
        xs = x[:, :, t * block:(t + 1) * block]
        s = _scale(np.max(np.abs(xs), axis=(2, 3)))
        scales[:, :, t] = s
        codes[:, :, t * block:(t + 1) * block] = e4m3_encode((xs / s[:, :, None, None]).astype(np.float32))
    return codes, scales


def quantize_heads(x):
    """V [B, H, N, d] -> codes [B, H, N, d] and one scale per (batch, head) [B, H]."""
    x = np.asarray(x, dtype=np.float32)
    s = _scale(np.max(np.abs(x), axis=(2, 3)))
    return e4m3_encode((x / s[:, :, None, None]).astype(np.float32)), s


def dequantize_rows(codes, scales, block: int = BLOCK):
    vals = _VALUES[np.asarray(codes, dtype=np.int64)]
    rep = np.repeat(np.asarray(scales, dtype=np.float64), block, axis=2)[:, :, :codes.shape[2]]
    return vals * rep[..., None]


def dequantize_heads(codes, scales):
    return _VALUES[np.asarray(codes, dtype=np.int64)] * np.asarray(scales, dtype=np.float64)[:, :, None, None]


def fp8_reference(q, k, v, scale, causal=False):
    """Quantize bf16-exact inputs as the FP8 path does, then exact attention on
    the dequantized tensors.  q [B, H, N, d], k and v [B, H_kv, N, d].
    Returns dict with o, lse (fp64), the codes and scales, and the
    dequantized tensors."""
    q8, sq = quantize_rows(q)
    k8, sk = quantize_rows(k)
    v8, sv = quantize_heads(v)
    qd, kd, vd = dequantize_rows(q8, sq), dequantize_rows(k8, sk), dequantize_heads(v8, sv)
    o, lse = gqa_forward(qd, kd, vd, scale, causal)
    return {"o": o, "lse": lse, "q8": q8, "sq": sq, "k8": k8, "sk": sk, "v8": v8, "sv": sv,
            "qd": qd, "kd": kd, "vd": vd}


def fp8_reference_rows(q, k, v, scale, causal, rows):
    """fp8_reference for the query positions ``rows`` only, of one head per
    K/V head: q [1, 1, N, d], k and v [1, 1, N, d].  The whole tensors are
    quantized (the scales depend on every row of a block); exact attention
    is then formed for the listed rows alone, so N may be far larger than
    the full score matrix allows.  Returns dict with o [1, 1, R, d] and lse
    [1, 1, R] (fp64) and the dequantized tensors."""
    q8, sq = quantize_rows(q)
    k8, sk = quantize_rows(k)
    v8, sv = quantize_heads(v)
    qd, kd, vd = dequantize_rows(q8, sq), dequantize_rows(k8, sk), dequantize_heads(v8, sv)
    o, lse = head_forward(qd[0, 0], kd[0, 0], vd[0, 0], scale, causal, rows=np.asarray(rows))
    return {"o": o[None, None], "lse": lse[None, None], "qd": qd, "kd": kd, "vd": vd}


def fp8_output_bound(qd, kd, vd, lse, scale, causal=False, p_scale_log2=0, rows=None):
    """Per-element bound on |O_fp8 - O_ref| from rounding P to E4M3 for the
    P V product, P being multiplied by 2^p_scale_log2 before rounding (and
    divided by it afterwards; p_scale_log2 = 0: no pre-scale).  A P_ij whose
    scaled value is a normal E4M3 number is off by at most 2^-4 of itself
    (half an ulp of a 3-bit mantissa); below that (subnormal) it is off by at
    most half the subnormal step, 2^-10 / 2^p_scale_log2, and never by more
    than itself.  The error of O_i is at most
    sum_j min(P_ij, max(2^-4 P_ij, 2^-10 / 2^p_scale_log2)) |V_j|.
    Returns (bound, weighted) [B, H, N, d] fp64, weighted = sum_j P_ij |V_j|.
    With ``rows`` (query positions) only those rows are formed: lse is then
    [B, H, len(rows)] and both results [B, H, len(rows), d] (for sequences
    too long for the whole N x N score matrix)."""
    B, H, N, d = qd.shape
    G = H // kd.shape[1]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    floor_ = 2.0 ** -10 / 2.0 ** p_scale_log2
    bound = np.zeros((B, H, len(rows), d))
    weighted = np.zeros((B, H, len(rows), d))
    for b in range(B):
        for h in range(H):
            s = scale * (qd[b, h][rows] @ kd[b, h // G].T)
            s = np.where(visible_mask(rows, N, causal), s, -np.inf)
            p = np.exp(s - lse[b, h][:, None])
            dp = np.minimum(p, np.maximum(2.0 ** -4 * p, floor_))
            bound[b, h] = dp @ np.abs(vd[b, h // G])
            weighted[b, h] = p @ np.abs(vd[b, h // G])
    return bound, weighted
