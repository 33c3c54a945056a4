"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module only draws random numbers and rounds them to the storage type; it
holds none of the attention arithmetic.  Both sides receive exactly the same
values: fp32 arrays whose entries are exactly representable in the storage
dtype ("bf16" or "f32"), plus the raw bf16 bit patterns for the device copy.

Recipe (one generator per call, numpy PCG64 ``default_rng(seed)``):
  * varlen only: sequence lengths first, uniform integers in [lo, hi];
  * then Q, K, V, dO in that order, each float64 standard normal times its
    sigma, cast to float32, then rounded to bf16 with round-to-nearest-even
    (bf16 storage only).
Dense layout is [B, H, N, d]; packed varlen layout is [T_total, H, d].
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "round_to_bf16",
    "bf16_bits",
    "bits_to_f32",
    "dense_inputs",
    "varlen_inputs",
    "decode_inputs",
    "left_padding_key_mask",
]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even; NaN kept quiet."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded (RNE) to the nearest bf16, returned as float32."""
    return bits_to_f32(bf16_bits(x))


def _draw(rng: np.random.Generator, shape, sigma: float, dtype: str) -> np.ndarray:
    x = (rng.standard_normal(shape) * sigma).astype(np.float32)
    if dtype == "bf16":
        x = round_to_bf16(x)
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return x


def dense_inputs(B: int, H: int, N: int, d: int, dtype: str = "bf16", seed: int = 0,
                 sigma_qk: float = 1.0, sigma_vdo: float = 1.0, with_do: bool = True,
                 kv_heads: int | None = None) -> dict:
    """Q, K, V (and dO) of shape [B, H, N, d] as float32 holding dtype-exact values.
    With ``kv_heads`` K and V have that many heads instead: [B, kv_heads, N, d]."""
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    kv_shape = (B, H if kv_heads is None else kv_heads, N, d)
    out = {
        "q": _draw(rng, shape, sigma_qk, dtype),
        "k": _draw(rng, kv_shape, sigma_qk, dtype),
        "v": _draw(rng, kv_shape, sigma_vdo, dtype),
    }
    if with_do:
        out["do"] = _draw(rng, shape, sigma_vdo, dtype)
    return out


def decode_inputs(B: int, H: int, Hkv: int, N: int, d: int, dtype: str = "bf16", seed: int = 0,
                  sigma: float = 1.0) -> dict:
    """One query token per sequence, q [B, H, d], and a KV cache k, v
    [B, Hkv, N, d], drawn in that order."""
    rng = np.random.default_rng(seed)
    return {
        "q": _draw(rng, (B, H, d), sigma, dtype),
        "k": _draw(rng, (B, Hkv, N, d), sigma, dtype),
        "v": _draw(rng, (B, Hkv, N, d), sigma, dtype),
    }


def varlen_inputs(nseq: int, len_lo: int, len_hi: int, H: int, d: int, dtype: str = "bf16",
                  seed: int = 0, sigma_qk: float = 1.0, sigma_vdo: float = 1.0,
                  with_do: bool = True, lengths=None) -> dict:
    """Packed sequences [T_total, H, d] with int32 cumulative offsets cu_seqlens[nseq+1]."""
    rng = np.random.default_rng(seed)
    if lengths is None:
        lengths = rng.integers(len_lo, len_hi, size=nseq, endpoint=True)
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    shape = (T, H, d)
    out = {
        "cu_seqlens": cu,
        "lengths": lengths.astype(np.int32),
        "max_seqlen": int(lengths.max()) if len(lengths) else 0,
        "q": _draw(rng, shape, sigma_qk, dtype),
        "k": _draw(rng, shape, sigma_qk, dtype),
        "v": _draw(rng, shape, sigma_vdo, dtype),
    }
    if with_do:
        out["do"] = _draw(rng, shape, sigma_vdo, dtype)
    return out


def left_padding_key_mask(cu_seqlens: np.ndarray, frac: float = 0.01) -> np.ndarray:
    """Per packed token, 1 = valid key.  The first max(1, round(frac*L)) tokens of
    every sequence are marked invalid (left padding), so under a causal mask the
    query rows at those positions see no valid key at all."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    valid = np.ones(int(cu[-1]), dtype=np.uint8)
    for s in range(len(cu) - 1):
        L = int(cu[s + 1] - cu[s])
        if L <= 0:
            continue
        p = min(L, max(1, int(round(frac * L))))
        valid[cu[s]:cu[s] + p] = 0
    return valid
