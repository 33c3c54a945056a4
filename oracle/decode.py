"""Decoding attention (one new query token per sequence) in float64.

Test infrastructure only (see the package docstring).

``decode_forward`` is the definition: the new token of sequence b, query head
h, attends the first ``len_b`` cached keys of its key/value head
h // (H / H_kv) with no further mask (every cached position precedes the new
token) -- one row of exact attention [P4 §18.8.2: in the decoding phase the
query of each token is a single row vector, Q: [b, 1, d], against a long KV
cache].  A sequence with an empty cache has no key: O = 0, LSE = -inf (the
all-masked-row convention of P3 §04).

``split_kv_decode`` follows the three steps of FlashDecoding as P4 §18.8.2
gives them: cut the cache into T equal-length pieces; for each piece compute
the local maximum m_t, exponent sum l_t and unnormalised output O_t; then
combine them with the online-softmax merge
    m = max_t m_t,   O = sum_t O_t e^(m_t - m) / sum_t l_t e^(m_t - m).
It exists to pin that merge rule (the GPU path implements it) against the
definition; the parity tests compare the GPU with ``decode_forward``.
"""
from __future__ import annotations

import numpy as np

from .attention import head_forward

__all__ = ["decode_forward", "split_kv_decode"]


def _lengths(B, n_kv, seqlens):
    if seqlens is None:
        return np.full(B, n_kv, dtype=np.int64)
    lens = np.asarray(seqlens, dtype=np.int64)
    if lens.shape != (B,) or np.any(lens < 0) or np.any(lens > n_kv):
        raise ValueError("seqlens must hold B lengths in [0, N_kv]")
    return lens


def decode_forward(q, k_cache, v_cache, scale, seqlens=None):
    """q [B, H, d]; k_cache, v_cache [B, H_kv, N_kv, d] with H_kv dividing H;
    seqlens: optional [B] cache lengths (default N_kv).  Returns O [B, H, d]
    and LSE [B, H] (natural log), fp64."""
    q = np.asarray(q, dtype=np.float64)
    B, H, d = q.shape
    Hkv, n_kv = k_cache.shape[1], k_cache.shape[2]
    if Hkv <= 0 or H % Hkv:
        raise ValueError("the key/value head count must divide the query head count")
    G = H // Hkv
    lens = _lengths(B, n_kv, seqlens)
    o = np.zeros((B, H, v_cache.shape[-1]))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        for h in range(H):
            ob, lb = head_forward(q[b, h][None, :], k_cache[b, h // G, :n], v_cache[b, h // G, :n], scale)
            o[b, h], lse[b, h] = ob[0], lb[0]
    return o, lse


def split_kv_decode(q, k_cache, v_cache, scale, n_splits, seqlens=None):
    """FlashDecoding in the order of P4 §18.8.2 (KV split, local attention per
    piece, merge).  Pieces are ceil(N_kv / n_splits) keys long; a piece past a
    sequence's length is empty (m_t = -inf, l_t = 0) and drops out of the
    merge.  Returns O [B, H, d] and LSE [B, H]."""
    q = np.asarray(q, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    B, H, d = q.shape
    Hkv, n_kv = k_cache.shape[1], k_cache.shape[2]
    G = H // Hkv
    lens = _lengths(B, n_kv, seqlens)
    piece = -(-n_kv // n_splits)
    o = np.zeros((B, H, v_cache.shape[-1]))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        for h in range(H):
            kk, vv = k_cache[b, h // G], v_cache[b, h // G]
            m_t, l_t, o_t = [], [], []
            # step 1 + 2: each piece's local max, exponent sum and output
            for t in range(n_splits):
                lo, hi = t * piece, min(int(lens[b]), (t + 1) * piece)
                if hi <= lo:
                    m_t.append(-np.inf)
                    l_t.append(0.0)
                    o_t.append(np.zeros(vv.shape[1]))
                    continue
                s = scale * (kk[lo:hi] @ q[b, h])
                m = s.max()
                e = np.exp(s - m)
                m_t.append(m)
                l_t.append(e.sum())
                o_t.append(e @ vv[lo:hi])
            # step 3: merge with the global maximum
            m_g = max(m_t)
            if m_g == -np.inf:
                continue
            w = np.array([np.exp(m - m_g) if m > -np.inf else 0.0 for m in m_t])
            den = float(np.dot(w, l_t))
            o[b, h] = (w @ np.array(o_t)) / den
            lse[b, h] = m_g + np.log(den)
    return o, lse
