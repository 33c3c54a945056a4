"""Block-by-block exact attention in float64 (test infrastructure only).

This module exists only to test the claim that tiling changes nothing but the
order of floating-point sums: its results are compared with the materialised
definition in ``oracle.attention`` for many tile sizes.  It follows the steps of
the pages' general forward and backward, in their order and notation:

  forward, per query block i, over key blocks j = 1..T_c   [P1 §四]
    S_i^(j) = scale Q_i K_j^T
    m_i^(j) = max(m_i^(j-1), rowmax S_i^(j))
    P~_i^(j) = exp(S_i^(j) - m_i^(j))
    l_i^(j) = exp(m_i^(j-1) - m_i^(j)) l_i^(j-1) + rowsum P~_i^(j)
    O_i^(j) = diag(exp(m_i^(j-1) - m_i^(j))) O_i^(j-1) + P~_i^(j) V_j
      (the old accumulator is MULTIPLIED by exp(m_old - m_new) <= 1, as the
       derivation in P1 §二 and the running state of P3 §01 state; the inverse
       diagonal printed in P1 §三/§四 contradicts them and is not followed)
    after the last block: O_i = O_i^(T_c) / l_i^(T_c), L_i = m_i + log l_i
  backward, per key block j (outer), query block i (inner)  [P1 §5.3-5.4]
    D = rowsum(dO o O) computed once over full rows          [P1 §5.2]
    P_i^(j) = exp(S_i^(j) - L_i); dV_j += P^T dO_i; dP = dO_i V_j^T;
    dS = P o (dP - D_i); dQ_i += scale dS K_j; dK_j += scale dS^T Q_i

Masking follows ``oracle.attention.visible_mask``.  A block in which a row has
seen no visible key yet keeps m = -inf, scale factor 1 and P~ = 0 for that row,
so -inf - (-inf) is never evaluated [P3 §04 all-masked-row convention].
"""
from __future__ import annotations

import numpy as np

from .attention import visible_mask

__all__ = ["tiled_forward", "tiled_backward", "visited_block_pairs"]


def tiled_forward(q, k, v, scale, br, bc, causal=False, key_valid=None):
    """One head, tiles of br query rows and bc keys (the last tile may be short).
    Returns (O [N, d], L [N]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, n_keys = q.shape[0], k.shape[0]
    o_out = np.zeros((n, v.shape[1]))
    l_out = np.zeros(n)
    for i0 in range(0, n, br):
        rows = np.arange(i0, min(n, i0 + br))
        m = np.full(len(rows), -np.inf)
        ell = np.zeros(len(rows))
        acc = np.zeros((len(rows), v.shape[1]))
        for j0 in range(0, n_keys, bc):
            cols = np.arange(j0, min(n_keys, j0 + bc))
            vis = visible_mask(rows, n_keys, causal, key_valid)[:, cols]
            s = np.where(vis, scale * (q[rows] @ k[cols].T), -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            alive = np.isfinite(m_new)
            m_use = np.where(alive, m_new, 0.0)
            p_tilde = np.exp(s - m_use[:, None])  # hidden keys give exp(-inf) = 0
            p_tilde[~alive] = 0.0
            # exp(m_old - m_new): 0 on the first visible block (m_old = -inf), 1 while dead
            alpha = np.where(alive, np.exp(np.where(np.isfinite(m), m, -np.inf) - m_use), 1.0)
            ell = alpha * ell + p_tilde.sum(axis=1)
            acc = alpha[:, None] * acc + p_tilde @ v[cols]
            m = m_new
        alive = np.isfinite(m)
        with np.errstate(divide="ignore", invalid="ignore"):
            o_out[rows] = np.where(alive[:, None], acc / np.where(alive, ell, 1.0)[:, None], 0.0)
            l_out[rows] = np.where(alive, m + np.log(np.where(alive, ell, 1.0)), -np.inf)
    return o_out, l_out


def tiled_backward(q, k, v, do, scale, br, bc, causal=False, key_valid=None):
    """One head; O and L come from ``tiled_forward`` with the same tiles.
    Returns (dQ, dK, dV) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n, n_keys = q.shape[0], k.shape[0]
    o, lse = tiled_forward(q, k, v, scale, br, bc, causal, key_valid)
    dvec = np.sum(do * o, axis=1)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for j0 in range(0, n_keys, bc):
        cols = np.arange(j0, min(n_keys, j0 + bc))
        dk_j = np.zeros((len(cols), k.shape[1]))
        dv_j = np.zeros((len(cols), v.shape[1]))
        for i0 in range(0, n, br):
            rows = np.arange(i0, min(n, i0 + br))
            vis = visible_mask(rows, n_keys, causal, key_valid)[:, cols]
            s = scale * (q[rows] @ k[cols].T)
            l_i = lse[rows]
            dead = ~np.isfinite(l_i)
            p = np.where(vis & ~dead[:, None], np.exp(s - np.where(dead, 0.0, l_i)[:, None]), 0.0)
            dv_j += p.T @ do[rows]
            dp = do[rows] @ v[cols].T
            ds = p * (dp - dvec[rows][:, None])
            dq[rows] += scale * (ds @ k[cols])
            dk_j += scale * (ds.T @ q[rows])
        dk[cols] = dk_j
        dv[cols] = dv_j
    return dq, dk, dv


def visited_block_pairs(n, br, bc, causal):
    """(query, key) index pairs whose score a tiled pass evaluates when it skips
    key blocks that lie wholly above the diagonal, and the number of blocks
    visited.  Used to check the pages' work ledger for the five-position example
    [P3 §05]: with causal masking each visible pair is computed once."""
    pairs = set()
    blocks = 0
    for i0 in range(0, n, br):
        i1 = min(n, i0 + br)
        for j0 in range(0, n, bc):
            if causal and j0 > i1 - 1:
                continue  # whole block above the diagonal: never loaded
            blocks += 1
            for i in range(i0, i1):
                for j in range(j0, min(n, j0 + bc)):
                    if not causal or j <= i:
                        pairs.add((i, j))
    return pairs, blocks
