"""Materialised exact attention in float64 -- the oracle's definition.

Test infrastructure only (see the package docstring).  Nothing here is blocked,
fused or reordered beyond computing whole query rows a few at a time: every
query row is produced from the full score row, exactly as written on the pages.

Definition followed (per batch b, head h; or per packed sequence s, head h):
  S = scale * Q K^T                      [P2 §1.1; P4 §18.2.1]
  masked entries of S are -inf           [P4 §18.2.2 item 3 (causal, j <= i kept),
                                          item 4 (padding masks act on keys)]
  P = row-softmax(S), O = P V            [P2 §1.1, §3.2 safe softmax]
  LSE_i = log sum_j exp(S_ij)            [P1 §三 end ("保存 logsumexp"); P3 §04]
  D_i  = rowsum(dO o O)                  [P1 §5.2]
  dP = dO V^T, dS = P o (dP - D)         [P1 §5.1-5.2; P4 §18.2.4]
  dV = P^T dO, dQ = scale dS K,
  dK = scale dS^T Q                      [P3 §04 (the 1/sqrt(d) factor);
                                          P4 §18.2.4 materialised backward]
A query row with no visible key is defined as O = 0, LSE = -inf and contributes
no gradient [P3 §04, the all-masked-row convention].

Readings where the pages are loose:
  * ``scale`` multiplies Q K^T and is an argument (1/sqrt(d) in every workload);
    LSE is that of the scaled scores and dQ, dK carry one factor of ``scale``.
  * LSE uses the natural logarithm.
  * Causal masking keeps key j for query i iff j <= i, counted within a sequence.
  * Sliding window (left, right), -1 meaning unbounded on that side: key j is
    visible to query i iff i - left <= j <= i + right, in addition to any
    causal or padding mask.
  * Block-sparse layout: positions are cut into blocks of ``block`` tokens;
    query block r lists, in CSR form (row_ptr, col_idx), the key blocks it
    attends; a listed index counts once however often it is listed.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "visible_mask",
    "head_forward",
    "head_backward",
    "head_backward_sampled",
    "head_backward_sampled_sparse",
    "forward",
    "backward",
    "varlen_forward",
    "varlen_backward",
    "gqa_forward",
    "gqa_backward",
    "block_table",
    "preprocess_d",
]


def block_table(row_ptr, col_idx, n_qblocks: int, n_kblocks: int) -> np.ndarray:
    """Boolean [n_qblocks, n_kblocks] from a CSR block list: entry (r, c) is True
    iff c appears among col_idx[row_ptr[r] : row_ptr[r+1]] [P4 §18.8.1: the
    preprocessing step stores, for every query block, the key blocks it must
    compute].  Raises on a malformed list."""
    rp = np.asarray(row_ptr, dtype=np.int64)
    ci = np.asarray(col_idx, dtype=np.int64)
    if rp.shape != (n_qblocks + 1,) or rp[0] != 0 or np.any(np.diff(rp) < 0) or rp[-1] != len(ci):
        raise ValueError("row_ptr must be non-decreasing, start at 0 and end at len(col_idx)")
    if len(ci) and (ci.min() < 0 or ci.max() >= n_kblocks):
        raise ValueError("col_idx entries must index key blocks")
    table = np.zeros((n_qblocks, n_kblocks), dtype=bool)
    for r in range(n_qblocks):
        table[r, ci[rp[r]:rp[r + 1]]] = True
    return table


def visible_mask(rows: np.ndarray, n_keys: int, causal: bool, key_valid=None, window=None,
                 blocks=None, keys=None) -> np.ndarray:
    """Boolean [len(rows), n_keys]: True where query ``rows[r]`` may attend key j
    (``keys``: only those key positions, giving [len(rows), len(keys)]).

    Causal: key j is visible to query i iff j <= i [P4 §18.2.2 item 3, M_ij = 0 for
    j <= i].  Key padding: invalid keys are hidden from every query [P4 §18.2.2
    item 4].  ``window`` = (left, right): key j is visible to query i only if
    i - left <= j <= i + right, a negative side being unbounded [P4 §18.7.1, the
    window_size argument; §18.8.1 sliding window].  ``blocks`` = (row_ptr,
    col_idx, block): key j is visible to query i only if key block j // block is
    listed for query block i // block [P4 §18.8.1, block-sparse FlashAttention:
    blocks that are not listed contribute nothing]."""
    rows = np.asarray(rows)
    keys = np.arange(n_keys) if keys is None else np.asarray(keys)
    vis = np.ones((len(rows), len(keys)), dtype=bool)
    if causal:
        vis &= keys[None, :] <= rows[:, None]
    if key_valid is not None:
        vis &= np.asarray(key_valid, dtype=bool)[keys][None, :]
    if window is not None:
        left, right = window
        if left >= 0:
            vis &= keys[None, :] >= rows[:, None] - left
        if right >= 0:
            vis &= keys[None, :] <= rows[:, None] + right
    if blocks is not None:
        row_ptr, col_idx, block = blocks
        n_q = len(row_ptr) - 1
        table = block_table(row_ptr, col_idx, n_q, -(-n_keys // block))
        rb = rows // block
        if len(rows) and rb.max() >= n_q:
            raise ValueError("a query row lies past the last query block of the list")
        vis &= table[rb][:, keys // block]
    return vis


def _scores(q_rows, k, scale, vis):
    """S = scale * Q K^T with hidden entries set to -inf."""
    s = scale * (q_rows @ k.T)
    return np.where(vis, s, -np.inf)


def _row_softmax_and_lse(s):
    """Safe softmax of each row [P2 §3.2]: subtract the row max before exp.

    Returns P (rows with no visible key are all zero) and LSE (-inf for such
    rows, per the all-masked-row convention of P3 §04)."""
    m = s.max(axis=1)
    dead = ~np.isfinite(m)  # every entry -inf
    m_safe = np.where(dead, 0.0, m)
    e = np.exp(s - m_safe[:, None])  # exp(-inf) = 0 for hidden keys
    e[dead] = 0.0
    denom = e.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(dead[:, None], 0.0, e / np.where(dead, 1.0, denom)[:, None])
        lse = np.where(dead, -np.inf, m_safe + np.log(np.where(dead, 1.0, denom)))
    return p, lse


def head_forward(q, k, v, scale, causal=False, key_valid=None, rows=None, row_chunk=2048, window=None, blocks=None):
    """O and LSE for one head.  q, k, v: [N, d] (any float dtype, used as fp64).

    ``rows`` selects query rows (default: all), which lets a test check sampled
    rows of a large problem; each row is still computed from its full score row.
    ``window`` / ``blocks``: optional sliding-window and block-sparse masks
    (see ``visible_mask``).  Returns (O [len(rows), d] fp64, LSE [len(rows)] fp64)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_keys = k.shape[0]
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    o = np.zeros((len(rows), v.shape[1]))
    lse = np.zeros(len(rows))
    for c0 in range(0, len(rows), row_chunk):
        r = rows[c0:c0 + row_chunk]
        s = _scores(q[r], k, scale, visible_mask(r, n_keys, causal, key_valid, window, blocks))
        p, l_ = _row_softmax_and_lse(s)
        o[c0:c0 + len(r)] = p @ v
        lse[c0:c0 + len(r)] = l_
    return o, lse


def head_backward(q, k, v, do, scale, causal=False, key_valid=None, row_chunk=2048,
                  check_d_identity=True, window=None, blocks=None):
    """dQ, dK, dV for one head, plus O, LSE and D (all fp64).

    P is rebuilt from the definition (not from any saved state), then the
    materialised backward of P4 §18.2.4 / P1 §五 is applied row block by row
    block: dV and dK are sums over query rows, dQ rows are independent.
    D is rowsum(dO o O) [P1 §5.2]; when ``check_d_identity`` it is asserted equal
    to rowsum(P o dP), the form it was derived from."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n, n_keys = q.shape[0], k.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    o = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    dvec = np.zeros(n)
    for c0 in range(0, n, row_chunk):
        r = np.arange(c0, min(n, c0 + row_chunk))
        s = _scores(q[r], k, scale, visible_mask(r, n_keys, causal, key_valid, window, blocks))
        p, l_ = _row_softmax_and_lse(s)
        o_r = p @ v
        dp = do[r] @ v.T                      # dP = dO V^T
        d_r = np.sum(do[r] * o_r, axis=1)     # D = rowsum(dO o O)
        if check_d_identity:
            alt = np.sum(p * dp, axis=1)      # D = rowsum(P o dP)
            tol = 1e-9 * (np.sum(np.abs(do[r]) * np.abs(o_r), axis=1) + np.sum(p * np.abs(dp), axis=1)) + 1e-300
            if not np.all(np.abs(alt - d_r) <= tol):
                raise AssertionError("D identity rowsum(dO o O) == rowsum(P o dP) violated")
        ds = p * (dp - d_r[:, None])          # dS = P o (dP - D)
        dv += p.T @ do[r]                     # dV = P^T dO
        dq[r] = scale * (ds @ k)              # dQ = scale dS K
        dk += scale * (ds.T @ q[r])           # dK = scale dS^T Q
        o[r] = o_r
        lse[r] = l_
        dvec[r] = d_r
    return dq, dk, dv, o, lse, dvec


def head_backward_sampled(q, k, v, do, scale, causal=False, key_valid=None, query_rows=(), key_cols=(),
                          row_chunk=2048, window=None, blocks=None):
    """The backward of one head evaluated only at chosen outputs: dQ at
    ``query_rows`` and dK, dV at ``key_cols`` (plus O, LSE and D for all rows).

    Same definition as ``head_backward``: dQ_i = scale sum_j dS_ij K_j needs
    row i of P and dP; dV_j = sum_i P_ij dO_i and dK_j = scale sum_i dS_ij Q_i
    need column j of P and dS, i.e. LSE and D of every row.  Lets a test check
    a problem too large to materialise whole on the CPU."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n, n_keys = q.shape[0], k.shape[0]
    o, lse = head_forward(q, k, v, scale, causal, key_valid, row_chunk=row_chunk, window=window, blocks=blocks)
    dvec = np.sum(do * o, axis=1)
    rows = np.asarray(query_rows, dtype=np.int64)
    cols = np.asarray(key_cols, dtype=np.int64)
    dq = np.zeros((len(rows), q.shape[1]))
    if len(rows):
        s = _scores(q[rows], k, scale, visible_mask(rows, n_keys, causal, key_valid, window, blocks))
        dead = ~np.isfinite(lse[rows])
        p = np.where(dead[:, None], 0.0, np.exp(s - np.where(dead, 0.0, lse[rows])[:, None]))
        dp = do[rows] @ v.T
        ds = p * (dp - dvec[rows][:, None])
        dq = scale * (ds @ k)
    dk = np.zeros((len(cols), k.shape[1]))
    dv = np.zeros((len(cols), v.shape[1]))
    if len(cols):
        for c0 in range(0, n, row_chunk):
            r = np.arange(c0, min(n, c0 + row_chunk))
            vis = visible_mask(r, n_keys, causal, key_valid, window, blocks)[:, cols]
            s = np.where(vis, scale * (q[r] @ k[cols].T), -np.inf)
            dead = ~np.isfinite(lse[r])
            p = np.where(dead[:, None], 0.0, np.exp(s - np.where(dead, 0.0, lse[r])[:, None]))
            dp = do[r] @ v[cols].T
            ds = p * (dp - dvec[r][:, None])
            dv += p.T @ do[r]
            dk += scale * (ds.T @ q[r])
    return dq, dk, dv, o, lse, dvec


def head_backward_sampled_sparse(q, k, v, do, scale, causal=False, key_valid=None, query_rows=(), key_cols=(),
                                 row_chunk=4096, window=None, blocks=None):
    """head_backward_sampled for a sequence too long for a forward over every
    row: dQ, O and LSE at ``query_rows`` and dK, dV at ``key_cols``.  O, LSE
    and D are formed only for the rows that matter: the query rows
    themselves and every row that sees one of the key columns.  A row that
    sees none of them adds exact zeros to their dK and dV.  The definition is
    that of ``head_backward``, so the results equal head_backward_sampled's
    up to the order of rounding.  Cheap when the mask (a window, a block
    list) leaves each sampled column to few rows.
    Returns (dQ, dK, dV, O at query_rows, LSE at query_rows), fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n, n_keys = q.shape[0], k.shape[0]
    rows = np.asarray(query_rows, dtype=np.int64)
    cols = np.asarray(key_cols, dtype=np.int64)
    seen = [np.zeros(0, np.int64)]
    if len(cols):
        for c0 in range(0, n, row_chunk):
            r = np.arange(c0, min(n, c0 + row_chunk))
            vis = visible_mask(r, n_keys, causal, key_valid, window, blocks, keys=cols)
            seen.append(r[vis.any(axis=1)])
    need = np.union1d(np.concatenate(seen), rows).astype(np.int64)
    o, lse = head_forward(q, k, v, scale, causal, key_valid, rows=need, row_chunk=row_chunk, window=window,
                          blocks=blocks)
    dvec = np.sum(do[need] * o, axis=1)
    at = np.searchsorted(need, rows)
    dq = np.zeros((len(rows), q.shape[1]))
    if len(rows):
        s = _scores(q[rows], k, scale, visible_mask(rows, n_keys, causal, key_valid, window, blocks))
        dead = ~np.isfinite(lse[at])
        p = np.where(dead[:, None], 0.0, np.exp(s - np.where(dead, 0.0, lse[at])[:, None]))
        dp = do[rows] @ v.T
        ds = p * (dp - dvec[at][:, None])
        dq = scale * (ds @ k)
    dk = np.zeros((len(cols), k.shape[1]))
    dv = np.zeros((len(cols), v.shape[1]))
    if len(cols):
        for c0 in range(0, len(need), row_chunk):
            sel = np.arange(c0, min(len(need), c0 + row_chunk))
            r = need[sel]
            vis = visible_mask(r, n_keys, causal, key_valid, window, blocks, keys=cols)
            s = np.where(vis, scale * (q[r] @ k[cols].T), -np.inf)
            dead = ~np.isfinite(lse[sel])
            p = np.where(dead[:, None], 0.0, np.exp(s - np.where(dead, 0.0, lse[sel])[:, None]))
            dp = do[r] @ v[cols].T
            ds = p * (dp - dvec[sel][:, None])
            dv += p.T @ do[r]
            dk += scale * (ds.T @ q[r])
    return dq, dk, dv, o[at], lse[at]


def preprocess_d(o, do):
    """D_i = rowsum(dO o O) over the last axis, in fp64 [P1 §5.2]: the backward's
    pre-pass on its own, for any leading shape ([B, H, N, d] -> [B, H, N]).
    ``o`` is whatever output the pre-pass is given (the GPU's bf16 O when it
    checks the GPU pre-pass)."""
    return np.sum(np.asarray(do, dtype=np.float64) * np.asarray(o, dtype=np.float64), axis=-1)


def forward(q, k, v, scale, causal=False, heads=None):
    """Dense layout [B, H, N, d].  Returns O [B, H, N, d] and LSE [B, H, N] (fp64).

    ``heads`` optionally restricts the work to a list of (b, h) pairs; the other
    entries of the outputs are left as NaN."""
    B, H, N, d = q.shape
    o = np.full((B, H, N, v.shape[-1]), np.nan)
    lse = np.full((B, H, N), np.nan)
    for b, h in (heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]):
        o[b, h], lse[b, h] = head_forward(q[b, h], k[b, h], v[b, h], scale, causal)
    return o, lse


def backward(q, k, v, do, scale, causal=False, heads=None):
    """Dense layout [B, H, N, d].  Returns dict with dq, dk, dv, o, lse, D (fp64)."""
    B, H, N, d = q.shape
    out = {name: np.full(q.shape, np.nan) for name in ("dq", "dk", "dv", "o")}
    out["lse"] = np.full((B, H, N), np.nan)
    out["D"] = np.full((B, H, N), np.nan)
    for b, h in (heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]):
        dq, dk, dv, o, lse, dvec = head_backward(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal)
        out["dq"][b, h], out["dk"][b, h], out["dv"][b, h] = dq, dk, dv
        out["o"][b, h], out["lse"][b, h], out["D"][b, h] = o, lse, dvec
    return out


def _seq_heads(cu_seqlens, H, seqs, heads):
    seqs = range(len(cu_seqlens) - 1) if seqs is None else seqs
    heads = range(H) if heads is None else heads
    return [(s, h) for s in seqs for h in heads]


def varlen_forward(q, k, v, cu_seqlens, scale, causal=False, key_valid=None, seqs=None, heads=None):
    """Packed layout [T, H, d] with offsets cu_seqlens[nseq+1].  No query attends
    across a sequence boundary; causal order is the position within the sequence
    [P4 §18.7.1, variable-length interface].  Returns O [T, H, d], LSE [H, T]."""
    T, H, d = q.shape
    o = np.full((T, H, v.shape[-1]), np.nan)
    lse = np.full((H, T), np.nan)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for s, h in _seq_heads(cu, H, seqs, heads):
        a, b = int(cu[s]), int(cu[s + 1])
        if b <= a:
            continue
        kv = None if key_valid is None else np.asarray(key_valid)[a:b]
        o[a:b, h], lse[h, a:b] = head_forward(q[a:b, h], k[a:b, h], v[a:b, h], scale, causal, kv)
    return o, lse


def varlen_backward(q, k, v, do, cu_seqlens, scale, causal=False, key_valid=None, seqs=None, heads=None):
    """Packed layout backward.  Returns dict with dq, dk, dv, o [T, H, d] and lse, D [H, T]."""
    T, H, d = q.shape
    out = {name: np.full(q.shape, np.nan) for name in ("dq", "dk", "dv", "o")}
    out["lse"] = np.full((H, T), np.nan)
    out["D"] = np.full((H, T), np.nan)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for s, h in _seq_heads(cu, H, seqs, heads):
        a, b = int(cu[s]), int(cu[s + 1])
        if b <= a:
            continue
        kv = None if key_valid is None else np.asarray(key_valid)[a:b]
        dq, dk, dv, o, lse, dvec = head_backward(q[a:b, h], k[a:b, h], v[a:b, h], do[a:b, h], scale, causal, kv)
        out["dq"][a:b, h], out["dk"][a:b, h], out["dv"][a:b, h], out["o"][a:b, h] = dq, dk, dv, o
        out["lse"][h, a:b], out["D"][h, a:b] = lse, dvec
    return out


def _group(H, Hkv):
    if Hkv <= 0 or H % Hkv:
        raise ValueError("the key/value head count must divide the query head count")
    return H // Hkv


def gqa_forward(q, k, v, scale, causal=False, heads=None, window=None, blocks=None):
    """Grouped key/value heads, dense layout: q [B, H, N, d], k and v
    [B, H_kv, N, d] with H_kv dividing H.  Query head h attends with key/value
    head h // (H / H_kv) [P4 §18.2.2: in GQA the query heads form groups that
    share one K/V head; §18.7.1: K and V with fewer heads are broadcast along
    the head dimension].  ``window`` / ``blocks`` as in ``visible_mask``, the
    same for every head.  Returns O [B, H, N, d] and LSE [B, H, N]."""
    B, H, N, d = q.shape
    G = _group(H, k.shape[1])
    o = np.full((B, H, N, v.shape[-1]), np.nan)
    lse = np.full((B, H, N), np.nan)
    for b, h in (heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]):
        o[b, h], lse[b, h] = head_forward(q[b, h], k[b, h // G], v[b, h // G], scale, causal,
                                          window=window, blocks=blocks)
    return o, lse


def gqa_backward(q, k, v, do, scale, causal=False, groups=None, window=None, blocks=None):
    """Backward of ``gqa_forward``.  dQ, O, LSE, D per query head as in the
    ungrouped case; dK and dV of key/value head j are the sums, over the query
    heads h with h // (H / H_kv) == j, of the gradients that head's attention
    gives to the shared K and V (the chain rule through the broadcast).
    ``groups``: optional list of (b, j) key/value heads to compute (with all
    their query heads); entries outside it stay NaN."""
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    G = _group(H, Hkv)
    out = {name: np.full(q.shape, np.nan) for name in ("dq", "o")}
    out["dk"] = np.full(k.shape, np.nan)
    out["dv"] = np.full(v.shape, np.nan)
    out["lse"] = np.full((B, H, N), np.nan)
    out["D"] = np.full((B, H, N), np.nan)
    todo = groups if groups is not None else [(b, j) for b in range(B) for j in range(Hkv)]
    for b, j in todo:
        out["dk"][b, j] = 0.0
        out["dv"][b, j] = 0.0
        for h in range(j * G, (j + 1) * G):
            dq, dk, dv, o, lse, dvec = head_backward(q[b, h], k[b, j], v[b, j], do[b, h], scale, causal,
                                                     window=window, blocks=blocks)
            out["dq"][b, h], out["o"][b, h], out["lse"][b, h], out["D"][b, h] = dq, o, lse, dvec
            out["dk"][b, j] += dk
            out["dv"][b, j] += dv
    return out
