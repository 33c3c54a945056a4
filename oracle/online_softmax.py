"""Single-row running softmax state (test infrastructure only).

One query row, its scores s_1..s_N and value vectors v_1..v_N, processed a block
of keys at a time with the running state of P3 §01 (m: largest score so far,
l: sum of exp(s - m) so far, a: sum of exp(s - m) v so far):

    m' = max(m, max_{j in B} s_j),  alpha = exp(m - m')
    l' = alpha l + sum_{j in B} exp(s_j - m')
    a' = alpha a + sum_{j in B} exp(s_j - m') v_j,   o' = a' / l'

starting from m = -inf, l = 0, a = 0, with the old-state factor taken as 0 on
the first block.  With blocks of one score this is the streaming recurrence
m_i = max(m_{i-1}, x_i), l_i = l_{i-1} exp(m_{i-1} - m_i) + exp(x_i - m_i) of
P2 §3.3.  ``block_ledger`` records, per block, the columns of the block table
on P3 §02: block scores, block max, running max, old-state scale and running
denominator.
"""
from __future__ import annotations

import math

__all__ = ["block_ledger", "online_row"]


def block_ledger(scores, bc):
    """Run the state over ``scores`` in blocks of ``bc``.

    Returns (ledger, m, l, lse) with one ledger dict per block."""
    m = -math.inf
    ell = 0.0
    ledger = []
    for start in range(0, len(scores), bc):
        blk = [float(x) for x in scores[start:start + bc]]
        blk_max = max(blk)
        m_new = max(m, blk_max)
        old_scale = 0.0 if m == -math.inf else math.exp(m - m_new)
        ell = old_scale * ell + sum(math.exp(x - m_new) for x in blk)
        ledger.append({
            "block": len(ledger) + 1,
            "scores": blk,
            "block_max": blk_max,
            "running_max": m_new,
            "old_scale": old_scale,
            "denominator": ell,
        })
        m = m_new
    return ledger, m, ell, m + math.log(ell)


def online_row(scores, values, bc):
    """Output o = a / l of one row after all blocks, with the state (m, l, a).

    ``values`` is a list of equal-length vectors, one per score."""
    m = -math.inf
    ell = 0.0
    a = [0.0] * len(values[0])
    for start in range(0, len(scores), bc):
        blk = [float(x) for x in scores[start:start + bc]]
        m_new = max(m, max(blk))
        alpha = 0.0 if m == -math.inf else math.exp(m - m_new)
        w = [math.exp(x - m_new) for x in blk]
        ell = alpha * ell + sum(w)
        for t in range(len(a)):
            a[t] = alpha * a[t] + sum(wj * values[start + j][t] for j, wj in enumerate(w))
        m = m_new
    return [x / ell for x in a], m, ell
