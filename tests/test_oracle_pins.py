"""Pins for the fp64 oracle: page examples, closed forms, invariants, finite
differences and a library cross-check.  CPU only.

None of these re-types the oracle's formula: each compares it with something
fixed independently (a closed form written from the scores, brute-force finite
differences, torch's autograd of a textbook softmax attention, or an invariant
the mathematics guarantees)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import online_softmax as OS
from oracle import tiled as T

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- six scores
SIX = _load("six_scores.json")["scores"]


def _closed_six():
    """Closed forms of the six-score row, written from the scores only."""
    m = 3.0
    ell = math.fsum(math.exp(s - m) for s in SIX)
    lse = m + math.log(ell)
    probs = [math.exp(s - lse) for s in SIX]
    return m, ell, lse, probs


def test_six_scores_closed_form_values():
    m, ell, lse, probs = _closed_six()
    # e^-2 + e^-1 + e^-4 + 1 + e^-3 + e^-0.5
    assert ell == pytest.approx(math.exp(-2) + math.exp(-1) + math.exp(-4) + 1 + math.exp(-3) + math.exp(-0.5), rel=1e-15)
    assert lse == pytest.approx(3.778337275235960, abs=1e-13)
    assert sum(probs) == pytest.approx(1.0, abs=1e-15)


def test_six_scores_ledger_blocks_of_two():
    """P3 §02 ledger columns for blocks [1,2], [-1,3], [0,2.5]."""
    ledger, m, ell, lse = OS.block_ledger(SIX, 2)
    assert [r["scores"] for r in ledger] == [[1, 2], [-1, 3], [0, 2.5]]
    assert [r["block_max"] for r in ledger] == [2, 3, 2.5]
    assert [r["running_max"] for r in ledger] == [2, 3, 3]
    # first block: old state scaled by 0; then e^(2-3); then e^(3-3) = 1
    assert ledger[0]["old_scale"] == 0.0
    assert ledger[1]["old_scale"] == pytest.approx(math.exp(-1), rel=1e-15)
    assert ledger[2]["old_scale"] == 1.0
    l1 = math.exp(1 - 2) + math.exp(0)
    l2 = math.exp(-1) * l1 + math.exp(-1 - 3) + math.exp(0)
    l3 = l2 + math.exp(0 - 3) + math.exp(2.5 - 3)
    assert [r["denominator"] for r in ledger] == pytest.approx([l1, l2, l3], rel=1e-15)
    assert l1 == pytest.approx(1.367879441171, abs=1e-12)
    assert l2 == pytest.approx(1.521530363297, abs=1e-12)
    assert l3 == pytest.approx(2.177848091377287, abs=1e-12)


@pytest.mark.parametrize("bc", [1, 2, 3, 4, 5, 6])
def test_six_scores_every_block_size_gives_full_row(bc):
    """Online state after all blocks equals the full-row softmax for any
    partition [P1 §二 proof; P4 §18.4.2]."""
    m0, ell0, lse0, probs0 = _closed_six()
    _, m, ell, lse = OS.block_ledger(SIX, bc)
    assert m == m0
    assert ell == pytest.approx(ell0, rel=1e-14)
    assert lse == pytest.approx(lse0, rel=1e-15)
    rng = np.random.default_rng(7)
    values = rng.standard_normal((6, 2)).tolist()
    o, _, _ = OS.online_row(SIX, values, bc)
    ref = [math.fsum(p * v[t] for p, v in zip(probs0, values)) for t in range(2)]
    assert o == pytest.approx(ref, rel=1e-13, abs=1e-15)


def test_six_scores_through_materialised_oracle():
    """The six scores as one query row (d = 1, q = 1, k_j = s_j, scale = 1)."""
    m0, ell0, lse0, probs0 = _closed_six()
    q = np.ones((1, 1))
    k = np.array(SIX, dtype=np.float64)[:, None]
    v = np.eye(6)  # O then equals the probability row itself
    o, lse = A.head_forward(q, k, v, 1.0)
    assert lse[0] == pytest.approx(lse0, rel=1e-15)
    assert o[0] == pytest.approx(probs0, rel=1e-14)
    assert o[0] == pytest.approx([0.062141746145, 0.168918779335, 0.008409970815,
                                  0.459168848350, 0.022860670845, 0.278499984510], abs=1e-12)


# ------------------------------------------------------------- five positions
FIVE = _load("five_position.json")


def _five():
    q = np.array(FIVE["Q"], dtype=np.float64)
    k = np.array(FIVE["K"], dtype=np.float64)
    v = np.array(FIVE["V"], dtype=np.float64)
    g = np.array(FIVE["G"], dtype=np.float64)
    return q, k, v, g, 1.0 / math.sqrt(2.0)


def test_five_position_row0_closed_form():
    """Row 0 sees only key 0: P_00 = 1, LSE_0 = S_00, O_0 = V_0, D_0 = G_0.V_0,
    dS_00 = P_00 (G_0.V_0 - D_0) = 0, hence dQ_0 = 0."""
    q, k, v, g, scale = _five()
    dq, dk, dv, o, lse, dvec = A.head_backward(q, k, v, g, scale, causal=True)
    s00 = (0.2 * 0.3 + (-0.3) * 0.5) / math.sqrt(2.0)
    assert s00 == pytest.approx(-0.063639610306789, abs=1e-15)
    assert lse[0] == pytest.approx(s00, abs=1e-15)
    assert o[0] == pytest.approx([1.0, 0.0], abs=1e-15)
    assert dvec[0] == pytest.approx(0.2, abs=1e-15)
    assert dq[0] == pytest.approx([0.0, 0.0], abs=1e-15)


def _loss(q, k, v, g, scale, causal, key_valid=None):
    o, _ = A.head_forward(q, k, v, scale, causal, key_valid)
    return float(np.sum(o * g))


def _fd_grads(q, k, v, g, scale, causal, key_valid=None, h=1e-6):
    grads = []
    for which in range(3):
        arrs = [q.copy(), k.copy(), v.copy()]
        x = arrs[which]
        gr = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            x0 = x[idx]
            x[idx] = x0 + h
            lp = _loss(*arrs, g, scale, causal, key_valid)
            x[idx] = x0 - h
            lm = _loss(*arrs, g, scale, causal, key_valid)
            x[idx] = x0
            gr[idx] = (lp - lm) / (2 * h)
        grads.append(gr)
    return grads


def test_five_position_finite_differences():
    """dQ, dK, dV of L = sum(O o G) against central differences, every entry."""
    q, k, v, g, scale = _five()
    dq, dk, dv, *_ = A.head_backward(q, k, v, g, scale, causal=True)
    fq, fk, fv = _fd_grads(q, k, v, g, scale, True)
    np.testing.assert_allclose(dq, fq, atol=1e-8)
    np.testing.assert_allclose(dk, fk, atol=1e-8)
    np.testing.assert_allclose(dv, fv, atol=1e-8)


def test_five_position_causal_work_ledger():
    """P3 §05: 15 causal QK dot products for 5 positions, with 2x2 tiles; the
    tiles wholly above the diagonal are never visited (3 of the 9)."""
    pairs, blocks = T.visited_block_pairs(5, 2, 2, causal=True)
    assert len(pairs) == FIVE["causal_qk_dot_products_forward"] == 15
    assert blocks == 6
    assert all(j <= i for i, j in pairs)


@pytest.mark.parametrize("n,b", [(5, 2), (8, 2), (9, 3), (64, 16), (100, 32)])
def test_causal_square_tile_count(n, b):
    t = -(-n // b)
    pairs, blocks = T.visited_block_pairs(n, b, b, causal=True)
    assert blocks == t * (t + 1) // 2
    assert len(pairs) == n * (n + 1) // 2


# ------------------------------------------------------ library cross-check
torch = pytest.importorskip("torch")


def _torch_reference(q, k, v, g, scale, causal, key_valid=None):
    """Textbook softmax attention in torch float64 on the CPU, differentiated by
    autograd [P3 method note: checked against a full reference and autograd]."""
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = scale * (tq @ tk.T)
    vis = torch.ones_like(s, dtype=torch.bool)
    n = s.shape[0]
    if causal:
        vis &= torch.ones(n, n, dtype=torch.bool).tril()
    if key_valid is not None:
        vis &= torch.tensor(key_valid, dtype=torch.bool)[None, :]
    s = s.masked_fill(~vis, float("-inf"))
    dead = ~vis.any(dim=1)
    s_safe = s.masked_fill(dead[:, None], 0.0)
    p = torch.softmax(s_safe, dim=1).masked_fill(dead[:, None], 0.0)
    o = p @ tv
    lse = torch.logsumexp(s, dim=1)
    (o * torch.tensor(g)).sum().backward()
    return o.detach().numpy(), lse.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
@pytest.mark.parametrize("n,d", [(1, 4), (7, 3), (33, 16), (70, 8)])
def test_against_torch_autograd(causal, padded, n, d):
    rng = np.random.default_rng(n * 100 + d)
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    scale = 1.0 / math.sqrt(d)
    kv = None
    if padded:
        kv = (rng.random(n) > 0.3).astype(np.uint8)
        kv[0] = 0  # with causal masking row 0 is then fully masked
    ro, rl, rdq, rdk, rdv = _torch_reference(q, k, v, g, scale, causal, kv)
    dq, dk, dv, o, lse, _ = A.head_backward(q, k, v, g, scale, causal, kv)
    np.testing.assert_allclose(o, ro, atol=1e-13)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(rl))
    fin = np.isfinite(rl)
    np.testing.assert_allclose(lse[fin], rl[fin], atol=1e-13)
    np.testing.assert_allclose(dq, rdq, atol=1e-12)
    np.testing.assert_allclose(dk, rdk, atol=1e-12)
    np.testing.assert_allclose(dv, rdv, atol=1e-12)


# ----------------------------------------------------------------- invariants
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
@pytest.mark.parametrize("br,bc", [(1, 1), (2, 2), (3, 5), (5, 3), (8, 8), (16, 16), (32, 32), (37, 37), (8, 32), (32, 8)])
def test_tiling_changes_nothing(causal, padded, br, bc):
    """Tiled fp64 forward/backward equal the materialised definition for every
    tile size, including sizes that do not divide N [P1 §二 2.4; P4 §18.4.2]."""
    n, d = 37, 5
    rng = np.random.default_rng(br * 1000 + bc)
    q, k, v, g = (rng.standard_normal((n, d)) * 1.5 for _ in range(4))
    kv = None
    if padded:
        kv = np.ones(n, np.uint8)
        kv[:3] = 0
        kv[20] = 0
    scale = 1.0 / math.sqrt(d)
    o_t, l_t = T.tiled_forward(q, k, v, scale, br, bc, causal, kv)
    dq_t, dk_t, dv_t = T.tiled_backward(q, k, v, g, scale, br, bc, causal, kv)
    dq, dk, dv, o, lse, _ = A.head_backward(q, k, v, g, scale, causal, kv)
    np.testing.assert_allclose(o_t, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(np.isneginf(l_t), np.isneginf(lse))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(l_t[fin], lse[fin], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dq_t, dq, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk_t, dk, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv_t, dv, rtol=1e-11, atol=1e-12)


def test_single_key_gives_value_row():
    q = np.array([[0.7, -1.2, 0.3]])
    k = np.array([[1.5, 0.2, -0.4]])
    v = np.array([[3.0, -2.0, 0.5]])
    o, lse = A.head_forward(q, k, v, 0.5)
    np.testing.assert_array_equal(o, v)
    assert lse[0] == pytest.approx(0.5 * float(q[0] @ k[0]), abs=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_is_uniform_average(causal):
    """scale = 0: every visible key weighs the same, O_i = mean of visible V
    rows and LSE_i = ln(number of visible keys)."""
    rng = np.random.default_rng(3)
    n, d = 11, 4
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    o, lse = A.head_forward(q, k, v, 0.0, causal)
    for i in range(n):
        cnt = i + 1 if causal else n
        np.testing.assert_allclose(o[i], v[:cnt].mean(axis=0), atol=1e-14)
        assert lse[i] == pytest.approx(math.log(cnt), abs=1e-14)


def test_constant_values_give_constant_output():
    rng = np.random.default_rng(4)
    n, d = 13, 6
    q, k = (rng.standard_normal((n, d)) * 3 for _ in range(2))
    v = np.full((n, d), -1.75)
    o, _ = A.head_forward(q, k, v, 0.4, causal=True)
    np.testing.assert_allclose(o, v, atol=1e-14)


def test_key_permutation_invariance():
    rng = np.random.default_rng(5)
    n, d = 17, 5
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    perm = rng.permutation(n)
    o1, l1 = A.head_forward(q, k, v, 0.3)
    o2, l2 = A.head_forward(q, k[perm], v[perm], 0.3)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    """K -> K + 1 c^T adds scale q_i.c to row i of S: O is unchanged and LSE_i
    moves by exactly scale q_i.c."""
    rng = np.random.default_rng(6)
    n, d = 15, 4
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    c = rng.standard_normal(d)
    scale = 0.6
    o1, l1 = A.head_forward(q, k, v, scale, causal)
    o2, l2 = A.head_forward(q, k + c[None, :], v, scale, causal)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l2 - l1, scale * (q @ c), atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_sum_identities(causal):
    """Each dS row sums to zero, so sum_j dK_j = 0; without a causal mask every
    P row sums to one over all keys, so sum_j dV_j = sum_i dO_i."""
    rng = np.random.default_rng(8)
    n, d = 19, 6
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    dq, dk, dv, *_ = A.head_backward(q, k, v, g, 0.45, causal)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    if not causal:
        np.testing.assert_allclose(dv.sum(axis=0), g.sum(axis=0), atol=1e-12)


def test_fully_masked_rows_convention():
    """A query row with no visible key: O = 0, LSE = -inf, no gradient flows
    from it, and the other rows are as if it had been left out."""
    rng = np.random.default_rng(9)
    n, d = 9, 3
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    kv = np.ones(n, np.uint8)
    kv[:3] = 0  # causal: rows 0, 1, 2 see only padded keys
    dq, dk, dv, o, lse, dvec = A.head_backward(q, k, v, g, 0.5, True, kv)
    assert np.all(np.isneginf(lse[:3])) and np.all(np.isfinite(lse[3:]))
    np.testing.assert_array_equal(o[:3], 0.0)
    np.testing.assert_array_equal(dq[:3], 0.0)
    np.testing.assert_array_equal(dvec[:3], 0.0)
    np.testing.assert_array_equal(dk[:3], 0.0)  # invalid keys get no gradient
    np.testing.assert_array_equal(dv[:3], 0.0)
    # rows 3.. are unchanged if the dead rows' upstream gradient is altered
    g2 = g.copy()
    g2[:3] = 123.0
    dq2, dk2, dv2, *_ = A.head_backward(q, k, v, g2, 0.5, True, kv)
    np.testing.assert_array_equal(dq2, dq)
    np.testing.assert_array_equal(dk2, dk)
    np.testing.assert_array_equal(dv2, dv)


def test_random_finite_differences_with_padding():
    rng = np.random.default_rng(10)
    n, d = 6, 3
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    kv = np.array([0, 1, 1, 0, 1, 1], np.uint8)
    dq, dk, dv, *_ = A.head_backward(q, k, v, g, 0.7, True, kv)
    fq, fk, fv = _fd_grads(q, k, v, g, 0.7, True, kv)
    np.testing.assert_allclose(dq, fq, atol=1e-8)
    np.testing.assert_allclose(dk, fk, atol=1e-8)
    np.testing.assert_allclose(dv, fv, atol=1e-8)


def test_varlen_sequences_do_not_interact():
    """Packed sequences are independent heads: each equals the dense oracle on
    its own slice, and changing one sequence leaves the others unchanged."""
    rng = np.random.default_rng(11)
    lengths = [5, 1, 9, 4]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T_, H, d = int(cu[-1]), 2, 3
    q, k, v, g = (rng.standard_normal((T_, H, d)) for _ in range(4))
    out = A.varlen_backward(q, k, v, g, cu, 0.5, causal=True)
    for s in range(len(lengths)):
        a, b = cu[s], cu[s + 1]
        for h in range(H):
            dq, dk, dv, o, lse, _ = A.head_backward(q[a:b, h], k[a:b, h], v[a:b, h], g[a:b, h], 0.5, True)
            np.testing.assert_array_equal(out["o"][a:b, h], o)
            np.testing.assert_array_equal(out["dk"][a:b, h], dk)
    k2 = k.copy()
    k2[cu[2]:cu[3]] += 5.0
    out2 = A.varlen_backward(q, k2, v, g, cu, 0.5, causal=True)
    np.testing.assert_array_equal(out2["o"][:cu[2]], out["o"][:cu[2]])
    np.testing.assert_array_equal(out2["dq"][cu[3]:], out["dq"][cu[3]:])


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_backward_matches_full_backward(causal):
    """The sampled form picks the same entries out of the full backward."""
    rng = np.random.default_rng(12)
    n, d = 45, 6
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    kv = np.ones(n, np.uint8)
    kv[[0, 7, 30]] = 0
    rows = [0, 3, 7, 44]
    cols = [0, 1, 30, 44]
    dq, dk, dv, o, lse, dvec = A.head_backward(q, k, v, g, 0.4, causal, kv, row_chunk=8)
    sq, sk, sv_, so, sl, sd = A.head_backward_sampled(q, k, v, g, 0.4, causal, kv, rows, cols, row_chunk=16)
    np.testing.assert_allclose(sq, dq[rows], atol=1e-13)
    np.testing.assert_allclose(sk, dk[cols], atol=1e-13)
    np.testing.assert_allclose(sv_, dv[cols], atol=1e-13)
    np.testing.assert_allclose(so, o, atol=1e-14)


@pytest.mark.parametrize("mask", ["causal", "padded", "window", "blocks"])
def test_row_sparse_sampled_backward_matches_full_backward(mask):
    """The row-sparse sampled form (O, LSE, D only for the rows that need
    them) picks the same entries out of the full backward under every mask,
    with a row chunk smaller than the problem so that rows are skipped."""
    rng = np.random.default_rng(21)
    n, d = 300, 6
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    kw = {"causal": mask in ("causal", "blocks")}
    if mask == "padded":
        kv = np.ones(n, np.uint8)
        kv[[0, 7, 130, 299]] = 0
        kw["key_valid"] = kv
    if mask == "window":
        kw["window"] = (20, 3)
    if mask == "blocks":
        rows_ = [[0, r] if r != 2 else [0, 1, 2] for r in range(3)]
        kw["blocks"] = (np.array([0, 2, 4, 7]), np.array([c for r in rows_ for c in r]), 128)
    rows = [0, 3, 127, 128, 200, 299]
    cols = [1, 150, 160, 260, 299]
    dq, dk, dv, o, lse, _ = A.head_backward(q, k, v, g, 0.4, row_chunk=64, **kw)
    sq, sk, sv_, so, sl = A.head_backward_sampled_sparse(q, k, v, g, 0.4, query_rows=rows, key_cols=cols,
                                                         row_chunk=50, **kw)
    np.testing.assert_allclose(sq, dq[rows], atol=1e-12)
    np.testing.assert_allclose(sk, dk[cols], atol=1e-12)
    np.testing.assert_allclose(sv_, dv[cols], atol=1e-12)
    np.testing.assert_allclose(so, o[rows], atol=1e-13)
    np.testing.assert_array_equal(np.isneginf(sl), np.isneginf(lse[rows]))
    fin = np.isfinite(lse[rows])
    np.testing.assert_allclose(sl[fin], lse[rows][fin], atol=1e-13)


def test_preprocess_d_pins():
    """The pre-pass alone: D = rowsum(dO o O) [P1 §5.2].  Pinned to the other
    form of the same quantity, rowsum(P o dP), which head_backward checks
    against its own D, and to one-hot rows of O, where D picks one entry of
    dO (a sum over the wrong axis or a dropped factor fails either)."""
    rng = np.random.default_rng(13)
    n, d = 23, 5
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    *_, o, _, dvec = A.head_backward(q, k, v, g, 0.5, True)
    np.testing.assert_allclose(A.preprocess_d(o, g), dvec, atol=1e-13)
    s = 0.5 * q @ k.T
    s[np.triu_indices(n, 1)] = -np.inf
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(A.preprocess_d(o, g), np.sum(p * (g @ v.T), axis=1), atol=1e-12)
    one_hot = np.zeros((2, 3, n, d))
    idx = rng.integers(0, d, size=(2, 3, n))
    np.put_along_axis(one_hot, idx[..., None], 1.0, axis=-1)
    dO = rng.standard_normal((2, 3, n, d))
    dd = A.preprocess_d(one_hot, dO)
    assert dd.shape == (2, 3, n)
    np.testing.assert_array_equal(dd, np.take_along_axis(dO, idx[..., None], axis=-1)[..., 0])
