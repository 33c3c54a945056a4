"""Pins for the grouped key/value head oracle (gqa_forward, gqa_backward).  CPU only.

Each compares the oracle with something fixed independently of it: torch's
autograd of a textbook softmax attention whose K and V are broadcast to the
query heads with repeat_interleave (so the group sums of dK and dV come from
autograd's chain rule through the broadcast), brute-force central differences
of L = sum(O o G) with respect to the shared K and V, and the ungrouped case,
which must be the already-pinned multi-head oracle."""
import numpy as np
import pytest

from oracle import attention as A

torch = pytest.importorskip("torch")


def _inputs(B, H, Hkv, N, d, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    g = rng.standard_normal((B, H, N, d))
    return q, k, v, g


def _torch_grouped(q, k, v, g, scale, causal):
    """Textbook attention in torch float64 with K/V repeated per query head."""
    H, Hkv = q.shape[1], k.shape[1]
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    ke = torch.repeat_interleave(tk, H // Hkv, dim=1)
    ve = torch.repeat_interleave(tv, H // Hkv, dim=1)
    s = scale * tq @ ke.transpose(-1, -2)
    n = q.shape[2]
    if causal:
        s = s.masked_fill(~torch.ones(n, n, dtype=torch.bool).tril(), float("-inf"))
    p = torch.softmax(s, dim=-1)
    o = p @ ve
    lse = torch.logsumexp(s, dim=-1)
    (o * torch.tensor(g)).sum().backward()
    return o.detach().numpy(), lse.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv", [(4, 2), (6, 3), (4, 1), (8, 2)])
def test_grouped_heads_against_torch_autograd(H, Hkv, causal):
    q, k, v, g = _inputs(2, H, Hkv, 11, 5, seed=H * 10 + Hkv)
    scale = 0.4
    ref = A.gqa_backward(q, k, v, g, scale, causal)
    o, lse, dq, dk, dv = _torch_grouped(q, k, v, g, scale, causal)
    np.testing.assert_allclose(ref["o"], o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ref["lse"], lse, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ref["dq"], dq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ref["dk"], dk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ref["dv"], dv, rtol=0, atol=1e-12)
    fo, flse = A.gqa_forward(q, k, v, scale, causal)
    np.testing.assert_array_equal(fo, ref["o"])
    np.testing.assert_array_equal(flse, ref["lse"])


def test_grouped_heads_finite_differences():
    """dK, dV of the shared heads (and dQ) against central differences of
    L = sum(O o G), every entry, on a tiny grouped problem."""
    q, k, v, g = _inputs(1, 4, 2, 5, 3, seed=7)
    scale = 0.7
    ref = A.gqa_backward(q, k, v, g, scale, True)

    def loss(q_, k_, v_):
        o, _ = A.gqa_forward(q_, k_, v_, scale, True)
        return float(np.sum(o * g))

    h = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            x0 = x[idx]
            x[idx] = x0 + h
            lp = loss(q, k, v)
            x[idx] = x0 - h
            lm = loss(q, k, v)
            x[idx] = x0
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(ref[name], num, rtol=0, atol=1e-8)


def test_one_head_per_group_is_multi_head():
    q, k, v, g = _inputs(2, 3, 3, 9, 4, seed=3)
    grouped = A.gqa_backward(q, k, v, g, 0.5, True)
    plain = A.backward(q, k, v, g, 0.5, True)
    for name in ("o", "lse", "dq", "dk", "dv", "D"):
        np.testing.assert_array_equal(grouped[name], plain[name])


def test_group_must_divide_heads():
    q, k, v, g = _inputs(1, 4, 3, 4, 2, seed=1)
    with pytest.raises(ValueError):
        A.gqa_forward(q, k, v, 1.0)


def test_group_selection_matches_full():
    q, k, v, g = _inputs(2, 6, 2, 7, 3, seed=9)
    full = A.gqa_backward(q, k, v, g, 0.3, True)
    part = A.gqa_backward(q, k, v, g, 0.3, True, groups=[(1, 0)])
    for name in ("o", "lse", "dq", "D"):
        np.testing.assert_array_equal(part[name][1, 0:3], full[name][1, 0:3])
        assert np.isnan(part[name][0]).all() and np.isnan(part[name][1, 3:]).all()
    for name in ("dk", "dv"):
        np.testing.assert_array_equal(part[name][1, 0], full[name][1, 0])
        assert np.isnan(part[name][1, 1]).all()
