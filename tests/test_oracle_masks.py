"""Pins for the sliding-window and block-sparse masks of the oracle.  CPU only.

Each masked result is reduced to the unmasked oracle (already pinned by the
worked examples of the pages, autograd and finite differences) on exactly the
keys the mask leaves to a row: a sliding window leaves a contiguous slice, a
block-sparse list leaves the union of the listed key blocks.  Attention of one
query row over a set of keys is the same whether the other keys are masked to
-inf or simply absent, so

  * row i of the masked forward equals the unmasked forward of q_i over that
    row's keys;
  * the masked backward equals the sum over rows of the unmasked backward of
    one row over its keys (dQ_i from its own row; dK, dV scattered back to
    the key positions);

plus central finite differences of the masked forward, the unbounded-window
and all-blocks special cases, rows with no key at all, and planted mistakes in
the mask code that these pins must catch."""
import os
import types

import numpy as np
import pytest

from oracle import attention as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _rand(n, d, seed, nk=None):
    rng = np.random.default_rng(seed)
    nk = n if nk is None else nk
    return (rng.standard_normal((n, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, d)),
            rng.standard_normal((n, d)))


def _window_keys(i, n, left, right, causal):
    lo = 0 if left < 0 else max(0, i - left)
    hi = n if right < 0 else min(n, i + right + 1)
    if causal:
        hi = min(hi, i + 1)
    return np.arange(lo, hi)


def _block_keys(i, n, table, block, causal):
    keys = np.concatenate([np.arange(c * block, min(n, (c + 1) * block))
                           for c in np.flatnonzero(table[i // block])] or [np.zeros(0, np.int64)])
    if causal:
        keys = keys[keys <= i]
    return keys.astype(np.int64)


def _per_row_reference(q, k, v, do, scale, keys_of_row):
    """Forward and backward assembled row by row from the unmasked oracle."""
    n, d = q.shape
    o = np.zeros((n, v.shape[1]))
    lse = np.full(n, -np.inf)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for i in range(n):
        ks = keys_of_row(i)
        if len(ks) == 0:
            continue  # a row with no key: O = 0, LSE = -inf, no gradient
        gq, gk, gv, oi, li, _ = A.head_backward(q[[i]], k[ks], v[ks], do[[i]], scale, False)
        o[i], lse[i], dq[i] = oi[0], li[0], gq[0]
        dk[ks] += gk
        dv[ks] += gv
    return o, lse, dq, dk, dv


def _assert_matches(mod, q, k, v, do, scale, causal, keys_of_row, **mask):
    o, lse, dq, dk, dv = _per_row_reference(q, k, v, do, scale, keys_of_row)
    mdq, mdk, mdv, mo, mlse, _ = mod.head_backward(q, k, v, do, scale, causal, **mask)
    fo, flse = mod.head_forward(q, k, v, scale, causal, **mask)
    for got, want in ((mo, o), (fo, o), (mdq, dq), (mdk, dk), (mdv, dv)):
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    for got in (mlse, flse):
        np.testing.assert_array_equal(np.isneginf(got), np.isneginf(lse))
        fin = np.isfinite(lse)
        np.testing.assert_allclose(got[fin], lse[fin], rtol=0, atol=1e-12)


WINDOWS = [(2, 0), (0, 0), (3, 2), (0, 4), (-1, 2), (5, -1), (20, 20), (1, 1)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", WINDOWS)
def test_window_rows_reduce_to_slices(window, causal):
    q, k, v, do = _rand(13, 3, seed=window[0] * 7 + window[1] + 40)
    left, right = window
    _assert_matches(A, q, k, v, do, 0.6, causal, lambda i: _window_keys(i, 13, left, right, causal), window=window)


def test_unbounded_window_is_no_mask_and_right_zero_is_causal():
    q, k, v, do = _rand(9, 4, seed=2)
    plain = A.head_backward(q, k, v, do, 0.5, False)
    unb = A.head_backward(q, k, v, do, 0.5, False, window=(-1, -1))
    causal = A.head_backward(q, k, v, do, 0.5, True)
    right0 = A.head_backward(q, k, v, do, 0.5, False, window=(-1, 0))
    for a_, b_ in zip(plain, unb):
        np.testing.assert_array_equal(a_, b_)
    for a_, b_ in zip(causal, right0):
        np.testing.assert_array_equal(a_, b_)


def _fd(q, k, v, g, scale, causal, **mask):
    dq, dk, dv, *_ = A.head_backward(q, k, v, g, scale, causal, **mask)
    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        arrs = [q.copy(), k.copy(), v.copy()]
        x = arrs[which]
        for idx in np.ndindex(*x.shape):
            x0 = x[idx]
            x[idx] = x0 + h
            lp = float(np.sum(A.head_forward(*arrs, scale, causal, **mask)[0] * g))
            x[idx] = x0 - h
            lm = float(np.sum(A.head_forward(*arrs, scale, causal, **mask)[0] * g))
            x[idx] = x0
            assert abs((lp - lm) / (2 * h) - grad[idx]) < 1e-7


def test_window_finite_differences():
    q, k, v, g = _rand(6, 2, seed=11)
    _fd(q, k, v, g, 0.8, False, window=(1, 1))
    _fd(q, k, v, g, 0.8, True, window=(2, 0))


# ---------------------------------------------------------------- block-sparse
def _csr(rows):
    row_ptr = np.zeros(len(rows) + 1, np.int32)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    col_idx = np.array([c for r in rows for c in r], np.int32)
    return row_ptr, col_idx


def test_block_table_from_csr():
    rp, ci = _csr([[0, 2], [], [1, 1, 0]])
    t = A.block_table(rp, ci, 3, 3)
    np.testing.assert_array_equal(t, [[1, 0, 1], [0, 0, 0], [1, 1, 0]])
    with pytest.raises(ValueError):
        A.block_table(rp, np.array([0, 3, 1, 1, 0]), 3, 3)   # key block 3 does not exist
    with pytest.raises(ValueError):
        A.block_table(np.array([0, 2, 1, 5]), ci, 3, 3)       # decreasing row_ptr


BLOCK_LISTS = [
    ("tridiagonal", 3, [[0, 1], [0, 1, 2], [1, 2, 3], [2, 3, 4], [3, 4]]),
    ("global first block + local", 3, [[0], [0, 1], [0, 1, 2], [0, 2, 3], [0, 3, 4]]),
    ("strided, unsorted, duplicates", 4, [[4, 0], [1, 3, 1], [], [0, 2, 4], [3]]),
    ("single block rows", 2, [[0], [1], [2], [3], [4]]),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("name,block,rows", BLOCK_LISTS, ids=[b[0] for b in BLOCK_LISTS])
def test_block_rows_reduce_to_gathered_keys(name, block, rows, causal):
    n = 5 * block - 1  # a ragged last block
    q, k, v, do = _rand(n, 3, seed=block * 13 + len(name))
    rp, ci = _csr(rows)
    table = A.block_table(rp, ci, 5, 5)
    _assert_matches(A, q, k, v, do, 0.7, causal, lambda i: _block_keys(i, n, table, block, causal),
                    blocks=(rp, ci, block))


def test_all_blocks_listed_is_no_mask():
    q, k, v, do = _rand(10, 3, seed=5)
    rp, ci = _csr([[0, 1, 2, 3]] * 4)
    plain = A.head_backward(q, k, v, do, 0.5, True)
    sparse = A.head_backward(q, k, v, do, 0.5, True, blocks=(rp, ci, 3))
    for a_, b_ in zip(plain, sparse):
        np.testing.assert_array_equal(a_, b_)


def test_empty_rows_and_unlisted_keys():
    """A query block with an empty list has dead rows (O = 0, LSE = -inf,
    dQ = 0); a key block no row lists gets dK = dV = 0."""
    q, k, v, do = _rand(8, 3, seed=9)
    rp, ci = _csr([[0], [], [0, 3], [3]])
    dq, dk, dv, o, lse, dvec = A.head_backward(q, k, v, do, 0.5, False, blocks=(rp, ci, 2))
    assert np.all(np.isneginf(lse[2:4])) and np.all(o[2:4] == 0) and np.all(dq[2:4] == 0) and np.all(dvec[2:4] == 0)
    assert np.all(np.isfinite(lse[[0, 1, 4, 5, 6, 7]]))
    assert np.all(dk[2:6] == 0) and np.all(dv[2:6] == 0)


def test_block_finite_differences():
    q, k, v, g = _rand(7, 2, seed=12)
    rp, ci = _csr([[0, 2], [1], [1, 3], [0, 3]])
    _fd(q, k, v, g, 0.9, False, blocks=(rp, ci, 2))
    _fd(q, k, v, g, 0.9, True, blocks=(rp, ci, 2))


# ---------------------------------------------------------------- planted mistakes
def _mutant(old, new):
    path = os.path.join(ROOT, "oracle", "attention.py")
    src = open(path).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mask_mutant")
    mod.__package__ = "oracle"
    mod.__file__ = path
    exec(compile(src.replace(old, new), path, "exec"), mod.__dict__)
    return mod


def _mask_pins_pass(mod):
    try:
        for window in ((2, 0), (0, 3), (3, 1)):
            for causal in (False, True):
                q, k, v, do = _rand(11, 3, seed=sum(window) + causal)
                _assert_matches(mod, q, k, v, do, 0.6, causal,
                                lambda i: _window_keys(i, 11, window[0], window[1], causal), window=window)
        for _, block, rows in BLOCK_LISTS:
            n = 5 * block - 1
            q, k, v, do = _rand(n, 3, seed=block)
            rp, ci = _csr(rows)
            table = A.block_table(rp, ci, 5, 5)
            _assert_matches(mod, q, k, v, do, 0.7, True, lambda i: _block_keys(i, n, table, block, True),
                            blocks=(rp, ci, block))
    except AssertionError:
        return False
    return True


MASK_MUTATIONS = [
    ("vis &= keys[None, :] >= rows[:, None] - left", "vis &= keys[None, :] > rows[:, None] - left", "window left edge excluded"),
    ("vis &= keys[None, :] <= rows[:, None] + right", "vis &= keys[None, :] < rows[:, None] + right", "window right edge excluded"),
    ("vis &= keys[None, :] >= rows[:, None] - left", "vis &= keys[None, :] >= rows[:, None] - right", "window sides swapped"),
    ("vis &= table[rb][:, keys // block]", "vis &= table.T[rb][:, keys // block]", "block table transposed"),
    ("table[r, ci[rp[r]:rp[r + 1]]] = True", "table[r, ci[rp[r]:rp[r + 1] - 1]] = True", "last listed block dropped"),
]


def test_unmutated_mask_code_passes():
    assert _mask_pins_pass(A)


@pytest.mark.parametrize("old,new,label", MASK_MUTATIONS, ids=[m[2] for m in MASK_MUTATIONS])
def test_planted_mask_mistake_is_caught(old, new, label):
    assert not _mask_pins_pass(_mutant(old, new)), f"pins did not catch: {label}"
