"""Pins for the decoding oracle (oracle/decode.py).  CPU only.

* Decoding the token at position n-1 against a cache of its first n keys is
  row n-1 of causal self-attention over those n tokens: checked against the
  (already pinned) grouped forward oracle, for every cache length.
* An empty cache gives O = 0, LSE = -inf.
* The pages' split-KV algorithm (local max / sum / output per piece, then the
  merge) equals the definition for any number of pieces, including pieces
  past a sequence's end; planted mistakes in the merge rule break it."""
import os
import types

import numpy as np
import pytest

from oracle import attention as A
from oracle import decode as Dc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _seq(B, H, Hkv, n, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, n, d)), rng.standard_normal((B, Hkv, n, d)),
            rng.standard_normal((B, Hkv, n, d)))


@pytest.mark.parametrize("H,Hkv", [(4, 4), (6, 2), (4, 1)])
def test_decode_is_last_row_of_causal_prefill(H, Hkv):
    q, k, v = _seq(2, H, Hkv, 9, 5, seed=H + Hkv)
    o_full, l_full = A.gqa_forward(q, k, v, 0.45, causal=True)
    for n in range(1, 10):
        o, lse = Dc.decode_forward(q[:, :, n - 1], k, v, 0.45, seqlens=[n, n])
        np.testing.assert_allclose(o, o_full[:, :, n - 1], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, l_full[:, :, n - 1], rtol=0, atol=1e-13)


def test_per_sequence_lengths_and_empty_cache():
    q, k, v = _seq(3, 4, 2, 7, 3, seed=1)
    o, lse = Dc.decode_forward(q[:, :, 0], k, v, 0.5, seqlens=[7, 0, 3])
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse[1]))
    o2, l2 = Dc.decode_forward(q[2:3, :, 0], k[2:3, :, :3], v[2:3, :, :3], 0.5)
    np.testing.assert_array_equal(o[2], o2[0])
    np.testing.assert_array_equal(lse[2], l2[0])
    with pytest.raises(ValueError):
        Dc.decode_forward(q[:, :, 0], k, v, 0.5, seqlens=[8, 1, 1])


@pytest.mark.parametrize("n_splits", [1, 2, 3, 5, 16, 40])
def test_split_kv_merge_equals_definition(n_splits):
    q, k, v = _seq(2, 8, 2, 37, 4, seed=n_splits)
    q1 = q[:, :, 0] * 2.0  # sharper scores: the pieces' maxima differ a lot
    lens = [37, 11]
    o, lse = Dc.decode_forward(q1, k, v, 0.7, seqlens=lens)
    os_, ls_ = Dc.split_kv_decode(q1, k, v, 0.7, n_splits, seqlens=lens)
    np.testing.assert_allclose(os_, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(ls_, lse, rtol=0, atol=1e-13)


def _mutant(old, new):
    path = os.path.join(ROOT, "oracle", "decode.py")
    src = open(path).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_decode_mutant")
    mod.__package__ = "oracle"
    mod.__file__ = path
    exec(compile(src.replace(old, new), path, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("old,new", [
    ("np.exp(m - m_g) if m > -np.inf", "np.exp(m_g - m) if m > -np.inf"),   # inverse rescale
    ("den = float(np.dot(w, l_t))", "den = float(np.sum(l_t))"),            # sums not rescaled
    ("o[b, h] = (w @ np.array(o_t)) / den", "o[b, h] = np.sum(o_t, axis=0) / den"),
])
def test_planted_merge_mistake_is_caught(old, new):
    mod = _mutant(old, new)
    q, k, v = _seq(1, 2, 1, 30, 4, seed=4)
    o, lse = Dc.decode_forward(q[:, :, 0] * 2, k, v, 0.7)
    om, lm = mod.split_kv_decode(q[:, :, 0] * 2, k, v, 0.7, 4)
    assert not (np.allclose(om, o, atol=1e-10) and np.allclose(lm, lse, atol=1e-10))
