"""Pins for the FP8 oracle (oracle/fp8.py).  CPU only.

* The E4M3 code table against the format's closed forms and the range the
  pages give (largest 448, smallest normal 2^-6).
* Encoding against brute force over all codes (nearest value, ties to the
  even code), constructed midpoints, the sign of zero, the top of the range.
* Per-block quantization: each block's largest magnitude lands on +-448,
  power-of-two scaling of the input changes only the scale, the relative
  error of every normal code is at most 2^-4, all-zero blocks.
* The FP8 reference equals exact attention when quantization is lossless,
  and the error bound covers an explicit simulation of rounding P to E4M3,
  with and without a power-of-two pre-scale of P.
* The row-restricted reference and bound equal the whole-head ones on the
  rows they form."""
import os
import types

import numpy as np
import pytest

from oracle import attention as A
from oracle import fp8 as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
V = F.e4m3_values()


def test_code_table():
    assert V[0x7E] == 448.0 and V[0xFE] == -448.0          # largest magnitude
    assert V[0x08] == 2.0 ** -6                             # smallest normal
    assert V[0x01] == 2.0 ** -9 and V[0x07] == 7 * 2.0 ** -9
    assert V[0x38] == 1.0 and V[0x00] == 0.0 and V[0x80] == 0.0 and np.signbit(V[0x80])
    assert np.isnan(V[0x7F]) and np.isnan(V[0xFF])
    assert np.all(np.diff(V[:0x7F]) > 0)
    np.testing.assert_array_equal(V[0x80:0xFF], -V[0x00:0x7F])
    # each binade holds 8 evenly spaced values
    for e in range(1, 15):
        np.testing.assert_allclose(np.diff(V[8 * e:8 * e + 8]), 2.0 ** (e - 10))


def _brute(x):
    fin = [c for c in range(256) if not np.isnan(V[c])]
    best = min(fin, key=lambda c: (abs(V[c] - x), c & 1, 0 if np.signbit(V[c]) == np.signbit(x) else 1))
    return best


def test_encode_matches_brute_force():
    rng = np.random.default_rng(0)
    xs = np.concatenate([rng.standard_normal(400) * 20, rng.standard_normal(200) * 0.01,
                         rng.uniform(-448, 448, 200)]).astype(np.float32)
    got = F.e4m3_encode(xs)
    for x, c in zip(xs.astype(np.float64), got):
        b = _brute(x)
        assert V[c] == V[b] and (c & 1) == (b & 1) or V[c] == V[b] == 0, (x, hex(c), hex(b))


def test_midpoints_round_to_even():
    for c in range(0x01, 0x7E):
        mid = (V[c] + V[c + 1]) / 2
        if np.float32(mid) != mid:
            continue
        want = c if c % 2 == 0 else c + 1
        assert F.e4m3_encode([mid])[0] == want
        assert F.e4m3_encode([-mid])[0] == want | 0x80


def test_sign_of_zero_and_top_of_range():
    assert F.e4m3_encode([-1e-6])[0] == 0x80 and F.e4m3_encode([1e-6])[0] == 0x00
    assert list(F.e4m3_encode([448.0, 450.0, 464.0, -460.0])) == [0x7E, 0x7E, 0x7E, 0xFE]
    with pytest.raises(ValueError):
        F.e4m3_encode([465.0])


def test_block_quantization_properties():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((2, 3, 150, 16)) * 2).astype(np.float32)
    codes, s = F.quantize_rows(x)
    assert s.shape == (2, 3, 3)
    for t in range(3):
        blk = x[:, :, 64 * t:64 * (t + 1)]
        cb = codes[:, :, 64 * t:64 * (t + 1)]
        for b in range(2):
            for h in range(3):
                i = np.unravel_index(np.argmax(np.abs(blk[b, h])), blk[b, h].shape)
                assert cb[b, h][i] & 0x7F == 0x7E
    deq = F.dequantize_rows(codes, s)
    normal = np.abs(deq) >= 2.0 ** -6 * np.repeat(s, 64, axis=2)[:, :, :150, None]
    rel = np.abs(deq - x) / np.abs(x)
    assert np.all(rel[normal] <= 2.0 ** -4 + 1e-12)
    codes2, s2 = F.quantize_rows(x * np.float32(8.0))
    np.testing.assert_array_equal(codes2, codes)
    np.testing.assert_array_equal(s2, s * np.float32(8.0))
    z = np.zeros((1, 1, 70, 8), np.float32)
    cz, sz = F.quantize_rows(z)
    assert np.all(cz == 0) and np.all(sz == 1.0)
    cv, sv = F.quantize_heads(x)
    assert sv.shape == (2, 3) and np.all(sv == np.max(np.abs(x), axis=(2, 3)) / np.float32(448))


def test_lossless_quantization_gives_exact_attention():
    """Inputs whose blocks are 2^-3 times E4M3 values with a +-448 entry in
    every block quantize exactly, so the reference is plain attention."""
    rng = np.random.default_rng(3)
    fin = np.array([c for c in range(0x7F) if c != 0x7F])
    def draw(shape):
        x = V[rng.choice(fin, size=shape)] * np.where(rng.random(shape) < 0.5, -1, 1) * 0.125
        x[..., ::64, 0] = 448 * 0.125
        return x.astype(np.float32)
    q, k, v = draw((1, 2, 130, 8)), draw((1, 1, 130, 8)), draw((1, 1, 130, 8))
    ref = F.fp8_reference(q, k, v, 0.05, causal=True)
    o, lse = A.gqa_forward(q, k, v, 0.05, causal=True)
    np.testing.assert_allclose(ref["o"], o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ref["lse"], lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_row_forms_equal_the_whole_head_forms(causal):
    """fp8_reference_rows and fp8_output_bound(rows=...) give, for the listed
    query positions, exactly the rows of the whole-head reference and bound
    (the row forms serve sequences too long for the full score matrix)."""
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((1, 1, 200, 16)).astype(np.float32) for _ in range(3))
    rows = np.array([0, 1, 63, 64, 130, 199])
    full = F.fp8_reference(q, k, v, 0.3, causal)
    part = F.fp8_reference_rows(q, k, v, 0.3, causal, rows)
    # the same arithmetic, up to the rounding order of differently shaped products
    np.testing.assert_allclose(part["o"], full["o"][:, :, rows], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(part["lse"], full["lse"][:, :, rows], rtol=1e-12, atol=0)
    bf, wf = F.fp8_output_bound(full["qd"], full["kd"], full["vd"], full["lse"], 0.3, causal, p_scale_log2=6)
    bp, wp = F.fp8_output_bound(part["qd"], part["kd"], part["vd"], part["lse"], 0.3, causal, p_scale_log2=6,
                                rows=rows)
    np.testing.assert_allclose(bp, bf[:, :, rows], rtol=1e-12, atol=0)
    np.testing.assert_allclose(wp, wf[:, :, rows], rtol=1e-12, atol=0)


@pytest.mark.parametrize("p_log2", [0, 6])
def test_bound_covers_rounding_p_to_e4m3(p_log2):
    """Rounding P (times 2^p_log2) to E4M3 before P V moves O by no more than
    fp8_output_bound with the same pre-scale; the second case of each pre-scale
    has many P in the E4M3 subnormal range after the scaling."""
    rng = np.random.default_rng(4 + p_log2)
    for sig, sc in ((1.0, 0.25), (3.0, 0.9)):
        q, k, v = (rng.standard_normal((1, 2, 96, 16)).astype(np.float32) * sig for _ in range(3))
        ref = F.fp8_reference(q, k, v, sc, causal=True)
        bound, weighted = F.fp8_output_bound(ref["qd"], ref["kd"], ref["vd"], ref["lse"], sc, causal=True,
                                             p_scale_log2=p_log2)
        floor_ = 2.0 ** -10 / 2.0 ** p_log2 * np.abs(ref["vd"]).sum(axis=2)[:, :, None]
        assert np.all(bound <= 2.0 ** -4 * weighted + floor_ + 1e-300)
        tight = 0.0
        pre = 2.0 ** p_log2
        for h in range(2):
            s = sc * ref["qd"][0, h] @ ref["kd"][0, h].T
            s = np.where(np.tril(np.ones((96, 96), bool)), s, -np.inf)
            p = np.exp(s - ref["lse"][0, h][:, None])
            pq = V[F.e4m3_encode((p * pre).astype(np.float32))] / pre
            o_sim = pq @ ref["vd"][0, h]
            err = np.abs(o_sim - ref["o"][0, h])
            assert np.all(err <= bound[0, h] * (1 + 1e-9) + 1e-15)
            tight = max(tight, float(np.max(err / np.maximum(bound[0, h], 1e-300))))
        assert tight > 0.2   # the bound is not vacuous


def test_bound_without_prescale_is_wider_below_the_normal_range():
    """Without a pre-scale every P below 2^-6 is an E4M3 subnormal, so the
    bound's floor is 2^-10 per unit |V| against 2^-16 with a 2^6 pre-scale."""
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((1, 1, 64, 16)).astype(np.float32) for _ in range(3))
    ref = F.fp8_reference(q, k, v, 0.25, causal=False)
    b0, w = F.fp8_output_bound(ref["qd"], ref["kd"], ref["vd"], ref["lse"], 0.25)
    b6, _ = F.fp8_output_bound(ref["qd"], ref["kd"], ref["vd"], ref["lse"], 0.25, p_scale_log2=6)
    assert np.all(b6 <= b0 + 1e-300) and np.any(b6 < b0)
    assert np.all(b6 >= 0) and np.all(b0 <= 2.0 ** -4 * w + 2.0 ** -10 * np.abs(ref["vd"]).sum(axis=2)[:, :, None])


def _mutant(old, new):
    path = os.path.join(ROOT, "oracle", "fp8.py")
    src = open(path).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_fp8_mutant")
    mod.__package__ = "oracle"
    mod.__file__ = path
    exec(compile(src.replace(old, new), path, "exec"), mod.__dict__)
    return mod


def test_planted_rounding_mistakes_are_caught():
    ties_up = _mutant("((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))", "(d_hi == d_lo)")
    mids = [(V[c] + V[c + 1]) / 2 for c in range(0x01, 0x7E) if c % 2 == 0]
    assert not np.array_equal(ties_up.e4m3_encode(mids), F.e4m3_encode(mids))
    wrong_max = _mutant("s = (amax / np.float32(E4M3_MAX)).astype(np.float32)",
                        "s = (amax / np.float32(240.0)).astype(np.float32)")
    x = np.random.default_rng(5).standard_normal((1, 1, 64, 8)).astype(np.float32)
    c, _ = wrong_max.quantize_rows(x)
    assert not np.any((c & 0x7F) == 0x7E)   # the block max no longer reaches 448
