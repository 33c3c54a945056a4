"""The sampled form of the bf16 bar (tests/parity_utils.py), CPU only: with
every row sampled it equals the exact relative Frobenius error; with a
sample, the weighted squared norms are unbiased estimates of the whole
tensor's; the first and last rows are always in the sample."""
import numpy as np

from parity_utils import check_bf16_sampled, rel_fro, sample_positions


def test_full_sample_is_exact():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((40, 8))
    got = ref + 1e-3 * rng.standard_normal((40, 8))
    pos, w = sample_positions(40, 100, rng)
    assert np.array_equal(pos, np.arange(40)) and np.all(w == 1.0)
    est, _ = check_bf16_sampled(got[pos], ref[pos], w, "x")
    assert abs(est - rel_fro(got, ref)) < 1e-12


def test_fixed_rows_and_unbiased_weights():
    rng = np.random.default_rng(1)
    n = 1000
    ref = rng.standard_normal((n, 4)) * np.linspace(0.1, 3, n)[:, None]
    e2 = np.sum(ref ** 2, axis=1)
    acc = []
    for _ in range(400):
        pos, w = sample_positions(n, 32, rng)
        assert {0, 1, n - 2, n - 1} <= set(pos.tolist()) and len(set(pos.tolist())) == 32
        assert abs(np.sum(w) - n) < 1e-9
        acc.append(np.sum(w * e2[pos]))
    assert abs(np.mean(acc) / np.sum(e2) - 1) < 0.03
