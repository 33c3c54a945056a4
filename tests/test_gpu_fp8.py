"""GPU parity of the FP8 (E4M3) path: attn_quantize_fp8_rows,
attn_quantize_fp8_vt and attn_fwd_fp8.

The quantizers are integer-valued work and must match the oracle bit for bit
(codes and fp32 scales): ragged N, huge and tiny magnitudes, all-zero blocks.
attn_quantize_fp8_vt writes its codes in the transposed tile order that
include/miattn.h declares (tile t, feature f, position p holds key
64 t + k(p)); the test inverts that declared order on the device's codes and
compares them with oracle.fp8.quantize_heads, so the oracle knows nothing of
the kernel's layout.

The forward is checked element by element against exact attention on the
dequantized inputs (oracle.fp8.fp8_reference, which quantizes the same bf16
inputs itself), within
    |O - O_ref| <= bound + (2^-8 + delta_i) * weighted + 2^-8 |O_ref|,
bound the effect of rounding P to E4M3 (oracle.fp8.fp8_output_bound with the
pre-scale of P by 2^6 that include/miattn.h declares for attn_fwd_fp8;
derived and pinned in the oracle's tests: 2^-4 of each P in the normal range,
half a subnormal step below it) and weighted = sum_j P_ij |V_j|.  The scores
come from FP8 MFMAs, whose accumulation of the 128 products of a score is not
exact: test_fp8_score_accumulation_error measures it through single-key rows
(where LSE equals the score) and requires it to stay within 2^-13 of the sum
of the products' magnitudes.  With twice that, a score of row i is off by at
most delta_i = 2^-12 |scale| max_j sum_f |q_if| |k_jf|, which moves each P_ij
by a factor e^(+-delta_i) and O_i by at most delta_i * weighted; 2^-8
weighted covers the P V accumulation, 2^-8 |O_ref| the bf16 rounding of O.
LSE within 1e-3 + delta_i (its scores carry the same accumulation error).  At
the full-size causal N = 4096 case the mean squared error of O against plain
bf16 attention on the unquantized inputs stays below the 1e-4 the pages quote
for FP8 attention at N = 4096 (short or sharply peaked rows average over few
keys, so the figure is only checked where the pages give it)."""
import math
import time

import numpy as np
import pytest

from attn_inputs import dense_inputs
from oracle import attention as A
from oracle import fp8 as F
from parity_utils import to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_09_amd as M
    M.load()
    return M


def _say(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def _quant(lib, x, vt=False):
    import torch
    xd = to_dev(x, "bf16")
    B, H, N, d = xd.shape
    nb = -(-N // 64)
    if vt:
        codes = torch.empty((B, H, nb, d, 64), dtype=torch.uint8, device="cuda")
        scales = torch.empty((B, H), dtype=torch.float32, device="cuda")
        lib.attn_quantize_fp8_vt(xd, codes, scales)
    else:
        codes = torch.empty((B, H, N, d), dtype=torch.uint8, device="cuda")
        scales = torch.empty((B, H, nb), dtype=torch.float32, device="cuda")
        lib.attn_quantize_fp8_rows(xd, codes, scales)
    return codes, scales


@pytest.mark.parametrize("sigma", [1.0, 300.0, 1e-3])
@pytest.mark.parametrize("N", [1, 63, 64, 65, 200, 300])
def test_quantizers_bit_exact(lib, N, sigma):
    import torch
    print(f"[case] quantize N={N} sigma={sigma}", flush=True)
    x = dense_inputs(2, 3, N, 128, "bf16", seed=N, sigma_qk=sigma, with_do=False)["q"]
    if N > 64:
        x[0, 1, 64:128] = 0.0          # an all-zero block: scale 1, codes 0
    codes, scales = _quant(lib, x)
    vcodes, vscales = _quant(lib, x, vt=True)
    torch.cuda.synchronize()
    rc, rs = F.quantize_rows(x)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    hc, hs = F.quantize_heads(x)
    got, past_end = _untile_vt(vcodes.cpu().numpy(), N)
    np.testing.assert_array_equal(got, hc)
    assert np.all(past_end == 0)
    np.testing.assert_array_equal(vscales.cpu().numpy().view(np.uint32), hs.view(np.uint32))


def _every_bf16_by_maximum():
    """[1, H, 512, 128] bf16-exact inputs: head h holds a maximum M_h first,
    then every finite bf16 value of magnitude at most M_h (in bit order, so
    the 64-row blocks see many different maxima), then zeros.  The maxima
    run from subnormal bf16 numbers (scales far below 2^-60) to the largest
    finite bf16 (a scale near 2^120), with powers of two and values between."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    finite = bits[(bits & 0x7F80) != 0x7F80]
    vals = (finite << 16).view(np.float32)
    maxima = [float(np.array([b << 16], np.uint32).view(np.float32)[0])
              for b in (0x0001, 0x007F, 0x0080, 0x0D00, 0x1A55, 0x2000, 0x3000, 0x3A80, 0x3C00, 0x3F80,
                        0x3FC1, 0x4100, 0x4388, 0x4500, 0x5000, 0x5E00, 0x6A12, 0x7000, 0x7F00, 0x7F7F)]
    x = np.zeros((1, len(maxima), 512, 128), np.float32)
    for h, m in enumerate(maxima):
        keep = vals[np.abs(vals) <= m]
        flat = np.concatenate([[m], keep])
        assert flat.size <= 512 * 128
        x[0, h].reshape(-1)[:flat.size] = flat
    return x


def test_quantizers_every_bf16_value(lib):
    """Both quantizers, bit for bit against the oracle, on every finite bf16
    value (both zeros and the subnormals included) under twenty head and
    block maxima, so the codes and scales cover the whole E4M3 range and
    both ways the kernels divide by a scale."""
    import torch
    x = _every_bf16_by_maximum()
    codes, scales = _quant(lib, x)
    vcodes, vscales = _quant(lib, x, vt=True)
    torch.cuda.synchronize()
    rc, rs = F.quantize_rows(x)
    np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    hc, hs = F.quantize_heads(x)
    np.testing.assert_array_equal(vscales.cpu().numpy().view(np.uint32), hs.view(np.uint32))
    got, _ = _untile_vt(vcodes.cpu().numpy(), x.shape[2])
    np.testing.assert_array_equal(got, hc)


# The order attn_quantize_fp8_vt declares in include/miattn.h: position p of a
# 64-key tile holds key k(p) of the tile.
_VT_KEY_OF_POS = np.array([32 * ((p % 32) // 16) + 8 * ((p % 16) // 4) + 4 * (p // 32) + p % 4
                           for p in range(64)])
# attn_fwd_fp8 multiplies P by 2^6 before rounding it to E4M3 (include/miattn.h).
_P_SCALE_LOG2 = 6


def test_declared_vt_order_is_a_permutation():
    assert sorted(_VT_KEY_OF_POS.tolist()) == list(range(64))


def _untile_vt(v8t, N):
    """[B, H, nt, d, 64] codes in the declared tile order -> [B, H, N, d] codes
    in key order, plus the codes at positions whose key is past N."""
    B, H, nt, d, _ = v8t.shape
    keys = (64 * np.arange(nt)[:, None] + _VT_KEY_OF_POS[None, :]).reshape(-1)   # [nt*64] key of (t, p)
    flat = np.transpose(v8t, (0, 1, 2, 4, 3)).reshape(B, H, nt * 64, d)        # row (t, p)
    out = np.zeros((B, H, nt * 64, d), dtype=np.uint8)
    out[:, :, keys] = flat
    return out[:, :, :N], out[:, :, N:]


def _fwd(lib, q, k, v, scale, causal):
    import torch
    q8, sq = _quant(lib, q)
    k8, sk = _quant(lib, k)
    v8, sv = _quant(lib, v, vt=True)
    B, H, N, d = q.shape
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    lib.attn_fwd_fp8(q8, sq, k8, sk, v8, sv, o, lse, scale, causal)
    torch.cuda.synchronize()
    return to_np(o), to_np(lse)


def _check(o, lse, q, k, v, scale, causal, mse_bar=None):
    ref = F.fp8_reference(q, k, v, scale, causal)
    bound, weighted = F.fp8_output_bound(ref["qd"], ref["kd"], ref["vd"], ref["lse"], scale, causal,
                                         p_scale_log2=_P_SCALE_LOG2)
    err = np.abs(o - ref["o"])
    B, H, N, d = q.shape
    G = H // k.shape[1]
    delta = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            a_ = np.abs(ref["qd"][b, h]) @ np.abs(ref["kd"][b, h // G]).T
            if causal:
                a_ = np.where(np.tril(np.ones((N, N), bool)), a_, 0.0)
            delta[b, h] = 2.0 ** -12 * abs(scale) * a_.max(axis=1)
    allowed = bound + (2.0 ** -8 + delta[..., None]) * weighted + 2.0 ** -8 * np.abs(ref["o"])
    worst = np.max(err - allowed)
    _say(f"  max |O - O_ref| {err.max():.3e}, max bound {bound.max():.3e}, worst margin {worst:.3e}")
    assert worst <= 0, f"O outside the FP8 bound by {worst:.3e}"
    assert np.array_equal(np.isneginf(lse), np.isneginf(ref["lse"]))
    fin = np.isfinite(ref["lse"])
    lerr = np.abs(lse[fin] - ref["lse"][fin]) - (1e-3 + delta[fin])
    _say(f"  LSE worst margin {lerr.max():.3e}")
    assert lerr.max() <= 0
    o_plain, _ = A.gqa_forward(q, k, v, scale, causal)
    mse = float(np.mean((o - o_plain) ** 2))
    _say(f"  MSE vs bf16 attention {mse:.2e}")
    if mse_bar is not None:
        assert mse <= mse_bar


def test_fp8_score_accumulation_error(lib):
    """A row that sees a single key has LSE equal to its score, so single-key
    problems (N = 1) expose the FP8 MFMA's accumulation of the 128 products of
    a score.  Inputs are 2^-3 times E4M3 values with a 56 = 448 / 8 entry in
    each row, so quantization is lossless (scale exactly 1/8) and the exact
    score is the fp64 dot product of the bf16 inputs.  Signs are random, so
    the products cancel.  Bar: |LSE - score| <= 2^-13 |scale| sum_f |q_f k_f|
    plus four fp32 roundings of the score."""
    vals = F.e4m3_values()
    fin = np.array([c for c in range(1, 0x7F) if vals[c] <= 240])
    rng = np.random.default_rng(11)
    B, H, d = 64, 16, 128

    def draw():
        x = vals[rng.choice(fin, size=(B, H, 1, d))] * np.where(rng.random((B, H, 1, d)) < 0.5, -1.0, 1.0) / 8
        x[..., 0] = 56.0 * np.where(rng.random((B, H, 1)) < 0.5, -1.0, 1.0)
        return x.astype(np.float32)

    q, k, v = draw(), draw(), draw()
    rq, sq = F.quantize_rows(q)
    assert np.all(sq == np.float32(0.125)) and np.array_equal(F.dequantize_rows(rq, sq), q.astype(np.float64))
    worst = 0.0
    for scale in (1 / math.sqrt(128), 0.5, -0.3):
        _, lse = _fwd(lib, q, k, v, scale, False)
        score = scale * np.sum(q.astype(np.float64) * k, axis=3)[..., 0]
        mag = abs(scale) * np.sum(np.abs(q.astype(np.float64) * k), axis=3)[..., 0]
        err = np.abs(lse[..., 0] - score)
        allowed = 2.0 ** -13 * mag + 4 * 2.0 ** -24 * np.abs(score)
        worst = max(worst, float(np.max((err - 4 * 2.0 ** -24 * np.abs(score)) / mag)))
        assert np.all(err <= allowed), f"scale {scale}: accumulation error above 2^-13 of sum |q k|"
    _say(f"  FP8 score accumulation: worst |error| / sum |q k| = {worst:.3e} = 2^{math.log2(max(worst, 1e-30)):.2f}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,Hkv", [(1, 2), (17, 4), (64, 4), (200, 2), (333, 4), (1000, 1)])
def test_fp8_forward_ragged(lib, N, Hkv, causal):
    print(f"[case] fp8 fwd N={N} Hkv={Hkv} causal={causal}", flush=True)
    inp = dense_inputs(2, 4, N, 128, "bf16", seed=N + Hkv, kv_heads=Hkv, with_do=False)
    scale = 1 / math.sqrt(128)
    o, lse = _fwd(lib, inp["q"], inp["k"], inp["v"], scale, causal)
    _check(o, lse, inp["q"], inp["k"], inp["v"], scale, causal)


@pytest.mark.parametrize("scale", [0.0, -0.1, 0.3])
def test_fp8_scale_edge_cases(lib, scale):
    """scale = 0 (uniform average), negative, and sharp scores (0.3 with
    N(0, 2^2) Q and K)."""
    inp = dense_inputs(1, 2, 300, 128, "bf16", seed=9, sigma_qk=2.0, with_do=False)
    o, lse = _fwd(lib, inp["q"], inp["k"], inp["v"], scale, True)
    _check(o, lse, inp["q"], inp["k"], inp["v"], scale, True)


def test_fp8_full_size_causal(lib):
    """B=4, H=32, N=4096, d=128, causal, N(0,1) bf16, seed 0: two heads
    against the oracle, every head finite."""
    import torch
    _say("fp8 full size: generate")
    inp = dense_inputs(4, 32, 4096, 128, "bf16", seed=0, with_do=False)
    scale = 1 / math.sqrt(128)
    o, lse = _fwd(lib, inp["q"], inp["k"], inp["v"], scale, True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    for b, h in ((0, 0), (3, 21)):
        _say(f"oracle head b={b} h={h}")
        sl = (slice(b, b + 1), slice(h, h + 1))
        _check(o[sl], lse[sl], inp["q"][sl], inp["k"][sl], inp["v"][sl], scale, True, mse_bar=1e-4)


def test_fp8_key_scales_past_the_lds_table(lib):
    """One sequence longer than the forward's LDS table of per-tile K scales
    (2048 tiles of 64 keys): B1 H1 N 131264 (2051 key tiles), causal.  The
    query tile at row 130816 visits exactly 2048 key tiles (the table's
    last entry); the tiles from row 131072 on visit 2051 and read their K
    scales from memory.  Sampled rows on both sides of that limit, and early
    rows, against the oracle's row-restricted FP8 reference and bound."""
    N = 131264
    _say(f"fp8 N={N}: generate")
    inp = dense_inputs(1, 1, N, 128, "bf16", seed=5, with_do=False)
    scale = 1 / math.sqrt(128)
    o, lse = _fwd(lib, inp["q"], inp["k"], inp["v"], scale, True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    rows = np.array([0, 1, 4095, 65536, 130815, 130816, 131000, 131071, 131072, 131073, 131200, N - 2, N - 1])
    _say("oracle rows")
    ref = F.fp8_reference_rows(inp["q"], inp["k"], inp["v"], scale, True, rows)
    bound, weighted = F.fp8_output_bound(ref["qd"], ref["kd"], ref["vd"], ref["lse"], scale, True,
                                         p_scale_log2=_P_SCALE_LOG2, rows=rows)
    a_ = np.abs(ref["qd"][0, 0][rows]) @ np.abs(ref["kd"][0, 0]).T
    a_ = np.where(np.arange(N)[None, :] <= rows[:, None], a_, 0.0)
    delta = 2.0 ** -12 * abs(scale) * a_.max(axis=1)       # [R], the accumulation term of _check
    got_o, got_lse = o[0, 0][rows], lse[0, 0][rows]
    allowed = bound[0, 0] + (2.0 ** -8 + delta[:, None]) * weighted[0, 0] + 2.0 ** -8 * np.abs(ref["o"][0, 0])
    worst = np.max(np.abs(got_o - ref["o"][0, 0]) - allowed)
    _say(f"  worst O margin {worst:.3e}")
    assert worst <= 0, f"O outside the FP8 bound by {worst:.3e}"
    lerr = np.abs(got_lse - ref["lse"][0, 0]) - (1e-3 + delta)
    _say(f"  LSE worst margin {lerr.max():.3e}")
    assert lerr.max() <= 0
