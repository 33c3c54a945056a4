"""GPU parity at small and ragged sizes: every output element against the fp64
oracle on the same seeded inputs, through the C ABI.  Sizes span several tiles
and a ragged tail; edge cases: a single key, zero and negative scale, very
large scores, fully masked rows."""
import math

import numpy as np
import pytest

from attn_inputs import dense_inputs, left_padding_key_mask, varlen_inputs
from oracle import attention as A
from parity_utils import (BF16_O_MAX_ABS, check_bf16, check_f32, check_lse, to_dev, to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_09_amd as M
    M.load()
    return M


def _run_dense(lib, inp, scale, causal, dtype, bwd=True):
    import torch
    q, k, v = (to_dev(inp[n], dtype) for n in ("q", "k", "v"))
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fwd = lib.attn_fwd if dtype == "bf16" else lib.attn_fwd_f32
    fwd(q, k, v, o, lse, scale, causal)
    out = {"o": o, "lse": lse}
    if bwd:
        do = to_dev(inp["do"], dtype)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        wsb = lib.attn_bwd_workspace_bytes if dtype == "bf16" else lib.attn_bwd_f32_workspace_bytes
        ws = torch.empty(wsb(B, H, N, d), dtype=torch.uint8, device="cuda")
        bw = lib.attn_bwd if dtype == "bf16" else lib.attn_bwd_f32
        bw(q, k, v, o, lse, do, dq, dk, dv, scale, causal, ws)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {k_: to_np(v_) for k_, v_ in out.items()}


def _check(out, ref, dtype, f32_relative=False):
    """f32: max abs <= 1e-5; with ``f32_relative`` the bar is 1e-5 times the
    largest reference magnitude (when above 1), for inputs scaled well past
    unit variance where fp32 rounding alone exceeds 1e-5."""
    if dtype == "f32":
        def tol(r):
            return 1e-5 * (max(1.0, float(np.max(np.abs(r)))) if f32_relative else 1.0)
        check_f32(out["o"], ref["o"], "O", tol(ref["o"]))
        fin = np.isfinite(ref["lse"])
        check_lse(out["lse"], ref["lse"], tol=tol(ref["lse"][fin]))
        for g in ("dq", "dk", "dv"):
            if g in out:
                check_f32(out[g], ref[g], g, tol(ref[g]))
    else:
        check_bf16(out["o"], ref["o"], "O", max_abs_tol=BF16_O_MAX_ABS)
        check_lse(out["lse"], ref["lse"])
        for g in ("dq", "dk", "dv"):
            if g in out:
                check_bf16(out[g], ref[g], g)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 17, 63, 64, 65, 127, 129, 300])
def test_bf16_fwd_bwd_ragged(lib, N, d, causal):
    print(f"[case] bf16 N={N} d={d} causal={causal}", flush=True)
    inp = dense_inputs(2, 3, N, d, "bf16", seed=N * 7 + d)
    scale = 1.0 / math.sqrt(d)
    out = _run_dense(lib, inp, scale, causal, "bf16")
    ref = A.backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal)
    _check(out, ref, "bf16")


@pytest.mark.parametrize("B,H,N,causal", [(1, 24, 768, True), (1, 40, 768, True), (2, 8, 1024, True),
                                          (1, 24, 1100, False), (2, 8, 1024, False)])
def test_order_with_narrowed_head_groups(lib, B, H, N, causal):
    """Shapes whose XCD ranges hold 3, 5 and 2 heads, so the query-tile order
    narrows its group of four heads to 3, 1 and 2 (non-causal passes group
    heads from 4 query tiles a head on, here with a ragged last tile): every
    head of the forward and the backward against the oracle."""
    print(f"[case] narrowed head groups B={B} H={H} N={N} causal={causal}", flush=True)
    inp = dense_inputs(B, H, N, 64, "bf16", seed=B * 100 + H)
    scale = 1.0 / 8.0
    out = _run_dense(lib, inp, scale, causal, "bf16")
    ref = A.backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal)
    _check(out, ref, "bf16")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 31, 32, 33, 128, 200])
def test_f32_fwd_bwd_ragged(lib, N, d, causal):
    print(f"[case] f32 N={N} d={d} causal={causal}", flush=True)
    inp = dense_inputs(2, 2, N, d, "f32", seed=N * 11 + d)
    scale = 1.0 / math.sqrt(d)
    out = _run_dense(lib, inp, scale, causal, "f32")
    ref = A.backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal)
    _check(out, ref, "f32")


def test_config1_f32_exact_problem(lib):
    """B=1, H=1, N=128, d=64 fp32, non-causal, scale 1/8, N(0,1) from seed 0,
    32 x 32 tiles: O, LSE, dQ, dK, dV within 1e-5 of the oracle."""
    inp = dense_inputs(1, 1, 128, 64, "f32", seed=0)
    out = _run_dense(lib, inp, 1.0 / 8.0, False, "f32")
    ref = A.backward(inp["q"], inp["k"], inp["v"], inp["do"], 1.0 / 8.0, False)
    _check(out, ref, "f32")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [0.0, -0.2, 0.9])
def test_scale_edge_cases(lib, dtype, scale):
    """scale = 0 (uniform average), a negative scale, and large scores
    (scale 0.9 with N(0, 2^2) inputs) under a causal mask."""
    print(f"[case] scale={scale} dtype={dtype}", flush=True)
    inp = dense_inputs(1, 2, 150, 64, dtype, seed=5, sigma_qk=2.0)
    out = _run_dense(lib, inp, scale, True, dtype)
    ref = A.backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, True)
    _check(out, ref, dtype, f32_relative=True)


def _run_varlen(lib, inp, scale, causal, key_valid=None, bwd=True):
    import torch
    q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
    T, H, d = q.shape
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    kv = None if key_valid is None else torch.from_numpy(key_valid).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
    lib.attn_fwd_varlen(q, k, v, o, lse, cu, inp["max_seqlen"], scale, causal, kv)
    out = {"o": o, "lse": lse}
    if bwd:
        do = to_dev(inp["do"], "bf16")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        ws = torch.empty(lib.attn_bwd_varlen_workspace_bytes(T, H, d), dtype=torch.uint8, device="cuda")
        lib.attn_bwd_varlen(q, k, v, o, lse, do, dq, dk, dv, cu, inp["max_seqlen"], scale, causal, ws, kv)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {k_: to_np(v_) for k_, v_ in out.items()}


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_varlen_ragged(lib, causal, padded, d):
    print(f"[case] varlen causal={causal} padded={padded} d={d}", flush=True)
    inp = varlen_inputs(6, 1, 1, 3, d, "bf16", seed=d, lengths=[1, 70, 257, 64, 5, 130])
    kv = left_padding_key_mask(inp["cu_seqlens"], frac=0.05) if padded else None
    scale = 1.0 / math.sqrt(d)
    out = _run_varlen(lib, inp, scale, causal, kv)
    ref = A.varlen_backward(inp["q"], inp["k"], inp["v"], inp["do"], inp["cu_seqlens"], scale, causal, kv)
    _check(out, ref, "bf16")
    if padded and causal:
        dead = np.isneginf(ref["lse"])
        assert dead.any()
        o_rows = out["o"].transpose(1, 0, 2)[dead]
        assert np.array_equal(o_rows, np.zeros_like(o_rows))
        g_rows = out["dq"].transpose(1, 0, 2)[dead]
        assert np.array_equal(g_rows, np.zeros_like(g_rows))


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_empty_sequences(lib, causal):
    """Zero-length sequences first, in the middle and last of a packed batch:
    their workgroups exit at once and the neighbours' rows are unaffected."""
    print(f"[case] varlen empty sequences causal={causal}", flush=True)
    inp = varlen_inputs(6, 1, 1, 2, 128, "bf16", seed=11, lengths=[0, 70, 0, 0, 129, 0])
    assert int(inp["cu_seqlens"][-1]) == 199
    out = _run_varlen(lib, inp, 128 ** -0.5, causal)
    ref = A.varlen_backward(inp["q"], inp["k"], inp["v"], inp["do"], inp["cu_seqlens"], 128 ** -0.5, causal)
    _check(out, ref, "bf16")


def test_whole_sequence_padded(lib):
    """A sequence whose keys are all padded: every row is fully masked, even
    without a causal mask, and its K/V receive no gradient."""
    inp = varlen_inputs(3, 1, 1, 2, 64, "bf16", seed=3, lengths=[40, 100, 33])
    kv = np.ones(int(inp["cu_seqlens"][-1]), np.uint8)
    kv[40:140] = 0
    out = _run_varlen(lib, inp, 0.125, False, kv)
    ref = A.varlen_backward(inp["q"], inp["k"], inp["v"], inp["do"], inp["cu_seqlens"], 0.125, False, kv)
    _check(out, ref, "bf16")
    assert np.all(np.isneginf(out["lse"][:, 40:140]))
    assert np.all(out["o"][40:140] == 0) and np.all(out["dk"][40:140] == 0) and np.all(out["dv"][40:140] == 0)


def test_backward_stages_match_attn_bwd(lib):
    """attn_bwd == attn_bwd_preprocess + attn_bwd_dkdv + attn_bwd_dq ==
    attn_bwd_dq_preprocess + attn_bwd_dkdv, bitwise (no output of the bf16
    backward is accumulated with atomics, and the dQ pass forms D in the
    pre-pass's summation order)."""
    import torch
    inp = dense_inputs(2, 4, 500, 128, "bf16", seed=21)
    q, k, v, do = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    scale = 1 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    lib.attn_fwd(q, k, v, o, lse, scale, True)
    ws = torch.empty(lib.attn_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    g1 = [torch.empty_like(q) for _ in range(3)]
    g2 = [torch.empty_like(q) for _ in range(3)]
    lib.attn_bwd(q, k, v, o, lse, do, *g1, scale, True, ws)
    lib.attn_bwd_preprocess(o, do, ws)
    lib.attn_bwd_dkdv(q, k, v, lse, do, g2[1], g2[2], scale, True, ws)
    lib.attn_bwd_dq(q, k, v, lse, do, g2[0], scale, True, ws)
    torch.cuda.synchronize()
    for a_, b_ in zip(g1, g2):
        assert torch.equal(a_, b_)
    d_pre = ws[: B * H * N * 4].clone()
    g3 = [torch.empty_like(q) for _ in range(3)]
    lib.attn_bwd(q, k, v, o, lse, do, *g3, scale, True, ws)
    torch.cuda.synchronize()
    for a_, b_ in zip(g1, g3):
        assert torch.equal(a_, b_)
    ws.zero_()
    g4 = [torch.empty_like(q) for _ in range(3)]
    lib.attn_bwd_dq_preprocess(q, k, v, o, lse, do, g4[0], scale, True, ws)
    torch.cuda.synchronize()
    assert torch.equal(ws[: B * H * N * 4], d_pre)   # the same D, bit for bit
    lib.attn_bwd_dkdv(q, k, v, lse, do, g4[1], g4[2], scale, True, ws)
    torch.cuda.synchronize()
    for a_, b_ in zip(g1, g4):
        assert torch.equal(a_, b_)


def test_launch_errors_surface(lib):
    import torch
    from exact_tiled_attention_09_amd import MiattnError
    q = torch.zeros((1, 1, 16, 96), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 1, 16), dtype=torch.float32, device="cuda")
    with pytest.raises(MiattnError) as e:
        lib.attn_fwd(q, q, q, q.clone(), lse, 0.1, False)
    assert e.value.status == -2
