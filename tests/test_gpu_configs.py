"""GPU parity at the five workload configurations, at full size, through the
same entry points and launch configuration the benchmark times.

Every head of every configuration is compared with the fp64 oracle:
  * whole heads element by element for a few heads per configuration (with
    the largest relative Frobenius error over 64-row tiles printed beside the
    head-wide bar);
  * every other head through oracle.attention.head_backward_sampled: O and
    LSE of every row of the head, dQ at 32 query rows and dK, dV at 32 key
    columns (always including the first two and last two of the head);
    packed sequences: 8 rows and 8 key columns of every sequence of every
    head.  The gradients' bar, a relative Frobenius error over the whole
    tensor, is applied to its estimate from the sample (each drawn row
    weighted by the share of the head it stands for); the worst single row
    is printed beside it.
Properties that hold at any size are checked too: finite outputs, the -inf
pattern of LSE, and for causal problems the first row of every head (it sees
one key: O_0 = V_0 exactly, LSE_0 = scale * q_0 . k_0).  The oracle work runs
on a thread pool over the host's cores."""
import math
import time

import numpy as np
import pytest

from attn_inputs import dense_inputs, left_padding_key_mask, varlen_inputs
from oracle import attention as A
from parity_utils import (BF16_O_MAX_ABS, LSE_MAX_ABS, check_bf16, check_bf16_sampled, check_f32, check_lse,
                          map_heads, sample_positions, tile_rel_fro_max, to_dev, to_np)

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


def _dense_run(lib, inp, scale, causal, bwd):
    import torch
    q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    lib.attn_fwd(q, k, v, o, lse, scale, causal)
    out = {"o": o, "lse": lse}
    if bwd:
        do = to_dev(inp["do"], "bf16")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        ws = torch.empty(lib.attn_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
        lib.attn_bwd(q, k, v, o, lse, do, dq, dk, dv, scale, causal, ws)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return out


def _all_heads_properties(out, inp, scale, causal):
    o = out["o"]
    lse = out["lse"]
    import torch
    assert bool(torch.isfinite(o.float()).all()), "non-finite O"
    assert bool(torch.isfinite(lse).all()), "non-finite LSE (no row is fully masked here)"
    for g in ("dq", "dk", "dv"):
        if g in out:
            assert bool(torch.isfinite(out[g].float()).all()), f"non-finite {g}"
    if causal:
        o0 = to_np(o[:, :, 0, :])
        np.testing.assert_array_equal(o0, inp["v"][:, :, 0, :].astype(np.float64))
        s00 = scale * np.einsum("bhd,bhd->bh", inp["q"][:, :, 0, :].astype(np.float64),
                                inp["k"][:, :, 0, :].astype(np.float64))
        assert np.max(np.abs(to_np(lse[:, :, 0]) - s00)) <= LSE_MAX_ABS


def _check_heads(out, inp, scale, causal, heads, bwd):
    for (b, h) in heads:
        _say(f"oracle head b={b} h={h}")
        if bwd:
            dq, dk, dv, o, lse, _ = A.head_backward(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h],
                                                    inp["do"][b, h], scale, causal)
        else:
            o, lse = A.head_forward(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h], scale, causal)
        check_bf16(to_np(out["o"][b, h]), o, f"O[{b},{h}]", max_abs_tol=BF16_O_MAX_ABS)
        check_lse(to_np(out["lse"][b, h]), lse)
        if bwd:
            for name, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
                g = to_np(out[name][b, h])
                fro, mab = check_bf16(g, ref, f"{name}[{b},{h}]")
                _say(f"  {name}: rel-fro {fro:.2e} max-abs {mab:.2e} worst 64-row tile {tile_rel_fro_max(g, ref):.2e}")


def _host_outputs(out):
    """Device outputs -> float32 numpy (bf16 values are exact in float32)."""
    return {n: t.detach().float().cpu().numpy() for n, t in out.items()}


def _sampled_dense_head(job):
    """One head against head_backward_sampled: O and LSE of every row, dQ at
    the sampled rows, dK and dV at the sampled key columns."""
    label, q, k, v, do, scale, causal, (rows, rw), (cols, cw), g = job
    dq, dk, dv, o, lse, _ = A.head_backward_sampled(q, k, v, do, scale, causal, None, rows, cols)
    fo, _ = check_bf16(g["o"], o, f"O{label}", max_abs_tol=BF16_O_MAX_ABS)
    check_lse(g["lse"], lse, what=f"LSE{label}")
    res = {"o": fo, "o_tile": tile_rel_fro_max(g["o"], o)}
    if len(rows):
        for name, got, ref, w in (("dq", g["dq"], dq, rw), ("dk", g["dk"], dk, cw), ("dv", g["dv"], dv, cw)):
            res[name], res[name + "_row"] = check_bf16_sampled(got, ref, w, f"{name}{label}")
    return res


def _every_head(inp, outh, scale, causal, heads, bwd, seed):
    """Sampled oracle check of the given (b, h) heads, in parallel."""
    jobs = []
    N = inp["q"].shape[2]
    for (b, h) in heads:
        rng = np.random.default_rng(seed * 100003 + b * 1009 + h)
        rows = sample_positions(N, 32, rng)
        cols = sample_positions(N, 32, rng)
        g = {"o": outh["o"][b, h], "lse": outh["lse"][b, h]}
        if bwd:
            g.update(dq=outh["dq"][b, h][rows[0]], dk=outh["dk"][b, h][cols[0]], dv=outh["dv"][b, h][cols[0]])
        none = (np.zeros(0, np.int64), np.zeros(0))
        jobs.append((f"[{b},{h}]", inp["q"][b, h], inp["k"][b, h], inp["v"][b, h],
                     inp["do"][b, h] if bwd else inp["q"][b, h], scale, causal,
                     rows if bwd else none, cols if bwd else none, g))
    res = map_heads(_sampled_dense_head, jobs)
    worst = {key: max(r[key] for r in res) for key in res[0]}
    _say(f"  {len(heads)} heads sampled; worst rel-fro " + ", ".join(f"{k_} {v_:.2e}" for k_, v_ in worst.items()))


def test_config2_fwd_noncausal_d64(lib):
    """B=8, H=16, N=2048, d=64, bf16 forward, non-causal, scale 1/8, seed 0."""
    _say("config 2: generate")
    inp = dense_inputs(8, 16, 2048, 64, "bf16", seed=0, with_do=False)
    out = _dense_run(lib, inp, 1 / 8, False, bwd=False)
    _all_heads_properties(out, inp, 1 / 8, False)
    _check_heads(out, inp, 1 / 8, False, [(0, 0), (3, 9), (7, 15)], bwd=False)
    _every_head(inp, _host_outputs(out), 1 / 8, False, [(b, h) for b in range(8) for h in range(16)], False, 2)


@pytest.fixture(scope="module")
def config3(lib):
    """B=4, H=32, N=4096, d=128, bf16 causal forward and backward, seed 0:
    inputs and the GPU's outputs on the host."""
    _say("config 3: generate")
    inp = dense_inputs(4, 32, 4096, 128, "bf16", seed=0)
    scale = 1 / math.sqrt(128)
    out = _dense_run(lib, inp, scale, True, bwd=True)
    _all_heads_properties(out, inp, scale, True)
    return inp, out, _host_outputs(out), scale


def test_config3_fwd_bwd_causal_d128(config3):
    """Three whole heads element by element."""
    inp, out, _, scale = config3
    _check_heads(out, inp, scale, True, [(0, 0), (2, 17), (3, 31)], bwd=True)


@pytest.mark.parametrize("batch", [0, 1, 2, 3])
def test_config3_every_head_sampled(config3, batch):
    """All 32 heads of one batch entry against the sampled oracle."""
    inp, _, outh, scale = config3
    _say(f"config 3: batch {batch}, every head sampled")
    _every_head(inp, outh, scale, True, [(batch, h) for h in range(32)], True, 3)


def test_short_sequences_noncausal_d64(lib):
    """B=64, H=16, N=512, d=64, bf16 forward and backward, non-causal: the
    short-sequence shape the benchmark times (two 256-row query tiles per
    head, 32768 tokens in all)."""
    _say("short sequences: generate")
    inp = dense_inputs(64, 16, 512, 64, "bf16", seed=0)
    out = _dense_run(lib, inp, 1 / 8, False, bwd=True)
    _all_heads_properties(out, inp, 1 / 8, False)
    _check_heads(out, inp, 1 / 8, False, [(0, 0), (31, 7), (63, 15)], bwd=True)
    _every_head(inp, _host_outputs(out), 1 / 8, False, [(b, h) for b in range(64) for h in range(16)], True, 6)


def test_d_prepass_benchmark_shape(lib):
    """The backward's D pre-pass (attn_bwd_preprocess) at B=4, H=32, N=4096,
    d=128, on the forward's own bf16 O: every row of D against the oracle's
    rowsum(dO o O) in fp64.  The bound is fp32 summation of 128 products,
    1e-5 of sum |dO o O| per row.  The dQ pass's D (attn_bwd_dq_preprocess)
    must be the same bits."""
    import torch
    _say("D pre-pass: generate")
    B, H, N, d = 4, 32, 4096, 128
    inp = dense_inputs(B, H, N, d, "bf16", seed=0)
    q, k, v, do = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    scale = 1 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    lib.attn_fwd(q, k, v, o, lse, scale, True)
    ws = torch.empty(lib.attn_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    lib.attn_bwd_preprocess(o, do, ws)
    torch.cuda.synchronize()
    d_gpu = ws[: B * H * N * 4].view(torch.float32).view(B, H, N).clone()
    o_h = to_np(o)
    ref = A.preprocess_d(o_h, inp["do"])
    bound = 1e-5 * A.preprocess_d(np.abs(o_h), np.abs(inp["do"])) + 1e-30
    err = np.abs(to_np(d_gpu) - ref)
    _say(f"  D: max abs err {err.max():.2e}, max err / bound {np.max(err / bound):.3f}")
    assert np.all(err <= bound)
    ws.zero_()
    dq = torch.empty_like(q)
    lib.attn_bwd_dq_preprocess(q, k, v, o, lse, do, dq, scale, True, ws)
    torch.cuda.synchronize()
    assert torch.equal(ws[: B * H * N * 4].view(torch.float32).view(B, H, N), d_gpu)


@pytest.fixture(scope="module")
def config4(lib):
    """B=1, H=16, N=16384, d=128, causal, Q and K ~ N(0, 1.5^2): the running
    max moves often."""
    _say("config 4: generate")
    inp = dense_inputs(1, 16, 16384, 128, "bf16", seed=0, sigma_qk=1.5)
    scale = 1 / math.sqrt(128)
    out = _dense_run(lib, inp, scale, True, bwd=True)
    _all_heads_properties(out, inp, scale, True)
    return inp, out, _host_outputs(out), scale


def test_config4_long_sequence_sharp_scores(config4):
    """Head 0 whole, element by element."""
    inp, out, _, scale = config4
    _check_heads(out, inp, scale, True, [(0, 0)], bwd=True)


@pytest.mark.parametrize("part", [0, 1, 2, 3])
def test_config4_every_head_sampled(config4, part):
    """Heads 4 part .. 4 part + 3 against the sampled oracle."""
    inp, _, outh, scale = config4
    _say(f"config 4: heads {4 * part}..{4 * part + 3} sampled")
    _every_head(inp, outh, scale, True, [(0, h) for h in range(4 * part, 4 * part + 4)], True, 4)


@pytest.fixture(scope="module")
def config5(lib):
    """16 packed sequences with lengths uniform in [64, 8192], H=32, d=128,
    causal, with left key padding that fully masks ~1% of query rows."""
    import torch
    _say("config 5: generate")
    inp = varlen_inputs(16, 64, 8192, 32, 128, "bf16", seed=0)
    cu = inp["cu_seqlens"]
    kv = left_padding_key_mask(cu, 0.01)
    T = int(cu[-1])
    scale = 1 / math.sqrt(128)
    q, k, v, do = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    cu_d = torch.from_numpy(cu).cuda()
    kv_d = torch.from_numpy(kv).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((32, T), dtype=torch.float32, device="cuda")
    lib.attn_fwd_varlen(q, k, v, o, lse, cu_d, inp["max_seqlen"], scale, True, kv_d, cu_seqlens_host=cu)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(lib.attn_bwd_varlen_workspace_bytes(T, 32, 128), dtype=torch.uint8, device="cuda")
    lib.attn_bwd_varlen(q, k, v, o, lse, do, dq, dk, dv, cu_d, inp["max_seqlen"], scale, True, ws, kv_d,
                        cu_seqlens_host=cu)
    torch.cuda.synchronize()
    out = {n: t.float().cpu().numpy() for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))}
    return inp, kv, out, scale


def test_config5_varlen_keypad_causal(config5):
    """Every head: the fully masked rows are exactly the left-padded
    positions, with O = 0 and zero gradients; head 5 over every sequence and
    head 30 over the two shortest, whole."""
    inp, kv, out, scale = config5
    cu = inp["cu_seqlens"]
    T = int(cu[-1])
    dead_expected = np.zeros(T, bool)
    for s in range(16):
        dead_expected[cu[s]:cu[s + 1]] = np.cumsum(kv[cu[s]:cu[s + 1]]) == 0
    frac = dead_expected.mean()
    _say(f"T={T}, fully masked rows {dead_expected.sum()} ({100 * frac:.2f}%)")
    assert 0.005 < frac < 0.02
    assert np.array_equal(np.isneginf(out["lse"]), np.broadcast_to(dead_expected, (32, T)))
    assert np.all(out["o"][dead_expected] == 0) and np.all(out["dq"][dead_expected] == 0)
    assert np.all(out["dk"][kv == 0] == 0) and np.all(out["dv"][kv == 0] == 0)
    for name in ("o", "dq", "dk", "dv"):
        assert np.all(np.isfinite(out[name])), name
    lengths = np.diff(cu)
    for h, seqs in ((5, list(range(16))), (30, list(np.argsort(lengths)[:2]))):
        _say(f"oracle head {h} over {len(seqs)} sequences")
        ref = A.varlen_backward(inp["q"], inp["k"], inp["v"], inp["do"], cu, scale, True, kv, seqs=seqs, heads=[h])
        sel = np.zeros(T, bool)
        for s in seqs:
            sel[cu[s]:cu[s + 1]] = True
        check_bf16(out["o"][sel, h], ref["o"][sel, h], f"O[:, {h}]", max_abs_tol=BF16_O_MAX_ABS)
        check_lse(out["lse"][h, sel], ref["lse"][h, sel])
        for name in ("dq", "dk", "dv"):
            g = out[name][sel, h]
            fro, mab = check_bf16(g, ref[name][sel, h], f"{name}[:, {h}]")
            _say(f"  {name}: rel-fro {fro:.2e} max-abs {mab:.2e} worst 64-row tile "
                 f"{tile_rel_fro_max(g, ref[name][sel, h]):.2e}")


def _sampled_packed_head(job):
    """One head of the packed problem: every sequence through
    head_backward_sampled (O and LSE of every row, dQ at 8 rows and dK, dV at
    8 key columns per sequence); the bar applies over the head's samples."""
    h, inp, kv, out, scale = job
    cu = inp["cu_seqlens"]
    rng = np.random.default_rng(5000 + h)
    acc = {n: ([], [], []) for n in ("dq", "dk", "dv")}
    og, orf = [], []
    for s in range(len(cu) - 1):
        t0, t1 = int(cu[s]), int(cu[s + 1])
        L = t1 - t0
        rows, rw = sample_positions(L, 8, rng)
        cols, cw = sample_positions(L, 8, rng)
        sl = slice(t0, t1)
        dq, dk, dv, o, lse, _ = A.head_backward_sampled(inp["q"][sl, h], inp["k"][sl, h], inp["v"][sl, h],
                                                        inp["do"][sl, h], scale, True, kv[sl], rows, cols)
        check_lse(out["lse"][h, sl], lse, what=f"LSE[seq {s}, head {h}]")
        og.append(out["o"][sl, h])
        orf.append(o)
        for name, got, ref, w in (("dq", out["dq"][sl, h][rows], dq, rw), ("dk", out["dk"][sl, h][cols], dk, cw),
                                  ("dv", out["dv"][sl, h][cols], dv, cw)):
            acc[name][0].append(got)
            acc[name][1].append(ref)
            acc[name][2].append(w)
    res = {"o": check_bf16(np.concatenate(og), np.concatenate(orf), f"O[head {h}]", max_abs_tol=BF16_O_MAX_ABS)[0]}
    for name, (gs, rs, ws) in acc.items():
        res[name], res[name + "_row"] = check_bf16_sampled(np.concatenate(gs), np.concatenate(rs),
                                                           np.concatenate(ws), f"{name}[head {h}] samples")
    return res


@pytest.mark.parametrize("part", [0, 1, 2, 3])
def test_config5_every_head_sampled(config5, part):
    """Heads 8 part .. 8 part + 7, every sequence, against the sampled oracle."""
    inp, kv, out, scale = config5
    _say(f"config 5: heads {8 * part}..{8 * part + 7} sampled")
    res = map_heads(_sampled_packed_head, [(h, inp, kv, out, scale) for h in range(8 * part, 8 * part + 8)])
    worst = {key: max(r[key] for r in res) for key in res[0]}
    _say("  worst rel-fro " + ", ".join(f"{k_} {v_:.2e}" for k_, v_ in worst.items()))


def test_config1_fwd_bwd_f32(lib):
    """B=1, H=1, N=128, d=64 fp32, non-causal, seed 0: within 1e-5."""
    import torch
    inp = dense_inputs(1, 1, 128, 64, "f32", seed=0)
    q, k, v, do = (to_dev(inp[n], "f32") for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, 128), dtype=torch.float32, device="cuda")
    lib.attn_fwd_f32(q, k, v, o, lse, 1 / 8, False)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(lib.attn_bwd_f32_workspace_bytes(1, 1, 128, 64), dtype=torch.uint8, device="cuda")
    lib.attn_bwd_f32(q, k, v, o, lse, do, dq, dk, dv, 1 / 8, False, ws)
    torch.cuda.synchronize()
    ref = A.backward(inp["q"], inp["k"], inp["v"], inp["do"], 1 / 8, False)
    check_f32(to_np(o), ref["o"], "O")
    check_lse(to_np(lse), ref["lse"], tol=1e-5)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        check_f32(to_np(t), ref[name], name)
