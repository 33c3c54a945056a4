"""GPU parity of the grouped key/value head entry points (attn_fwd_gqa,
attn_bwd_gqa): query head h reads key/value head h // (H / H_kv).

Small and ragged sizes are compared element by element with the fp64 oracle
for several group sizes (H_kv = H is plain multi-head, H_kv = 1 is
multi-query).  At the Llama-style size B=4, H=32, H_kv=8, N=4096, d=128
(causal) whole key/value groups are checked against the oracle, and on every
head the forward and dQ must equal, bit for bit, the multi-head entry points
run on K and V repeated per query head: both read the same key/value rows in
the same order, only the head index differs."""
import math
import time

import numpy as np
import pytest

from attn_inputs import dense_inputs
from oracle import attention as A
from parity_utils import BF16_O_MAX_ABS, check_bf16, check_lse, to_dev, to_np

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


def _run_gqa(lib, inp, scale, causal):
    import torch
    q, k, v, do = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    lib.attn_fwd_gqa(q, k, v, o, lse, scale, causal)
    dq = torch.empty_like(q)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(lib.attn_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    lib.attn_bwd_gqa(q, k, v, o, lse, do, dq, dk, dv, scale, causal, ws)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def _check(out, ref, heads=None, groups=None):
    sel_h = (lambda x: x) if heads is None else (lambda x: x[heads])
    sel_g = (lambda x: x) if groups is None else (lambda x: x[groups])
    check_bf16(sel_h(to_np(out["o"])), sel_h(ref["o"]), "O", max_abs_tol=BF16_O_MAX_ABS)
    check_lse(sel_h(to_np(out["lse"])), sel_h(ref["lse"]))
    fro, mab = check_bf16(sel_h(to_np(out["dq"])), sel_h(ref["dq"]), "dq")
    _say(f"  dq: rel-fro {fro:.2e} max-abs {mab:.2e}")
    for name in ("dk", "dv"):
        fro, mab = check_bf16(sel_g(to_np(out[name])), sel_g(ref[name]), name)
        _say(f"  {name}: rel-fro {fro:.2e} max-abs {mab:.2e}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 63, 129, 200])
@pytest.mark.parametrize("Hkv", [1, 2, 4, 8])
def test_gqa_ragged(lib, Hkv, N, d, causal):
    print(f"[case] gqa H=8 Hkv={Hkv} N={N} d={d} causal={causal}", flush=True)
    inp = dense_inputs(2, 8, N, d, "bf16", seed=Hkv * 1000 + N + d, kv_heads=Hkv)
    scale = 1.0 / math.sqrt(d)
    out = _run_gqa(lib, inp, scale, causal)
    ref = A.gqa_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal)
    _check(out, ref)


def test_gqa_one_head_per_group_is_attn_fwd_bwd(lib):
    """H_kv = H through the grouped entry points equals attn_fwd / attn_bwd
    bit for bit."""
    import torch
    inp = dense_inputs(2, 4, 300, 128, "bf16", seed=17)
    scale = 1 / math.sqrt(128)
    out = _run_gqa(lib, inp, scale, True)
    q, k, v, do = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((2, 4, 300), dtype=torch.float32, device="cuda")
    lib.attn_fwd(q, k, v, o, lse, scale, True)
    g = [torch.empty_like(q) for _ in range(3)]
    ws = torch.empty(lib.attn_bwd_workspace_bytes(2, 4, 300, 128), dtype=torch.uint8, device="cuda")
    lib.attn_bwd(q, k, v, o, lse, do, *g, scale, True, ws)
    torch.cuda.synchronize()
    for name, t in (("o", o), ("lse", lse), ("dq", g[0]), ("dk", g[1]), ("dv", g[2])):
        assert torch.equal(out[name], t), name


def test_gqa_full_size_causal(lib):
    """B=4, H=32, H_kv=8, N=4096, d=128, causal, N(0,1) bf16 inputs, seed 0."""
    import torch
    _say("gqa full size: generate")
    B, H, Hkv, N, d = 4, 32, 8, 4096, 128
    G = H // Hkv
    inp = dense_inputs(B, H, N, d, "bf16", seed=0, kv_heads=Hkv)
    scale = 1 / math.sqrt(d)
    out = _run_gqa(lib, inp, scale, True)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert bool(torch.isfinite(out[name].float()).all()), f"non-finite {name}"
    # forward and dQ of every head against the multi-head path on repeated K/V
    _say("multi-head path on repeated K/V")
    q, do = to_dev(inp["q"], "bf16"), to_dev(inp["do"], "bf16")
    k_rep = torch.repeat_interleave(to_dev(inp["k"], "bf16"), G, dim=1).contiguous()
    v_rep = torch.repeat_interleave(to_dev(inp["v"], "bf16"), G, dim=1).contiguous()
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    lib.attn_fwd(q, k_rep, v_rep, o, lse, scale, True)
    g = [torch.empty_like(q) for _ in range(3)]
    ws = torch.empty(lib.attn_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    lib.attn_bwd(q, k_rep, v_rep, o, lse, do, *g, scale, True, ws)
    torch.cuda.synchronize()
    assert torch.equal(out["o"], o)
    assert torch.equal(out["lse"], lse)
    assert torch.equal(out["dq"], g[0])
    # dK / dV of a group are the group sums of the repeated heads' gradients
    # (fp32 sums of bf16-rounded terms against one fp32 sum: rounding only)
    dk_sum = g[1].float().view(B, Hkv, G, N, d).sum(2)
    dv_sum = g[2].float().view(B, Hkv, G, N, d).sum(2)
    for name, s in (("dk", dk_sum), ("dv", dv_sum)):
        check_bf16(to_np(out[name]), s.cpu().numpy().astype(np.float64), f"{name} vs group sum")
    del k_rep, v_rep, g
    # two whole key/value groups against the oracle
    for b, j in ((0, 0), (3, 7)):
        _say(f"oracle group b={b} j={j}")
        ref = A.gqa_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, True, groups=[(b, j)])
        hs = (b, slice(j * G, (j + 1) * G))
        _check(out, ref, heads=hs, groups=(b, j))
