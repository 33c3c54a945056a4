"""Repeat runs, bit for bit.

Every output of these entry points is formed without atomics: each element
is written by one workgroup, in a fixed order of operations.  So running the
same call three times on the same inputs must give the same bits.  A missing
barrier, an LDS hazard or a read of memory a concurrent workgroup is still
writing would show up here as a run-to-run difference.  The shapes are
mid-sized, so that hundreds of workgroups run at once: dense causal and not
at d 64 and 128, grouped heads, packed sequences with key padding, a sliding
window, a block list, split-KV decoding and the FP8 forward with its
quantizers."""
import math

import numpy as np
import pytest

from attn_inputs import decode_inputs, dense_inputs, left_padding_key_mask, varlen_inputs
from parity_utils import to_dev

pytestmark = pytest.mark.gpu

RUNS = 3


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_09_amd as M
    M.load()
    return M


def _same(runs):
    import torch
    first = runs[0]
    for other in runs[1:]:
        for name in first:
            assert torch.equal(first[name], other[name]), f"{name} differs between runs"


def _dense(lib, inp, scale, causal, mode=None, arg=None):
    import torch
    q, k, v, do = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if mode is None:
        ws = torch.empty(lib.attn_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
        fwd = lib.attn_fwd if k.shape[1] == H else lib.attn_fwd_gqa
        bwd = lib.attn_bwd if k.shape[1] == H else lib.attn_bwd_gqa
        outs = []
        for _ in range(RUNS):
            fwd(q, k, v, o, lse, scale, causal)
            bwd(q, k, v, o, lse, do, dq, dk, dv, scale, causal, ws)
            torch.cuda.synchronize()
            outs.append({n: t.clone() for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))})
        return outs
    outs = []
    if mode == "window":
        left, right = arg
        ws = torch.empty(lib.attn_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
        for _ in range(RUNS):
            lib.attn_fwd_window(q, k, v, o, lse, scale, causal, left, right)
            lib.attn_bwd_window(q, k, v, o, lse, do, dq, dk, dv, scale, causal, left, right, ws)
            torch.cuda.synchronize()
            outs.append({n: t.clone() for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))})
    else:
        rp, ci = (torch.from_numpy(np.asarray(x, np.int32)).cuda() for x in arg)
        ws = torch.empty(lib.attn_bwd_block_sparse_workspace_bytes(B, H, k.shape[1], N, d, int(ci.numel())),
                         dtype=torch.uint8, device="cuda")
        for _ in range(RUNS):
            lib.attn_fwd_block_sparse(q, k, v, o, lse, scale, causal, rp, ci)
            lib.attn_bwd_block_sparse(q, k, v, o, lse, do, dq, dk, dv, scale, causal, rp, ci, ws)
            torch.cuda.synchronize()
            outs.append({n: t.clone() for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))})
    return outs


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_repeat_dense(lib, d, causal):
    print(f"[case] repeat dense d={d} causal={causal}", flush=True)
    inp = dense_inputs(2, 8, 2048 + 37, d, "bf16", seed=51)
    _same(_dense(lib, inp, 1 / math.sqrt(d), causal))


def test_repeat_grouped_heads(lib):
    print("[case] repeat grouped heads", flush=True)
    inp = dense_inputs(2, 16, 1500, 128, "bf16", seed=52, kv_heads=4)
    _same(_dense(lib, inp, 1 / math.sqrt(128), True))


def test_repeat_window_and_blocks(lib):
    print("[case] repeat window and block list", flush=True)
    inp = dense_inputs(1, 8, 4096, 128, "bf16", seed=53, kv_heads=2)
    _same(_dense(lib, inp, 1 / math.sqrt(128), True, "window", (700, 0)))
    nb = 4096 // 128
    rows = [sorted({0} | {c for c in (r - 1, r, r + 1) if 0 <= c < nb} | set(range(0, nb, 8))) for r in range(nb)]
    rp = np.zeros(nb + 1, np.int32)
    rp[1:] = np.cumsum([len(r) for r in rows])
    ci = np.array([c for r in rows for c in r], np.int32)
    _same(_dense(lib, inp, 1 / math.sqrt(128), False, "blocks", (rp, ci)))


def test_repeat_packed_with_key_padding(lib):
    import torch
    print("[case] repeat packed sequences with key padding", flush=True)
    inp = varlen_inputs(9, 1, 1, 8, 128, "bf16", seed=54, lengths=[3000, 1, 700, 2049, 0, 64, 1500, 333, 4096])
    cu = inp["cu_seqlens"]
    kv = torch.from_numpy(left_padding_key_mask(cu, 0.02)).cuda()
    q, k, v, do = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    T, H, d = q.shape
    cu_d = torch.from_numpy(cu).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(lib.attn_bwd_varlen_workspace_bytes(T, H, d), dtype=torch.uint8, device="cuda")
    scale = 1 / math.sqrt(d)
    outs = []
    for _ in range(RUNS):
        lib.attn_fwd_varlen(q, k, v, o, lse, cu_d, inp["max_seqlen"], scale, True, kv)
        lib.attn_bwd_varlen(q, k, v, o, lse, do, dq, dk, dv, cu_d, inp["max_seqlen"], scale, True, ws, kv)
        torch.cuda.synchronize()
        outs.append({n: t.clone() for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))})
    _same(outs)


def test_repeat_decode(lib):
    import torch
    print("[case] repeat split-KV decode", flush=True)
    x = decode_inputs(4, 32, 8, 20000, 128, "bf16", seed=55)
    q, kc, vc = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    B, H, d = q.shape
    Hkv, N = kc.shape[1], kc.shape[2]
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    sl = torch.tensor([20000, 1, 12345, 0], dtype=torch.int32, device="cuda")
    ws = torch.empty(lib.attn_decode_workspace_bytes(B, H, Hkv, N, d), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(RUNS):
        lib.attn_decode(q, kc, vc, o, lse, 1 / math.sqrt(d), sl, ws)
        torch.cuda.synchronize()
        outs.append({"o": o.clone(), "lse": lse.clone()})
    _same(outs)


def test_repeat_fp8(lib):
    import torch
    print("[case] repeat FP8 quantizers and forward", flush=True)
    inp = dense_inputs(2, 8, 2048 + 37, 128, "bf16", seed=56, with_do=False)
    x = {n: to_dev(inp[n], "bf16") for n in ("q", "k", "v")}
    B, H, N, d = x["q"].shape
    nb = -(-N // 64)
    outs = []
    for _ in range(RUNS):
        q8, k8 = (torch.empty((B, H, N, d), dtype=torch.uint8, device="cuda") for _ in range(2))
        v8 = torch.empty((B, H, nb, d, 64), dtype=torch.uint8, device="cuda")
        sq, sk = (torch.empty((B, H, nb), dtype=torch.float32, device="cuda") for _ in range(2))
        sv = torch.empty((B, H), dtype=torch.float32, device="cuda")
        lib.attn_quantize_fp8_rows(x["q"], q8, sq)
        lib.attn_quantize_fp8_rows(x["k"], k8, sk)
        lib.attn_quantize_fp8_vt(x["v"], v8, sv)
        o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        lib.attn_fwd_fp8(q8, sq, k8, sk, v8, sv, o, lse, 1 / math.sqrt(d), True)
        torch.cuda.synchronize()
        outs.append({"q8": q8, "sq": sq, "v8": v8, "sv": sv, "o": o, "lse": lse})
    _same(outs)
