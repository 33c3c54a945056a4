"""Tensors past 2^31 elements (dense, packed, the decode caches, FP8 codes).

B65 H32 N8192 d128 bf16 causal holds 2.18e9 elements per tensor.  Every
element offset of the last head (b = 64, h = 31) lies past 2^31, where 32-bit
indexing would wrap.  Heads are independent, so only the first and the last
head carry the seeded synthetic inputs (Q, K, V, dO ~ N(0, 1) -> bf16,
seed 31); every other head is zero.  The forward and the backward run on
the whole problem.  The two heads are then checked against
oracle.attention.head_backward_sampled: O and LSE of every row, dQ at 32
query rows, dK and dV at 32 key columns, to the bf16 bars of the other
full-size tests."""
import math

import numpy as np
import pytest

from attn_inputs import decode_inputs, dense_inputs
from oracle import attention as A
from oracle import decode as D
from oracle import fp8 as F
from parity_utils import (BF16_O_MAX_ABS, check_bf16, check_bf16_sampled, check_lse, sample_positions, to_dev,
                          to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_09_amd as M
    M.load()
    return M


def test_offsets_past_2_to_31_elements(lib):
    import torch
    B, H, N, d = 65, 32, 8192, 128
    heads = [(0, 0), (B - 1, H - 1)]
    assert B * H * N * d > 2 ** 31 and ((B - 1) * H + H - 1) * N * d > 2 ** 31
    print(f"[case] B{B} H{H} N{N} d{d} causal: allocate", flush=True)
    src = dense_inputs(len(heads), 1, N, d, "bf16", seed=31)
    dev = {}
    for name in ("q", "k", "v", "do"):
        t = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda")
        for i, (b, h) in enumerate(heads):
            t[b, h] = to_dev(src[name][i, 0], "bf16")
        dev[name] = t
    scale = 1 / math.sqrt(d)
    o = torch.empty_like(dev["q"])
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(dev["q"]) for _ in range(3))
    ws = torch.empty(lib.attn_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    print("[case] forward and backward", flush=True)
    lib.attn_fwd(dev["q"], dev["k"], dev["v"], o, lse, scale, True)
    lib.attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], dq, dk, dv, scale, True, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(31)
    for i, (b, h) in enumerate(heads):
        print(f"[case] oracle head b={b} h={h}", flush=True)
        rows, rw = sample_positions(N, 32, rng)
        cols, cw = sample_positions(N, 32, rng)
        q, k, v, do = (src[n][i, 0] for n in ("q", "k", "v", "do"))
        rdq, rdk, rdv, ro, rlse, _ = A.head_backward_sampled(q, k, v, do, scale, True, None, rows, cols)
        label = f"[b={b} h={h}]"
        check_bf16(to_np(o[b, h]), ro, f"O{label}", max_abs_tol=BF16_O_MAX_ABS)
        check_lse(to_np(lse[b, h]), rlse, what=f"LSE{label}")
        check_bf16_sampled(to_np(dq[b, h])[rows], rdq, rw, f"dQ{label}")
        check_bf16_sampled(to_np(dk[b, h])[cols], rdk, cw, f"dK{label}")
        check_bf16_sampled(to_np(dv[b, h])[cols], rdv, cw, f"dV{label}")


def test_packed_offsets_past_2_to_31_elements(lib):
    """Packed sequences past 2^31 elements: 65 causal sequences of 8192 tokens,
    H32 d128, [T, H, d] with T = 532480.  Sequence 0 / head 0 and sequence
    64 / head 31 (offsets past 2^31) carry the seeded inputs, the rest is
    zero; both against head_backward_sampled."""
    import torch
    nseq, L, H, d = 65, 8192, 32, 128
    T = nseq * L
    cu = np.arange(nseq + 1, dtype=np.int32) * L
    picks = [(0, 0), (nseq - 1, H - 1)]
    assert T * H * d > 2 ** 31 and ((nseq - 1) * L * H + H - 1) * d > 2 ** 31
    print(f"[case] packed {nseq} x {L} H{H} d{d} causal: allocate", flush=True)
    src = dense_inputs(len(picks), 1, L, d, "bf16", seed=32)
    dev = {}
    for name in ("q", "k", "v", "do"):
        t = torch.zeros((T, H, d), dtype=torch.bfloat16, device="cuda")
        for i, (s, h) in enumerate(picks):
            t[s * L:(s + 1) * L, h] = to_dev(src[name][i, 0], "bf16")
        dev[name] = t
    scale = 1 / math.sqrt(d)
    cu_d = torch.from_numpy(cu).cuda()
    o = torch.empty_like(dev["q"])
    lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(dev["q"]) for _ in range(3))
    ws = torch.empty(lib.attn_bwd_varlen_workspace_bytes(T, H, d), dtype=torch.uint8, device="cuda")
    print("[case] forward and backward", flush=True)
    lib.attn_fwd_varlen(dev["q"], dev["k"], dev["v"], o, lse, cu_d, L, scale, True)
    lib.attn_bwd_varlen(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], dq, dk, dv, cu_d, L, scale, True, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(32)
    for i, (s, h) in enumerate(picks):
        print(f"[case] oracle sequence {s} head {h}", flush=True)
        rows, rw = sample_positions(L, 32, rng)
        cols, cw = sample_positions(L, 32, rng)
        q, k, v, do = (src[n][i, 0] for n in ("q", "k", "v", "do"))
        rdq, rdk, rdv, ro, rlse, _ = A.head_backward_sampled(q, k, v, do, scale, True, None, rows, cols)
        sl = slice(s * L, (s + 1) * L)
        label = f"[seq {s} head {h}]"
        check_bf16(to_np(o[sl, h]), ro, f"O{label}", max_abs_tol=BF16_O_MAX_ABS)
        check_lse(to_np(lse[h, sl]), rlse, what=f"LSE{label}")
        check_bf16_sampled(to_np(dq[sl, h])[rows], rdq, rw, f"dQ{label}")
        check_bf16_sampled(to_np(dk[sl, h])[cols], rdk, cw, f"dK{label}")
        check_bf16_sampled(to_np(dv[sl, h])[cols], rdv, cw, f"dV{label}")


def test_decode_cache_past_2_to_31_elements(lib):
    """Split-KV decoding with K/V caches past 2^31 elements: B65 H32 H_kv8
    N_kv 32768 d128.  Batch 0 / K/V head 0 and batch 64 / K/V head 7 (and
    their four query heads each) carry the seeded inputs, the rest is zero;
    O and LSE of those query heads against the oracle's definition."""
    import torch
    B, H, Hkv, N, d = 65, 32, 8, 32768, 128
    G = H // Hkv
    picks = [(0, 0), (B - 1, Hkv - 1)]
    assert B * Hkv * N * d > 2 ** 31 and ((B - 1) * Hkv + Hkv - 1) * N * d > 2 ** 31
    print(f"[case] decode B{B} H{H} H_kv{Hkv} N_kv{N} d{d}: allocate", flush=True)
    src = decode_inputs(len(picks), G, 1, N, d, "bf16", seed=33)
    q = torch.zeros((B, H, d), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((B, Hkv, N, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    for i, (b, hk) in enumerate(picks):
        q[b, hk * G:(hk + 1) * G] = to_dev(src["q"][i], "bf16")
        kc[b, hk] = to_dev(src["k"][i, 0], "bf16")
        vc[b, hk] = to_dev(src["v"][i, 0], "bf16")
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(lib.attn_decode_workspace_bytes(B, H, Hkv, N, d), dtype=torch.uint8, device="cuda")
    scale = 1 / math.sqrt(d)
    print("[case] decode", flush=True)
    lib.attn_decode(q, kc, vc, o, lse, scale, None, ws)
    torch.cuda.synchronize()
    ro, rlse = D.decode_forward(src["q"], src["k"], src["v"], scale)
    for i, (b, hk) in enumerate(picks):
        hs = slice(hk * G, (hk + 1) * G)
        label = f"[b={b} kv head {hk}]"
        check_bf16(to_np(o[b, hs]), ro[i], f"O{label}", max_abs_tol=BF16_O_MAX_ABS)
        check_lse(to_np(lse[b, hs]), rlse[i], what=f"LSE{label}")


def test_fp8_past_2_to_31_bytes(lib):
    """The FP8 path with code tensors past 2^31 bytes: B65 H32 N8192 d128,
    causal.  The first and the last head carry the seeded inputs, the rest
    is zero; quantization and the forward run on the whole problem, and the
    two heads' sampled rows are checked against the oracle's row-restricted
    FP8 reference within its bound (the terms of the other FP8 tests)."""
    import torch
    B, H, N, d = 65, 32, 8192, 128
    heads = [(0, 0), (B - 1, H - 1)]
    nb = N // 64
    print(f"[case] fp8 B{B} H{H} N{N} d{d} causal: allocate", flush=True)
    src = dense_inputs(len(heads), 1, N, d, "bf16", seed=34, with_do=False)
    x = {}
    for name in ("q", "k", "v"):
        t = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda")
        for i, (b, h) in enumerate(heads):
            t[b, h] = to_dev(src[name][i, 0], "bf16")
        x[name] = t
    q8, k8 = (torch.empty((B, H, N, d), dtype=torch.uint8, device="cuda") for _ in range(2))
    v8 = torch.empty((B, H, nb, d, 64), dtype=torch.uint8, device="cuda")
    sq, sk = (torch.empty((B, H, nb), dtype=torch.float32, device="cuda") for _ in range(2))
    sv = torch.empty((B, H), dtype=torch.float32, device="cuda")
    lib.attn_quantize_fp8_rows(x["q"], q8, sq)
    lib.attn_quantize_fp8_rows(x["k"], k8, sk)
    lib.attn_quantize_fp8_vt(x["v"], v8, sv)
    del x
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    scale = 1 / math.sqrt(d)
    print("[case] fp8 forward", flush=True)
    lib.attn_fwd_fp8(q8, sq, k8, sk, v8, sv, o, lse, scale, True)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 63, 64, 1000, 4095, 4096, 8000, N - 2, N - 1])
    for i, (b, h) in enumerate(heads):
        print(f"[case] oracle head b={b} h={h}", flush=True)
        q, k, v = (src[n][i:i + 1] for n in ("q", "k", "v"))
        ref = F.fp8_reference_rows(q, k, v, scale, True, rows)
        bound, weighted = F.fp8_output_bound(ref["qd"], ref["kd"], ref["vd"], ref["lse"], scale, True,
                                             p_scale_log2=6, rows=rows)
        a_ = np.abs(ref["qd"][0, 0][rows]) @ np.abs(ref["kd"][0, 0]).T
        a_ = np.where(np.arange(N)[None, :] <= rows[:, None], a_, 0.0)
        delta = 2.0 ** -12 * abs(scale) * a_.max(axis=1)
        got_o, got_lse = to_np(o[b, h])[rows], to_np(lse[b, h])[rows]
        allowed = bound[0, 0] + (2.0 ** -8 + delta[:, None]) * weighted[0, 0] + 2.0 ** -8 * np.abs(ref["o"][0, 0])
        assert np.max(np.abs(got_o - ref["o"][0, 0]) - allowed) <= 0, f"O [b={b} h={h}] outside the FP8 bound"
        assert np.max(np.abs(got_lse - ref["lse"][0, 0]) - (1e-3 + delta)) <= 0, f"LSE [b={b} h={h}]"
