"""Tensors past 2^31 elements.

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

from attn_inputs import dense_inputs
from oracle import attention as A
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
