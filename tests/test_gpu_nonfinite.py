"""Non-finite inputs are valid inputs: they propagate and nothing faults.

A query row of Q holding a NaN, and another holding a +inf, make that row's
scores NaN / +-inf.  Softmax of such a row is undefined, and the forward
reports it as NaN in that row's O and LSE; the rows are independent in the
forward, so every other row still matches the oracle (run on the same inputs
with the two rows zeroed).  The backward runs to completion and dQ of the
clean rows (which does not involve the bad rows' queries) still matches the
oracle.  dK and dV take the bad rows' Q and scores into matrix products in
which masked pairs are exact zeros, and 0 * Inf and 0 * NaN are NaN, so the
NaN reaches the keys that share a backward tile with a bad row even where the
causal mask hides the pair; keys more than 128 positions (the largest tile)
after the last bad row are untouched and match the oracle."""
import math

import numpy as np
import pytest

from attn_inputs import dense_inputs
from oracle import attention as A
from parity_utils import BF16_O_MAX_ABS, check_bf16, check_f32, check_lse, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_09_amd as M
    M.load()
    return M


def _run(lib, inp, q_bad, scale, causal, dtype):
    import torch
    q = to_dev(q_bad, dtype)
    k, v, do = (to_dev(inp[n], dtype) for n in ("k", "v", "do"))
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    (lib.attn_fwd if dtype == "bf16" else lib.attn_fwd_f32)(q, k, v, o, lse, scale, causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    wsb = lib.attn_bwd_workspace_bytes if dtype == "bf16" else lib.attn_bwd_f32_workspace_bytes
    ws = torch.empty(wsb(B, H, N, d), dtype=torch.uint8, device="cuda")
    (lib.attn_bwd if dtype == "bf16" else lib.attn_bwd_f32)(q, k, v, o, lse, do, dq, dk, dv, scale, causal, ws)
    torch.cuda.synchronize()
    return {n: to_np(t) for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_nan_and_inf_query_rows(lib, causal, dtype):
    N, d = 512, 128
    print(f"[case] non-finite Q rows, causal={causal} dtype={dtype}", flush=True)
    inp = dense_inputs(1, 2, N, d, dtype, seed=31)
    scale = 1 / math.sqrt(d)
    bad_rows = (70, 201)
    q_bad = inp["q"].copy()
    q_bad[0, 1, bad_rows[0], 5] = np.nan
    q_bad[0, 1, bad_rows[1], 9] = np.inf
    out = _run(lib, inp, q_bad, scale, causal, dtype)

    # the two rows: NaN in O (every feature) and in LSE
    for r in bad_rows:
        assert np.all(np.isnan(out["o"][0, 1, r])), f"O row {r} not NaN"
        assert np.isnan(out["lse"][0, 1, r]), f"LSE row {r} not NaN"
    # every other row: finite and equal to the oracle on clean inputs
    q_clean = inp["q"].copy()
    q_clean[0, 1, list(bad_rows)] = 0.0
    ref = A.backward(q_clean, inp["k"], inp["v"], inp["do"], scale, causal)
    keep = np.ones(N, bool)
    keep[list(bad_rows)] = False
    chk = check_bf16 if dtype == "bf16" else check_f32
    for h in range(2):
        rows = keep if h == 1 else np.ones(N, bool)
        if dtype == "bf16":
            check_bf16(out["o"][0, h][rows], ref["o"][0, h][rows], f"O[{h}]", max_abs_tol=BF16_O_MAX_ABS)
        else:
            check_f32(out["o"][0, h][rows], ref["o"][0, h][rows], f"O[{h}]")
        check_lse(out["lse"][0, h][rows], ref["lse"][0, h][rows], tol=1e-3 if dtype == "bf16" else 1e-5)
        chk(out["dq"][0, h][rows], ref["dq"][0, h][rows], f"dQ[{h}] clean rows")
    # head 0 has no bad row: its whole backward is clean
    for g in ("dk", "dv"):
        chk(out[g][0, 0], ref[g][0, 0], f"{g}[0]")
    # head 1: the bad rows reach dK, dV of the keys they see
    if causal:
        after = np.arange(N) > max(bad_rows) + 128
        for g in ("dk", "dv"):
            chk(out[g][0, 1][after], ref[g][0, 1][after], f"{g}[1] keys past the bad rows' tiles")
        assert np.all(np.isnan(out["dv"][0, 1][: bad_rows[0] + 1]).any(axis=1))
    else:
        assert np.all(np.isnan(out["dv"][0, 1]).any(axis=1))
