"""GPU parity of attn_decode (one query token per sequence against a KV
cache, split along the cache and merged) with the fp64 oracle's definition
(oracle/decode.py), element by element on every head.

Cases: a one-key cache, ragged cache lengths per sequence including empty
caches (O = 0, LSE = -inf), lengths that are not multiples of the 64-key tile
or of the piece size, multi-head (H_kv = H), grouped and multi-query heads
(G = 64 needs two 32-row query chunks), d = 64 and 128, zero / negative /
large scales, and the full-size shape B=8, H=32, H_kv=8, N_kv=32768, d=128,
which the oracle checks whole (decoding is one matrix-vector product per
head)."""
import math

import numpy as np
import pytest

from attn_inputs import decode_inputs
from oracle import decode as Dc
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


def _inputs(B, H, Hkv, N, d, seed, sigma=1.0):
    x = decode_inputs(B, H, Hkv, N, d, "bf16", seed=seed, sigma=sigma)
    return x["q"], x["k"], x["v"]


def _run(lib, q, k, v, scale, seqlens):
    import torch
    B, H, d = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    o = torch.empty_like(qd)
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    ws = torch.empty(lib.attn_decode_workspace_bytes(B, H, Hkv, N, d), dtype=torch.uint8, device="cuda")
    lib.attn_decode(qd, kd, vd, o, lse, scale, sl, ws)
    torch.cuda.synchronize()
    return to_np(o), to_np(lse)


def _check(o, lse, ref_o, ref_lse):
    check_bf16(o, ref_o, "O", max_abs_tol=BF16_O_MAX_ABS)
    check_lse(lse, ref_lse)
    dead = np.isneginf(ref_lse)
    assert np.all(o[dead] == 0)


CASES = [
    # B, H, Hkv, N, d, seqlens
    (2, 8, 8, 1, 64, None),
    (3, 8, 2, 63, 128, [63, 0, 17]),
    (2, 32, 8, 1000, 128, None),
    (1, 64, 1, 4097, 128, None),
    (4, 16, 4, 5000, 64, [5000, 1, 4999, 2345]),
    (2, 6, 3, 300, 64, [299, 300]),
    (3, 12, 12, 777, 128, [0, 0, 777]),
    (1, 40, 8, 70000, 128, [65537]),
    (1, 8, 1, 1 << 20, 64, [1048000]),  # a 2^20-token cache: 1024 pieces to merge
]


@pytest.mark.parametrize("B,H,Hkv,N,d,seqlens", CASES)
def test_decode_ragged(lib, B, H, Hkv, N, d, seqlens):
    print(f"[case] decode B={B} H={H} Hkv={Hkv} N={N} d={d} seqlens={seqlens}", flush=True)
    q, k, v = _inputs(B, H, Hkv, N, d, seed=N + H)
    scale = 1 / math.sqrt(d)
    o, lse = _run(lib, q, k, v, scale, seqlens)
    ref_o, ref_lse = Dc.decode_forward(q, k, v, scale, seqlens)
    _check(o, lse, ref_o, ref_lse)


@pytest.mark.parametrize("scale", [0.0, -0.3, 0.9])
def test_decode_scale_edge_cases(lib, scale):
    """scale = 0 (uniform average), a negative scale, and sharp scores
    (scale 0.9 with N(0, 2^2) inputs): the pieces' maxima differ widely."""
    q, k, v = _inputs(2, 8, 2, 3000, 128, seed=5, sigma=2.0)
    o, lse = _run(lib, q, k, v, scale, [3000, 1234])
    ref_o, ref_lse = Dc.decode_forward(q, k, v, scale, [3000, 1234])
    _check(o, lse, ref_o, ref_lse)


def test_decode_full_size(lib):
    """B=8, H=32, H_kv=8, N_kv=32768, d=128, N(0,1) bf16, every head."""
    q, k, v = _inputs(8, 32, 8, 32768, 128, seed=0)
    scale = 1 / math.sqrt(128)
    o, lse = _run(lib, q, k, v, scale, None)
    ref_o, ref_lse = Dc.decode_forward(q, k, v, scale)
    _check(o, lse, ref_o, ref_lse)
