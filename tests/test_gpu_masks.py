"""GPU parity of the sliding-window and block-sparse entry points
(attn_fwd_window / attn_bwd_window, attn_fwd_block_sparse /
attn_bwd_block_sparse) against the fp64 oracle, element by element.

Small and ragged sizes cover windows that are one-sided, two-sided, only the
diagonal, wider than the sequence, and combined with the causal mask;
block lists that are tridiagonal, global + local, strided with unsorted and
repeated entries, with empty query blocks (rows without any key) and with
out-of-range entries (ignored).  Grouped key/value heads run through the same
calls.  At full size: a sliding window of 4096 keys over N = 16384 and a
global + local + strided block list over N = 16384, both with 32 query heads
on 8 key/value heads: every output finite, and one key/value group against
the oracle (O and LSE of its query heads whole, dQ at sampled query rows, dK
and dV at sampled key columns).  At the block list's limit: N = 131072 with a
query block listing all 1024 key blocks, on sampled rows and columns."""
import math
import time

import numpy as np
import pytest

from attn_inputs import dense_inputs
from oracle import attention as A
from parity_utils import BF16_O_MAX_ABS, check_bf16, check_lse, to_dev, to_np

pytestmark = pytest.mark.gpu

BLOCK = 128


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


def _alloc(inp):
    import torch
    q, k, v, do = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    return q, k, v, do, torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device="cuda")


def _run_window(lib, inp, scale, causal, left, right):
    import torch
    q, k, v, do, o, lse = _alloc(inp)
    B, H, N, d = q.shape
    lib.attn_fwd_window(q, k, v, o, lse, scale, causal, left, right)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(lib.attn_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    lib.attn_bwd_window(q, k, v, o, lse, do, dq, dk, dv, scale, causal, left, right, ws)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def _run_sparse(lib, inp, scale, causal, row_ptr, col_idx):
    import torch
    q, k, v, do, o, lse = _alloc(inp)
    B, H, N, d = q.shape
    rp = torch.from_numpy(np.asarray(row_ptr, np.int32)).cuda()
    ci = torch.from_numpy(np.asarray(col_idx, np.int32)).cuda()
    lib.attn_fwd_block_sparse(q, k, v, o, lse, scale, causal, rp, ci)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(lib.attn_bwd_block_sparse_workspace_bytes(B, H, k.shape[1], N, d, int(ci.numel())),
                     dtype=torch.uint8, device="cuda")
    lib.attn_bwd_block_sparse(q, k, v, o, lse, do, dq, dk, dv, scale, causal, rp, ci, ws)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def _check(out, ref, heads=None, groups=None):
    sel_h = (lambda x: x) if heads is None else (lambda x: x[heads])
    sel_g = (lambda x: x) if groups is None else (lambda x: x[groups])
    check_bf16(sel_h(to_np(out["o"])), sel_h(ref["o"]), "O", max_abs_tol=BF16_O_MAX_ABS)
    check_lse(sel_h(to_np(out["lse"])), sel_h(ref["lse"]))
    check_bf16(sel_h(to_np(out["dq"])), sel_h(ref["dq"]), "dq")
    for name in ("dk", "dv"):
        fro, mab = check_bf16(sel_g(to_np(out[name])), sel_g(ref[name]), name)
        _say(f"  {name}: rel-fro {fro:.2e} max-abs {mab:.2e}")


WINDOWS = [
    (64, 0, False),     # sliding window over the past (left side only, diagonal included)
    (100, 37, False),   # two-sided
    (0, 0, False),      # the diagonal only
    (31, 65, False),
    (5, -1, False),     # unbounded right side
    (-1, 20, False),    # unbounded left side
    (50, -1, True),     # causal sliding window
    (1000, 1000, False),  # wider than the sequence: plain attention
    (-1, 7, True),      # causal overrides the right side: plain causal
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [200, 333])
@pytest.mark.parametrize("left,right,causal", WINDOWS)
def test_window_ragged(lib, left, right, causal, N, d):
    Hkv = 2 if (N + d) % 2 else 4
    print(f"[case] window ({left},{right}) causal={causal} N={N} d={d} Hkv={Hkv}", flush=True)
    inp = dense_inputs(2, 4, N, d, "bf16", seed=N * 3 + d + left, kv_heads=Hkv)
    scale = 1 / math.sqrt(d)
    out = _run_window(lib, inp, scale, causal, left, right)
    ref = A.gqa_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal, window=(left, right))
    _check(out, ref)


def test_window_matches_plain_entry_points_when_unrestricted(lib):
    """An unbounded window is attn_fwd_gqa / attn_bwd_gqa, bit for bit."""
    import torch
    inp = dense_inputs(1, 4, 300, 128, "bf16", seed=3, kv_heads=2)
    out = _run_window(lib, inp, 0.09, True, -1, -1)
    q, k, v, do, o, lse = _alloc(inp)
    lib.attn_fwd_gqa(q, k, v, o, lse, 0.09, True)
    g = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    ws = torch.empty(lib.attn_bwd_workspace_bytes(1, 4, 300, 128), dtype=torch.uint8, device="cuda")
    lib.attn_bwd_gqa(q, k, v, o, lse, do, *g, 0.09, True, ws)
    torch.cuda.synchronize()
    for name, t in (("o", o), ("lse", lse), ("dq", g[0]), ("dk", g[1]), ("dv", g[2])):
        assert torch.equal(out[name], t), name


def _csr(rows):
    row_ptr = np.zeros(len(rows) + 1, np.int32)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    col_idx = np.array([c for r in rows for c in r], np.int32)
    return row_ptr, col_idx


def _patterns(nb):
    tri = [[c for c in (r - 1, r, r + 1) if 0 <= c < nb] for r in range(nb)]
    glob = [sorted({0, r, max(r - 1, 0)}) for r in range(nb)]
    strided = [[(r + 2) % nb, r, r, (r + 3) % nb][::-1] for r in range(nb)]  # unsorted, repeated
    holes = [[] if r % 2 else [r, (r + 1) % nb] for r in range(nb)]        # empty query blocks
    full = [list(range(nb)) for _ in range(nb)]
    return {"tridiagonal": tri, "global+local": glob, "strided": strided, "empty rows": holes, "all": full}


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [300, 640])
@pytest.mark.parametrize("pattern", ["tridiagonal", "global+local", "strided", "empty rows", "all"])
def test_block_sparse_ragged(lib, pattern, N, d, causal):
    nb = -(-N // BLOCK)
    Hkv = 4 if d == 64 else 2
    print(f"[case] blocks {pattern} causal={causal} N={N} d={d} Hkv={Hkv}", flush=True)
    rp, ci = _csr(_patterns(nb)[pattern])
    inp = dense_inputs(2, 4, N, d, "bf16", seed=N + d + len(pattern), kv_heads=Hkv)
    scale = 1 / math.sqrt(d)
    out = _run_sparse(lib, inp, scale, causal, rp, ci)
    ref = A.gqa_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal, blocks=(rp, ci, BLOCK))
    _check(out, ref)
    dead = np.isneginf(ref["lse"])
    if dead.any():
        assert np.all(np.isneginf(to_np(out["lse"])[dead]))
        assert np.all(to_np(out["o"])[dead] == 0) and np.all(to_np(out["dq"])[dead] == 0)


@pytest.mark.parametrize("N", [1, 17, 127, 128, 129])
@pytest.mark.parametrize("kind", ["window(0,0)", "window(16,5)", "causal window(3)", "blocks all",
                                  "blocks empty rows"])
def test_masked_short_sequences(lib, kind, N):
    """Single and partial tiles: one token, less than a tile, and lengths
    around the 128-token block (one block ragged, one full, a second block of
    one token)."""
    d = 64
    print(f"[case] short {kind} N={N}", flush=True)
    inp = dense_inputs(1, 4, N, d, "bf16", seed=N * 11 + len(kind), kv_heads=2)
    scale = 0.125
    if kind.startswith("blocks"):
        nb = -(-N // BLOCK)
        rp, ci = _csr(_patterns(nb)["all" if kind == "blocks all" else "empty rows"])
        causal = kind == "blocks all"
        out = _run_sparse(lib, inp, scale, causal, rp, ci)
        ref = A.gqa_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal, blocks=(rp, ci, BLOCK))
    else:
        left, right, causal = {"window(0,0)": (0, 0, False), "window(16,5)": (16, 5, False),
                               "causal window(3)": (3, -1, True)}[kind]
        out = _run_window(lib, inp, scale, causal, left, right)
        ref = A.gqa_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal, window=(left, right))
    _check(out, ref)


def test_block_sparse_ignores_out_of_range_entries(lib):
    """Entries outside [0, nb) are skipped: the result is that of the list
    without them."""
    N, nb = 500, 4
    rows = [[0, 7], [-1, 1, 0], [2, 1000], [3, 2, -5]]
    clean = [[c for c in r if 0 <= c < nb] for r in rows]
    rp, ci = _csr(rows)
    rpc, cic = _csr(clean)
    inp = dense_inputs(1, 2, N, 64, "bf16", seed=77)
    out = _run_sparse(lib, inp, 0.125, False, rp, ci)
    ref = A.gqa_backward(inp["q"], inp["k"], inp["v"], inp["do"], 0.125, False, blocks=(rpc, cic, BLOCK))
    _check(out, ref)


def _check_group_sampled(out, inp, scale, causal, b, j, G, seed, **mask):
    """Key/value group j of batch b: O and LSE of its G query heads whole; dQ
    at sampled query rows; dK and dV at sampled key columns, summed over the
    group (head_backward_sampled evaluates exactly those outputs)."""
    N = inp["q"].shape[2]
    rng = np.random.default_rng(seed)
    rows = np.sort(np.concatenate([[0, 1, N - 1], rng.choice(N, 45, replace=False)]))
    cols = np.sort(np.concatenate([[0, 1, N - 1], rng.choice(N, 45, replace=False)]))
    dk_sum = np.zeros((len(cols), inp["k"].shape[-1]))
    dv_sum = np.zeros_like(dk_sum)
    for h in range(j * G, (j + 1) * G):
        _say(f"oracle head {h} (group {j}), sampled")
        dq, dk, dv, o, lse, _ = A.head_backward_sampled(inp["q"][b, h], inp["k"][b, j], inp["v"][b, j],
                                                        inp["do"][b, h], scale, causal, None, rows, cols, **mask)
        check_bf16(to_np(out["o"][b, h]), o, f"O[{b},{h}]", max_abs_tol=BF16_O_MAX_ABS)
        check_lse(to_np(out["lse"][b, h]), lse)
        check_bf16(to_np(out["dq"][b, h])[rows], dq, f"dq[{b},{h}] rows")
        dk_sum += dk
        dv_sum += dv
    fro, mab = check_bf16(to_np(out["dk"][b, j])[cols], dk_sum, f"dk[{b},{j}] cols")
    _say(f"  dk: rel-fro {fro:.2e} max-abs {mab:.2e}")
    fro, mab = check_bf16(to_np(out["dv"][b, j])[cols], dv_sum, f"dv[{b},{j}] cols")
    _say(f"  dv: rel-fro {fro:.2e} max-abs {mab:.2e}")


def test_window_full_size_sliding_4096(lib):
    """B=1, H=32, H_kv=8, N=16384, d=128, causal sliding window of 4096 keys
    (window (4095, 0)), N(0,1) bf16 inputs, seed 0."""
    import torch
    _say("window full size: generate")
    B, H, Hkv, N, d = 1, 32, 8, 16384, 128
    inp = dense_inputs(B, H, N, d, "bf16", seed=0, kv_heads=Hkv)
    scale = 1 / math.sqrt(d)
    out = _run_window(lib, inp, scale, True, 4095, 0)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert bool(torch.isfinite(out[name].float()).all()), f"non-finite {name}"
    _check_group_sampled(out, inp, scale, True, 0, 5, H // Hkv, seed=1, window=(4095, 0))


def test_block_sparse_full_size(lib):
    """B=1, H=32, H_kv=8, N=16384, d=128, non-causal; query block r lists
    block 0 (global), r-1, r, r+1 (local) and every 16th block (strided)."""
    import torch
    _say("block-sparse full size: generate")
    B, H, Hkv, N, d = 1, 32, 8, 16384, 128
    nb = N // BLOCK
    rows = [sorted({0} | {c for c in (r - 1, r, r + 1) if 0 <= c < nb} | set(range(0, nb, 16))) for r in range(nb)]
    rp, ci = _csr(rows)
    inp = dense_inputs(B, H, N, d, "bf16", seed=0, kv_heads=Hkv)
    scale = 1 / math.sqrt(d)
    out = _run_sparse(lib, inp, scale, False, rp, ci)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert bool(torch.isfinite(out[name].float()).all()), f"non-finite {name}"
    _check_group_sampled(out, inp, scale, False, 0, 6, H // Hkv, seed=2, blocks=(rp, ci, BLOCK))


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_cut_key_blocks(lib, causal):
    """N = 2048 (16 blocks), block 0 global plus a local band: block 0 is
    listed by all 16 query blocks, about four times the average, so the
    key-tile pass cuts it into chunks whose partial sums are added in a fixed
    order.  Whole comparison with the oracle, and a second run bit for bit
    equal to the first."""
    import torch
    nb = 16
    rows = [sorted({0} | {c for c in (r - 1, r, r + 1) if 0 <= c < nb}) for r in range(nb)]
    rp, ci = _csr(rows)
    inp = dense_inputs(1, 4, 2048, 128, "bf16", seed=31, kv_heads=2)
    scale = 1 / math.sqrt(128)
    out = _run_sparse(lib, inp, scale, causal, rp, ci)
    out2 = _run_sparse(lib, inp, scale, causal, rp, ci)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(out[name], out2[name]), name
    ref = A.gqa_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal, blocks=(rp, ci, BLOCK))
    _check(out, ref)


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_longest_lists(lib, causal):
    """The largest block list the entry points take: N = 131072 (1024 blocks
    of 128), B1 H2 on one K/V head, d = 64.  Query block r lists r-1, r, r+1
    and every 128th block (block 0 included); the last query block lists all
    1024, the longest list there can be.  O, LSE and dQ at sampled rows (the
    first and last rows of the sequence and of the longest list's block among
    them) and dK, dV at key columns of blocks that only their neighbours and
    the last query block list, summed over the two query heads, against the
    oracle's row-sparse sampled backward."""
    _say(f"block-sparse longest lists causal={causal}: generate")
    B, H, Hkv, N, d = 1, 2, 1, 131072, 64
    nb = N // BLOCK
    strided = set(range(0, nb, 128))
    rows_ = [sorted({c for c in (r - 1, r, r + 1) if 0 <= c < nb} | strided) for r in range(nb - 1)]
    rows_.append(list(range(nb)))
    rp, ci = _csr(rows_)
    inp = dense_inputs(B, H, N, d, "bf16", seed=41, kv_heads=Hkv)
    scale = 1 / math.sqrt(d)
    out = _run_sparse(lib, inp, scale, causal, rp, ci)
    rng = np.random.default_rng(41)
    rows = np.sort(np.concatenate([[0, 1, 500 * BLOCK + 5, (nb - 1) * BLOCK, N - 2, N - 1],
                                   rng.choice(N, 10, replace=False)]))
    cols = np.array([5 * BLOCK + 7, 300 * BLOCK + 64, 1000 * BLOCK + 127, (nb - 1) * BLOCK, N - 1])
    dk_sum = np.zeros((len(cols), d))
    dv_sum = np.zeros_like(dk_sum)
    for h in range(H):
        _say(f"oracle head {h}, row-sparse sampled")
        dq, dk, dv, o, lse = A.head_backward_sampled_sparse(inp["q"][0, h], inp["k"][0, 0], inp["v"][0, 0],
                                                            inp["do"][0, h], scale, causal, None, rows, cols,
                                                            blocks=(rp, ci, BLOCK))
        check_bf16(to_np(out["o"][0, h])[rows], o, f"O[{h}] rows", max_abs_tol=BF16_O_MAX_ABS)
        check_lse(to_np(out["lse"][0, h])[rows], lse)
        check_bf16(to_np(out["dq"][0, h])[rows], dq, f"dq[{h}] rows")
        dk_sum += dk
        dv_sum += dv
    check_bf16(to_np(out["dk"][0, 0])[cols], dk_sum, "dk cols")
    check_bf16(to_np(out["dv"][0, 0])[cols], dv_sum, "dv cols")


def test_window_long_sequence(lib):
    """A causal window of 128 keys over N = 131072, B1 H2 on one K/V head,
    d = 64: O, LSE and dQ at sampled rows and dK, dV at sampled key columns
    (summed over the two query heads) against the oracle's row-sparse
    sampled backward."""
    _say("window over N = 131072: generate")
    B, H, Hkv, N, d = 1, 2, 1, 131072, 64
    inp = dense_inputs(B, H, N, d, "bf16", seed=43, kv_heads=Hkv)
    scale = 1 / math.sqrt(d)
    out = _run_window(lib, inp, scale, True, 127, 0)
    rng = np.random.default_rng(43)
    rows = np.sort(np.concatenate([[0, 1, 127, 128, N - 2, N - 1], rng.choice(N, 10, replace=False)]))
    cols = np.sort(np.concatenate([[0, 1, N - 129, N - 1], rng.choice(N, 6, replace=False)]))
    dk_sum = np.zeros((len(cols), d))
    dv_sum = np.zeros_like(dk_sum)
    for h in range(H):
        _say(f"oracle head {h}, row-sparse sampled")
        dq, dk, dv, o, lse = A.head_backward_sampled_sparse(inp["q"][0, h], inp["k"][0, 0], inp["v"][0, 0],
                                                            inp["do"][0, h], scale, True, None, rows, cols,
                                                            window=(127, 0))
        check_bf16(to_np(out["o"][0, h])[rows], o, f"O[{h}] rows", max_abs_tol=BF16_O_MAX_ABS)
        check_lse(to_np(out["lse"][0, h])[rows], lse)
        check_bf16(to_np(out["dq"][0, h])[rows], dq, f"dq[{h}] rows")
        dk_sum += dk
        dv_sum += dv
    check_bf16(to_np(out["dk"][0, 0])[cols], dk_sum, "dk cols")
    check_bf16(to_np(out["dv"][0, 0])[cols], dv_sum, "dv cols")
