"""The C-ABI library loads on the CPU and exports every symbol the header
declares; host-side validation rejects bad arguments before any launch.
CPU only: nothing here launches a kernel."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "miattn.h")
LIB = os.path.join(ROOT, "exact_tiled_attention_09_amd", "libmiattn.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmiattn.so not built")


def _declared():
    with open(HEADER) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(?:int|size_t|const char\*)\s+(\w+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = _declared()
    for need in ("attn_fwd", "attn_bwd", "attn_bwd_workspace_bytes", "attn_fwd_f32", "attn_bwd_f32",
                 "attn_fwd_gqa", "attn_bwd_gqa", "attn_fwd_window", "attn_bwd_window",
                 "attn_fwd_block_sparse", "attn_bwd_block_sparse", "attn_bwd_block_sparse_workspace_bytes",
                 "attn_decode", "attn_decode_workspace_bytes",
                 "attn_quantize_fp8_rows", "attn_quantize_fp8_vt", "attn_fwd_fp8",
                 "attn_fwd_varlen", "attn_bwd_varlen", "attn_bwd_varlen_workspace_bytes",
                 "miattn_status_string"):
        assert need in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"


def test_binding_signatures_cover_the_header():
    from exact_tiled_attention_09_amd import _lib
    assert sorted(_lib.SIGNATURES) == _declared()
    _lib.load()


def _lib():
    from exact_tiled_attention_09_amd import _lib as L
    return L.load()


def test_status_strings_and_version():
    lib = _lib()
    assert lib.miattn_version() >= 100
    assert lib.miattn_status_string(0) == b"ok"
    assert b"invalid" in lib.miattn_status_string(-1)
    assert b"unsupported" in lib.miattn_status_string(-2)


def test_workspace_sizes():
    lib = _lib()
    B, H, N, d = 4, 32, 4096, 128
    rows = B * H * N
    assert lib.attn_bwd_workspace_bytes(B, H, N, d) == (rows * 4 + 255) // 256 * 256
    assert lib.attn_bwd_f32_workspace_bytes(B, H, N, d) == (rows * 4 + 255) // 256 * 256 + rows * d * 4
    assert lib.attn_bwd_workspace_bytes(B, H, N, 96) == 0
    assert lib.attn_bwd_workspace_bytes(0, H, N, d) == 0
    assert lib.attn_bwd_varlen_workspace_bytes(1000, 32, 64) == (32000 * 4 + 255) // 256 * 256


# A fake, aligned, non-null "device" address: validation fails before it is used.
FAKE = ctypes.c_void_p(1 << 20)
NULL = ctypes.c_void_p(0)
MIS = ctypes.c_void_p((1 << 20) + 2)


@pytest.mark.parametrize("case,expect", [
    (dict(q=NULL), -1),
    (dict(o=MIS), -1),
    (dict(B=0), -1),
    (dict(N=-5), -1),
    (dict(scale=float("inf")), -1),
    (dict(scale=float("nan")), -1),
    (dict(d=96), -2),
    (dict(d=256), -2),
])
def test_forward_argument_validation(case, expect):
    lib = _lib()
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=16, d=64, scale=0.125)
    args.update(case)
    st = lib.attn_fwd(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"], args["H"], args["N"],
                      args["d"], args["scale"], 0, NULL)
    assert st == expect


def test_backward_rejects_small_workspace():
    lib = _lib()
    need = lib.attn_bwd_workspace_bytes(1, 2, 64, 64)
    st = lib.attn_bwd(*([FAKE] * 9), 1, 2, 64, 64, 0.125, 1, FAKE, need - 4, NULL)
    assert st == -1
    need32 = lib.attn_bwd_f32_workspace_bytes(1, 2, 64, 64)
    st = lib.attn_bwd_f32(*([FAKE] * 9), 1, 2, 64, 64, 0.125, 1, FAKE, need32 - 4, NULL)
    assert st == -1
    dqp = lambda o, ws: lib.attn_bwd_dq_preprocess(FAKE, FAKE, FAKE, o, *([FAKE] * 3), 1, 2, 64, 64, 0.125, 1,
                                                    FAKE, ws, NULL)
    assert dqp(FAKE, need - 4) == -1        # workspace too small
    assert dqp(NULL, need) == -1            # no O to form D from


def test_varlen_validation():
    lib = _lib()
    base = [FAKE] * 5
    assert lib.attn_fwd_varlen(*base, NULL, 2, 10, 15, 2, 64, 0.1, 1, NULL, NULL) == -1
    assert lib.attn_fwd_varlen(*base, FAKE, 0, 10, 15, 2, 64, 0.1, 1, NULL, NULL) == -1
    assert lib.attn_fwd_varlen(*base, FAKE, 2, 10, 15, 2, 80, 0.1, 1, NULL, NULL) == -2
    assert lib.attn_fwd_varlen(*base, ctypes.c_void_p((1 << 20) + 2), 2, 10, 15, 2, 64, 0.1, 1, NULL, NULL) == -1


def test_grouped_head_validation():
    lib = _lib()
    fwd = lambda H, Hkv, d=64: lib.attn_fwd_gqa(*([FAKE] * 5), 1, H, Hkv, 16, d, 0.125, 1, NULL)
    assert fwd(8, 0) == -1       # no key/value heads
    assert fwd(8, 3) == -1       # 3 does not divide 8
    assert fwd(8, 16) == -1      # more key/value heads than query heads
    assert fwd(0, 1) == -1
    assert fwd(8, 2, d=96) == -2
    need = lib.attn_bwd_workspace_bytes(1, 8, 64, 64)
    bwd = lambda H, Hkv, ws: lib.attn_bwd_gqa(*([FAKE] * 9), 1, H, Hkv, 64, 64, 0.125, 1, FAKE, ws, NULL)
    assert bwd(8, 3, need) == -1
    assert bwd(8, 2, need - 4) == -1
    assert lib.attn_bwd_gqa(*([FAKE] * 8), NULL, 1, 8, 2, 64, 64, 0.125, 1, FAKE, need, NULL) == -1


def test_window_and_block_sparse_validation():
    lib = _lib()
    win = lambda L, R, Hkv=2: lib.attn_fwd_window(*([FAKE] * 5), 1, 8, Hkv, 64, 64, 0.125, 0, L, R, NULL)
    assert win(-2, 0) == -1      # a side below -1
    assert win(4, -5) == -1
    assert win(4, 4, Hkv=3) == -1
    need = lib.attn_bwd_workspace_bytes(1, 8, 64, 64)
    bwin = lambda L, R, ws: lib.attn_bwd_window(*([FAKE] * 9), 1, 8, 2, 64, 64, 0.125, 1, L, R, FAKE, ws, NULL)
    assert bwin(-3, 0, need) == -1
    assert bwin(16, 0, need - 4) == -1
    sp = lambda N, rp, ci, nnz: lib.attn_fwd_block_sparse(*([FAKE] * 5), 1, 8, 2, N, 64, 0.125, 1, rp, ci, nnz, NULL)
    assert sp(131072 + 1, FAKE, FAKE, 4) == -2     # more than 1024 blocks
    assert sp(512, NULL, FAKE, 4) == -1            # no row pointers
    assert sp(512, FAKE, NULL, 4) == -1            # entries but no column indices
    assert sp(512, FAKE, FAKE, -1) == -1
    assert lib.attn_bwd_block_sparse_workspace_bytes(1, 8, 2, 131072 + 1, 64, 4) == 0
    assert lib.attn_bwd_block_sparse_workspace_bytes(1, 8, 3, 512, 64, 4) == 0
    assert lib.attn_bwd_block_sparse_workspace_bytes(1, 8, 2, 512, 64, -1) == 0
    nb = 4  # N = 512
    ws = lib.attn_bwd_block_sparse_workspace_bytes(1, 8, 2, 512, 64, 4)
    assert ws >= lib.attn_bwd_workspace_bytes(1, 8, 512, 64) + nb * nb
    bsp = lambda wsb: lib.attn_bwd_block_sparse(*([FAKE] * 9), 1, 8, 2, 512, 64, 0.125, 1, FAKE, FAKE, 4, FAKE,
                                                wsb, NULL)
    assert bsp(ws - 1) == -1
    # A list longer than nb * nb entries (repeats) plans like nb * nb entries;
    # nnz near INT_MAX must not overflow the plan.
    full = lib.attn_bwd_block_sparse_workspace_bytes(1, 8, 2, 512, 64, nb * nb)
    assert lib.attn_bwd_block_sparse_workspace_bytes(1, 8, 2, 512, 64, 1000) == full
    assert lib.attn_bwd_block_sparse_workspace_bytes(1, 8, 2, 512, 64, 2**31 - 1) == full
    big = lib.attn_bwd_block_sparse_workspace_bytes(1, 8, 2, 131072, 64, 2**31 - 1)
    assert 0 < big < 1 << 40


def test_decode_validation():
    lib = _lib()
    need = lib.attn_decode_workspace_bytes(2, 8, 2, 1000, 128)
    assert need > 0
    assert lib.attn_decode_workspace_bytes(2, 8, 3, 1000, 128) == 0   # 3 does not divide 8
    assert lib.attn_decode_workspace_bytes(2, 8, 2, 0, 128) == 0      # empty cache dimension
    dec = lambda H, Hkv, N, d, ws, sl=NULL: lib.attn_decode(*([FAKE] * 5), 2, H, Hkv, N, d, 0.1, sl, FAKE, ws, NULL)
    assert dec(8, 2, 1000, 128, need - 1) == -1
    assert dec(8, 3, 1000, 128, need) == -1
    assert dec(8, 2, 1000, 96, need) == -2
    assert dec(8, 2, 1000, 128, need, ctypes.c_void_p((1 << 20) + 2)) == -1   # misaligned lengths


def test_fp8_validation():
    lib = _lib()
    assert lib.attn_quantize_fp8_rows(FAKE, FAKE, FAKE, 1, 2, 64, 64, NULL) == -2     # head dim 64
    assert lib.attn_quantize_fp8_vt(FAKE, FAKE, NULL, 1, 2, 64, 128, NULL) == -1      # no scales
    fwd = lambda Hkv, d: lib.attn_fwd_fp8(*([FAKE] * 8), 1, 8, Hkv, 64, d, 0.1, 1, NULL)
    assert fwd(3, 128) == -1
    assert fwd(2, 64) == -2
    assert lib.attn_fwd_fp8(FAKE, NULL, *([FAKE] * 6), 1, 8, 2, 64, 128, 0.1, 1, NULL) == -1
