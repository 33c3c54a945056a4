"""The Python binding refuses tensors whose shape or dtype does not match the
problem, before anything reaches the library (the C ABI sees raw pointers,
so such a tensor would make a kernel read or write past its buffer).  Host
logic only: CPU tensors, no library call."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import exact_tiled_attention_09_amd as M  # noqa: E402

BF, F32 = torch.bfloat16, torch.float32


def _dense(B=1, H=2, N=64, d=64, dtype=BF):
    return [torch.zeros((B, H, N, d), dtype=dtype) for _ in range(4)] + [torch.zeros((B, H, N), dtype=F32)]


def test_dense_shape_and_dtype():
    q, k, v, o, lse = _dense()
    with pytest.raises(ValueError, match="k has shape"):
        M.attn_fwd(q, k[:, :, :32], v, o, lse, 0.125, True)
    with pytest.raises(ValueError, match="lse has shape"):
        M.attn_fwd(q, k, v, o, lse[:, :1], 0.125, True)
    with pytest.raises(ValueError, match="v is torch.float32"):
        M.attn_fwd(q, k, v.float(), o, lse, 0.125, True)
    with pytest.raises(ValueError, match="lse is torch.bfloat16"):
        M.attn_fwd(q, k, v, o, lse.to(BF), 0.125, True)
    ws = torch.zeros(1024, dtype=torch.uint8)
    with pytest.raises(ValueError, match="dq has shape"):
        M.attn_bwd(q, k, v, o, lse, q, q[:, :1], k, v, 0.125, True, ws)
    with pytest.raises(ValueError, match="dk has shape"):
        M.attn_bwd_dkdv(q, k, v, lse, q, k[:1, :1], v, 0.125, True, ws)
    fq, fk, fv, fo, flse = _dense(dtype=F32)
    with pytest.raises(ValueError, match="q is torch.bfloat16"):
        M.attn_fwd_f32(q, fk, fv, fo, flse, 0.125, False)


def test_grouped_and_masked_shapes():
    q = torch.zeros((1, 8, 256, 64), dtype=BF)
    k = torch.zeros((1, 2, 256, 64), dtype=BF)
    o = torch.zeros_like(q)
    lse = torch.zeros((1, 8, 256), dtype=F32)
    with pytest.raises(ValueError, match="v has shape"):
        M.attn_fwd_gqa(q, k, q, o, lse, 0.125, True)              # V with the query heads
    with pytest.raises(ValueError, match="o has shape"):
        M.attn_fwd_window(q, k, k, o[:, :2], lse, 0.125, False, 16, 0)
    rp = torch.zeros(3, dtype=torch.int32)                         # N = 256: two query blocks
    ci = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="row_ptr has shape"):
        M.attn_fwd_block_sparse(q, k, k, o, lse, 0.125, False, rp[:2], ci)
    with pytest.raises(ValueError, match="col_idx is torch.int64"):
        M.attn_fwd_block_sparse(q, k, k, o, lse, 0.125, False, rp, ci.long())


def test_decode_fp8_and_packed_shapes():
    q = torch.zeros((2, 8, 128), dtype=BF)
    kc = torch.zeros((2, 2, 300, 128), dtype=BF)
    lse = torch.zeros((2, 8), dtype=F32)
    ws = torch.zeros(1024, dtype=torch.uint8)
    with pytest.raises(ValueError, match="v_cache has shape"):
        M.attn_decode(q, kc, kc[:, :, :100], q, lse, 0.1, None, ws)
    with pytest.raises(ValueError, match="cache_seqlens is torch.int64"):
        M.attn_decode(q, kc, kc, q, lse, 0.1, torch.zeros(2, dtype=torch.int64), ws)

    x = torch.zeros((1, 2, 130, 128), dtype=BF)
    with pytest.raises(ValueError, match="scales has shape"):
        M.attn_quantize_fp8_rows(x, torch.zeros(x.shape, dtype=torch.uint8), torch.zeros((1, 2, 2), dtype=F32))
    with pytest.raises(ValueError, match="v8t has shape"):
        M.attn_quantize_fp8_vt(x, torch.zeros((1, 2, 3, 128, 32), dtype=torch.uint8), torch.zeros((1, 2), dtype=F32))

    T, H, d = 100, 2, 64
    pq = torch.zeros((T, H, d), dtype=BF)
    plse = torch.zeros((H, T), dtype=F32)
    cu = torch.tensor([0, 40, 100], dtype=torch.int32)
    with pytest.raises(ValueError, match="lse has shape"):
        M.attn_fwd_varlen(pq, pq, pq, pq, plse.t(), cu, 60, 0.125, True)
    with pytest.raises(ValueError, match="key_valid has shape"):
        M.attn_fwd_varlen(pq, pq, pq, pq, plse, cu, 60, 0.125, True, key_valid=torch.ones(99, dtype=torch.uint8))
    with pytest.raises(ValueError, match="cu_seqlens is torch.int64"):
        M.attn_fwd_varlen(pq, pq, pq, pq, plse, cu.long(), 60, 0.125, True)


def test_host_cu_seqlens_check():
    """check_cu_seqlens refuses offsets the kernels would misread: not
    starting at 0, decreasing, not ending at total_tokens, a sequence longer
    than max_seqlen."""
    from exact_tiled_attention_09_amd import check_cu_seqlens
    check_cu_seqlens([0, 5, 5, 12], 12, 7)
    check_cu_seqlens(np.array([0, 64], np.int32), 64, 64)
    for cu, T, m in (([1, 5, 12], 12, 7), ([0, 6, 5, 12], 12, 7), ([0, 5, 11], 12, 7), ([0, 5, 13], 13, 7),
                     ([0], 0, 1)):
        with pytest.raises(ValueError):
            check_cu_seqlens(cu, T, m)
