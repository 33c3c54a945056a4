"""Shared helpers for the GPU parity tests: device copies of the seeded inputs,
error metrics and the tolerance bar (not a test module).

Tolerances (fixed here, used by every parity test):
  fp32 path:  max |GPU - oracle| <= 1e-5 on O, LSE, dQ, dK, dV.
  bf16 path:  O: max abs <= 2e-2; O, dQ, dK, dV: relative Frobenius error
              <= 1e-2; LSE: max abs <= 1e-3.  The oracle runs in fp64 on the
              identical bf16-rounded inputs.  Rows whose LSE is -inf must be
              -inf on both sides with O exactly zero.
"""
from __future__ import annotations

import numpy as np

F32_MAX_ABS = 1e-5
BF16_O_MAX_ABS = 2e-2
BF16_REL_FRO = 1e-2
LSE_MAX_ABS = 1e-3


def torch_mod():
    import torch
    return torch


def to_dev(x: np.ndarray, dtype: str):
    """float32 numpy (values exact in dtype) -> contiguous device tensor."""
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype != "f32":
        raise ValueError(dtype)
    return t.cuda().contiguous()


def to_np(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_abs(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = float(np.linalg.norm(b))
    num = float(np.linalg.norm(a - b))
    if den == 0.0:
        return num
    return num / den


def check_lse(gpu_lse, ref_lse, tol=LSE_MAX_ABS, what="LSE"):
    g = np.asarray(gpu_lse, np.float64)
    r = np.asarray(ref_lse, np.float64)
    dead_r = np.isneginf(r)
    dead_g = np.isneginf(g)
    assert np.array_equal(dead_r, dead_g), f"{what}: -inf rows differ ({dead_r.sum()} oracle vs {dead_g.sum()} GPU)"
    assert np.all(np.isfinite(g[~dead_g])), f"{what}: non-finite values"
    err = max_abs(g[~dead_r], r[~dead_r])
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"
    return err


def check_bf16(gpu, ref, what, max_abs_tol=None):
    err_fro = rel_fro(gpu, ref)
    err_abs = max_abs(gpu, ref)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    assert err_fro <= BF16_REL_FRO, f"{what}: relative Frobenius error {err_fro:.3e} > {BF16_REL_FRO:.0e}"
    if max_abs_tol is not None:
        assert err_abs <= max_abs_tol, f"{what}: max abs error {err_abs:.3e} > {max_abs_tol:.0e}"
    return err_fro, err_abs


def check_f32(gpu, ref, what, tol=F32_MAX_ABS):
    err = max_abs(gpu, ref)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.0e}"
    return err


def tile_rel_fro_max(gpu, ref, tile=64) -> float:
    """Largest relative Frobenius error over consecutive blocks of `tile` rows
    (a diagnostic beside the whole-head bar: one bad 32-row block can hide in
    a head-wide norm)."""
    a = np.asarray(gpu, np.float64)
    b = np.asarray(ref, np.float64)
    worst = 0.0
    for r0 in range(0, a.shape[0], tile):
        den = float(np.linalg.norm(b[r0:r0 + tile]))
        if den > 0.0:
            worst = max(worst, float(np.linalg.norm(a[r0:r0 + tile] - b[r0:r0 + tile])) / den)
    return worst


def host_workers() -> int:
    """Worker threads for oracle work on the host: the cores this process may
    use, at most 16."""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def map_heads(fn, jobs):
    """Run fn(job) for every job on a thread pool, one BLAS thread per worker
    (numpy's large array operations release the GIL, so the heads run in
    parallel).  Returns the results in job order; the first failure raises."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"):
        with ThreadPoolExecutor(host_workers()) as ex:
            return list(ex.map(fn, jobs))


def sample_positions(n: int, count: int, rng):
    """`count` distinct positions of [0, n): the first two and the last two,
    the rest drawn uniformly by rng; sorted.  Returns (positions, weights):
    a fixed position stands for itself (weight 1), a drawn one for its share
    of the positions not fixed, so weighted sums over the sample estimate
    sums over all n positions without bias."""
    fixed = sorted({0, 1, n - 2, n - 1} & set(range(n)))
    rest = np.setdiff1d(np.arange(n), fixed)
    extra = rng.choice(rest, size=min(len(rest), max(0, count - len(fixed))), replace=False)
    pos = np.concatenate([np.asarray(fixed, np.int64), extra.astype(np.int64)])
    w = np.concatenate([np.ones(len(fixed)), np.full(len(extra), len(rest) / max(1, len(extra)))])
    order = np.argsort(pos)
    return pos[order], w[order]


def check_bf16_sampled(gpu, ref, weights, what):
    """The bf16 relative Frobenius bar on sampled rows: the whole tensor's
    ||gpu - ref|| / ||ref||, estimated from the rows with their sample
    weights (sample_positions).  Returns (estimate, worst single-row relative
    error) -- the latter is a diagnostic: a row that sees only a couple of keys
    can carry a few percent of bf16 rounding on its own without breaking the
    tensor-wide bar."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    w = np.asarray(weights, np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    e2 = np.sum((g - r) ** 2, axis=1)
    r2 = np.sum(r ** 2, axis=1)
    den = float(np.sum(w * r2))
    est = float(np.sqrt(np.sum(w * e2) / den)) if den > 0 else float(np.sqrt(np.sum(w * e2)))
    assert est <= BF16_REL_FRO, f"{what}: estimated relative Frobenius error {est:.3e} > {BF16_REL_FRO:.0e}"
    rows = r2 > 0
    worst = float(np.max(np.sqrt(e2[rows] / r2[rows]))) if np.any(rows) else 0.0
    return est, worst
