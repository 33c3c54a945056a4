"""Host-side logic of bench.py, CPU only: the FLOP accounting of the masked
workloads counts exactly the (query, key) pairs the oracle's mask keeps, and
the block patterns are valid CSR lists."""
import math

import numpy as np
import pytest

import bench
from oracle import attention as A


def _oracle_pairs(cfg):
    N = cfg["N"]
    mask = bench.oracle_mask(cfg)
    vis = A.visible_mask(np.arange(N), N, cfg["causal"], None, mask.get("window"), mask.get("blocks"))
    return int(vis.sum())


@pytest.mark.parametrize("cfg", [
    dict(N=300, causal=True, window=(63, 0)),
    dict(N=300, causal=False, window=(10, 25)),
    dict(N=300, causal=False, window=(-1, 7)),
    dict(N=256, causal=True),
    dict(N=256, causal=False),
    dict(N=640, causal=False, blocks="global+local+strided16"),
    dict(N=2048 + 37, causal=True, blocks="global+local+strided16"),
])
def test_visible_pairs_match_the_oracle_mask(cfg):
    assert bench.visible_pairs(cfg) == _oracle_pairs(cfg)


def test_flop_accounting():
    dense = dict(B=2, H=3, N=128, d=64, causal=False)
    f, b = bench.workload_flops(dense)
    assert f == 4.0 * 2 * 3 * 128 * 128 * 64 and b == 2.5 * f
    win = dict(B=1, H=2, N=300, d=64, causal=True, window=(63, 0))
    f, b = bench.workload_flops(win)
    assert f == 4.0 * 1 * 2 * 64 * _oracle_pairs(win) and b == 2.5 * f


def test_bench_workloads_are_well_formed():
    for name, cfg in bench.WORKLOADS.items():
        if "blocks" in cfg:
            rp, ci, blk = bench.oracle_mask(cfg)["blocks"]
            nb = -(-cfg["N"] // blk)
            assert len(rp) == nb + 1 and rp[0] == 0 and rp[-1] == len(ci)
            assert np.all(np.diff(rp) >= 0) and ci.min() >= 0 and ci.max() < nb
        if "Hkv" in cfg:
            assert cfg["H"] % cfg["Hkv"] == 0
    assert bench.DEFAULT in bench.WORKLOADS
    assert set(bench.DECODE_WORKLOADS).isdisjoint(bench.WORKLOADS)


def test_byte_accounting_and_roofline_bound():
    """Algorithmic bytes per kernel, and the bound taken from arithmetic
    intensity: the benchmark shape's kernels are MFMA-bound, the D pre-pass
    and the short-sequence forward are HBM-bound."""
    by = bench.kernel_bytes(4, 32, 32, 4096, 128)
    e, r = 4 * 32 * 4096 * 128 * 2, 4 * 32 * 4096 * 4
    assert by["fwd"] == 4 * e + r and by["prep"] == 2 * e + r
    assert by["dq"] == 6 * e + 2 * r and by["dkdv"] == 6 * e + 2 * r and by["bwd"] == 8 * e + r
    g = bench.kernel_bytes(1, 8, 2, 100, 64)                  # grouped heads read 1/4 of the K/V bytes
    assert g["fwd"] == 2 * (8 * 100 * 64 * 2) + 2 * (2 * 100 * 64 * 2) + 8 * 100 * 4
    f, _ = bench.flops(4, 32, 4096, 128, True)
    big = bench.roofline_entry("k", 1.0, 2.0 * f, by["dkdv"], None)
    assert big["bound"] == "mfma" and big["unit"] == "TFLOP/s"
    assert math.isclose(big["achieved"], round(2.0 * f / 1e-3 / 1e12, 2))
    prep = bench.roofline_entry("p", 0.05, 2.0 * 4 * 32 * 4096 * 128, by["prep"], None)
    assert prep["bound"] == "hbm" and prep["unit"] == "GB/s" and prep["peak"] == bench.PEAK_HBM_GBPS
    assert math.isclose(prep["achieved"], round(by["prep"] / 0.05e-3 / 1e9, 1))
    c = bench.WORKLOADS["noncausal_b64_h16_n512_d64"]
    fs, _ = bench.flops(c["B"], c["H"], c["N"], c["d"], c["causal"])
    fb = bench.kernel_bytes(c["B"], c["H"], c["H"], c["N"], c["d"])["fwd"]
    assert fs / fb < bench.MACHINE_BALANCE


def test_every_workload_name_is_unique():
    names = [*bench.WORKLOADS, *bench.DECODE_WORKLOADS, *bench.FP8_WORKLOADS, *bench.PREP_WORKLOADS]
    assert len(names) == len(set(names))


def test_cli_refuses_several_gpus_and_bad_counts(capsys):
    """One GPU only: --gpus above 1 ends with a message and status 2 before
    anything touches a device; so do non-positive step counts."""
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU only" in capsys.readouterr().err
    assert bench.main(["--steps", "0"]) == 2
    assert bench.main(["--warmup", "-1"]) == 2


def test_cpu_baseline_cores_are_the_affinity_set():
    """The CPU baseline reports the cores of this process's affinity set and
    runs the oracle's BLAS with exactly that many threads."""
    import os

    from threadpoolctl import threadpool_info
    assert bench.host_cores() == len(os.sched_getaffinity(0))
    with bench.pinned_blas() as pin:
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        assert pin.cores == len(os.sched_getaffinity(0))
        assert all(p["num_threads"] == pin.cores for p in blas)


def test_new_workloads_are_listed():
    assert "varlen_causal_keypad_h32_d128" in bench.VARLEN_WORKLOADS
    assert "f32_b1_h1_n128_d64" in bench.F32_WORKLOADS
