"""Host-side logic of bench.py, CPU only: the FLOP accounting of the masked
workloads counts exactly the (query, key) pairs the oracle's mask keeps, and
the block patterns are valid CSR lists."""
import math
import os

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
    assert bench.main(["--settle-ms", "-1"]) == 2


def test_settle_off_touches_nothing():
    """--settle-ms 0 runs no step (so the phase is off, not one step long)."""
    calls = []
    bench.settle(lambda: calls.append(1), None, 0)
    assert calls == []


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


def _counter_csv(path, rows):
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], r)))


def test_traffic_record_from_counter_runs(tmp_path):
    """The traffic record divides each kernel's mean FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch, rows of one dispatch summed) by what the counters read
    per byte of the calibration copy, and stamps the kernel sources' hash."""
    import hashlib
    import json
    copy = "__amd_rocclr_copyBuffer"
    fwd = "void miattn::fwd_stag_kernel<128, true, false, false, 0>(miattn::AttnArgs, int)"
    nbytes = 1 << 30
    # the copy reads 0.5 KiB per KiB moved and writes 1.0
    _counter_csv(str(tmp_path / "cal_fetch" / "run_counter_collection.csv"),
                 [(1, copy, "FETCH_SIZE", nbytes / 1024 * 0.5)])
    _counter_csv(str(tmp_path / "cal_write" / "run_counter_collection.csv"),
                 [(1, copy, "WRITE_SIZE", nbytes / 1024)])
    (tmp_path / "calibration.json").write_text(json.dumps({"copy_calibration_bytes": nbytes, "launches": 3}))
    # two dispatches, the first split over two rows: mean (300 + 100) KiB read
    _counter_csv(str(tmp_path / "fetch" / "run_counter_collection.csv"),
                 [(1, fwd, "FETCH_SIZE", 200.0), (1, fwd, "FETCH_SIZE", 100.0), (2, fwd, "FETCH_SIZE", 100.0)])
    _counter_csv(str(tmp_path / "write" / "run_counter_collection.csv"),
                 [(1, fwd, "WRITE_SIZE", 64.0), (2, fwd, "WRITE_SIZE", 64.0)])
    out = tmp_path / "rec.json"
    rec = bench.write_traffic_record(str(tmp_path), "w", log_fn=lambda m: None, out_path=str(out))
    k = rec["kernels"]["fwd_stag_kernel"]
    assert k["hbm_read_bytes"] == int(200.0 * 1024 / 0.5)
    assert k["hbm_write_bytes"] == 64 * 1024
    assert rec["calibration"]["fetch_factor"] == 0.5 and rec["calibration"]["write_factor"] == 1.0
    h = hashlib.sha256()
    for src in k["source_files"]:
        h.update(open(os.path.join(bench.ROOT, "exact_tiled_attention_09_amd", "csrc", src), "rb").read())
    assert k["source_sha256"] == h.hexdigest()
    assert json.loads(out.read_text()) == rec
