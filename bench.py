#!/usr/bin/env python3
"""Benchmark: fused exact attention forward + backward on one MI355X.

One step is one full pass of the hot path over the workload: the forward
(attn_fwd) followed by the whole backward as attn_bwd runs it (the query-tile
pass for dQ, which also forms D = rowsum(dO o O), then the key-tile pass for
dK/dV).  Inputs are seeded synthetic tensors already resident in HBM before
the timed region.

Workload (default): causal self-attention, B=4, H=32, N=4096, d=128, bf16,
scale 1/sqrt(128), Q/K/V/dO ~ N(0,1) rounded to bf16, seed 0.  With grouped
key/value heads (H_kv < H) or a window / block list the step is the
forward entry point + one backward call (its kernels are not split by
events).

FLOP accounting: forward 4*B*H*N^2*d, halved under the causal mask; backward
2.5x the forward (five N^2*d products, the recompute of S included).  The
key-tile pass executes four N^2*d products (S, dP, dV, dK; 2.0x the forward)
and the query-tile pass three (S, dP, dQ; 1.5x the forward).  Per-kernel
rates below use the products each kernel executes; the backward TFLOP/s
uses the method's 2.5x.  Byte accounting: each kernel's algorithmic HBM
bytes (every input it needs read once, every output written once).  The
roofline object takes the bound from the dominant kernel's arithmetic
intensity against the machine balance (2516.6 TFLOP/s / 8 TB/s): below it the
kernel is HBM-bound and reported in GB/s.

Other workloads: the D pre-pass alone (attn_bwd_preprocess, HBM-bound),
decoding against a KV cache (HBM-bound), the FP8 forward, packed
variable-length sequences with key padding, and the small fp32 problem.

Timing: the step first runs back to back for --settle-ms (default 250 ms)
of host time, then --warmup untimed steps, then exactly --steps steps
between two device synchronizations, with no other host work in between.
Per-kernel times come from HIP events on the library's stream (mean,
median, minimum); `value` is whole-job throughput over the wall time of the
timed steps.

The CPU baseline runs the fp64 oracle on the host with its BLAS threads
pinned to the cores of this process's affinity set (the count reported).

Prints ONE JSON line on stdout (progress goes to stderr).
"""
from __future__ import annotations

import argparse
import gc
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published dense peaks (256 CUs at 2.4 GHz).
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4e9 clk/s x 4096 FLOP/clk/CU
PEAK_HBM_GBPS = 8000.0

WORKLOADS = {
    "causal_b4_h32_n4096_d128": dict(B=4, H=32, N=4096, d=128, causal=True, sigma_qk=1.0),
    "causal_b1_h16_n16384_d128": dict(B=1, H=16, N=16384, d=128, causal=True, sigma_qk=1.5),
    "noncausal_b8_h16_n2048_d64": dict(B=8, H=16, N=2048, d=64, causal=False, sigma_qk=1.0),
    # short sequences: N = 512, d = 64, 32768 tokens per batch as in the 16-head N4096 B8 comparison;
    # the forward's arithmetic intensity (N / 2 FLOP per byte) is below the machine balance
    "noncausal_b64_h16_n512_d64": dict(B=64, H=16, N=512, d=64, causal=False, sigma_qk=1.0),
    # grouped key/value heads: 32 query heads share 8 K/V heads (groups of 4)
    "gqa_causal_b4_h32_hkv8_n4096_d128": dict(B=4, H=32, Hkv=8, N=4096, d=128, causal=True, sigma_qk=1.0),
    # causal sliding window of 4096 keys (window (4095, 0)) over 16384 tokens
    "swa4096_b1_h32_hkv8_n16384_d128": dict(B=1, H=32, Hkv=8, N=16384, d=128, causal=True, sigma_qk=1.0,
                                             window=(4095, 0)),
    # block-sparse, 128 x 128 blocks: block 0 (global), r-1, r, r+1 (local), every 16th block (strided)
    "blocksparse_b1_h32_hkv8_n16384_d128": dict(B=1, H=32, Hkv=8, N=16384, d=128, causal=False, sigma_qk=1.0,
                                                 blocks="global+local+strided16"),
}
SPARSE_BLOCK = 128
# FP8 (E4M3) forward: quantize Q, K, V from bf16, then the FP8 forward
FP8_WORKLOADS = {
    "fp8_causal_b4_h32_n4096_d128": dict(B=4, H=32, N=4096, d=128, causal=True),
}
PEAK_FP8_TFLOPS = 5033.2    # 2 x the bf16 dense peak
# the backward's D pre-pass alone (attn_bwd_preprocess) on the benchmark shape's O and dO
PREP_WORKLOADS = {
    "prep_b4_h32_n4096_d128": dict(B=4, H=32, N=4096, d=128),
}
# packed variable-length sequences: 16 sequences, lengths uniform in [64, 8192] (seed 0), H32 d128, causal,
# left key padding of max(1, round(0.01 L)) tokens per sequence (fully masks ~1% of the query rows)
VARLEN_WORKLOADS = {
    "varlen_causal_keypad_h32_d128": dict(nseq=16, len_lo=64, len_hi=8192, H=32, d=128, causal=True, pad=0.01),
}
# the fp32 problem: B1 H1 N128 d64, non-causal, scale 1/8 (latency-bound: one workgroup per 32 query rows)
F32_WORKLOADS = {
    "f32_b1_h1_n128_d64": dict(B=1, H=1, N=128, d=64, causal=False),
}
PEAK_FP32_MFMA_TFLOPS = 157.3
# decoding: one new token per sequence against a 32768-token KV cache
DECODE_WORKLOADS = {
    "decode_b8_h32_hkv8_n32768_d128": dict(B=8, H=32, Hkv=8, N=32768, d=128),
}


def block_rows(pattern, nb):
    """Key blocks listed per query block for a named block-sparse pattern."""
    if pattern == "global+local+strided16":
        return [sorted({0} | {c for c in (r - 1, r, r + 1) if 0 <= c < nb} | set(range(0, nb, 16)))
                for r in range(nb)]
    raise ValueError(pattern)


def visible_pairs(cfg):
    """Number of (query, key) pairs the mask keeps, per (batch, head)."""
    import numpy as np
    N = cfg["N"]
    i = np.arange(N, dtype=np.int64)
    if "window" in cfg:
        left, right = cfg["window"]
        lo = np.maximum(0, i - left) if left >= 0 else np.zeros_like(i)
        hi = np.minimum(N - 1, i + right) if right >= 0 else np.full_like(i, N - 1)
        if cfg["causal"]:
            hi = np.minimum(hi, i)
        return int(np.sum(hi - lo + 1))
    if "blocks" in cfg:
        nb = -(-N // SPARSE_BLOCK)
        size = np.minimum(SPARSE_BLOCK, N - np.arange(nb) * SPARSE_BLOCK)
        total = 0
        for r, cols in enumerate(block_rows(cfg["blocks"], nb)):
            for c in cols:
                if cfg["causal"] and c > r:
                    continue
                if cfg["causal"] and c == r:
                    total += int(size[r]) * (int(size[r]) + 1) // 2
                else:
                    total += int(size[r]) * int(size[c])
        return total
    return N * (N + 1) // 2 if cfg["causal"] else N * N
DEFAULT = "causal_b4_h32_n4096_d128"
METRIC = "attn fwd/bwd TFLOPS + % MFMA bf16 peak, causal B4 H32 N4096 d128, 1 MI355X"


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def flops(B, H, N, d, causal):
    fwd = 4.0 * B * H * N * N * d * (0.5 if causal else 1.0)
    return fwd, 2.5 * fwd


def workload_flops(cfg):
    """Forward and backward FLOPs.  Plain workloads use the customary count
    (N^2 per head, halved under the causal mask); windowed and block-sparse
    ones count only the (query, key) pairs their mask keeps."""
    if "window" in cfg or "blocks" in cfg:
        fwd = 4.0 * cfg["B"] * cfg["H"] * cfg["d"] * visible_pairs(cfg)
        return fwd, 2.5 * fwd
    return flops(cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["causal"])


def oracle_mask(cfg):
    """The oracle's mask arguments for a workload."""
    import numpy as np
    if "window" in cfg:
        return {"window": cfg["window"]}
    if "blocks" in cfg:
        nb = -(-cfg["N"] // SPARSE_BLOCK)
        rows = block_rows(cfg["blocks"], nb)
        row_ptr = np.zeros(nb + 1, np.int32)
        row_ptr[1:] = np.cumsum([len(r) for r in rows])
        col_idx = np.array([c for r in rows for c in r], np.int32)
        return {"blocks": (row_ptr, col_idx, SPARSE_BLOCK)}
    return {}


MACHINE_BALANCE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)   # FLOP per byte
KERNEL_KEYS = {"fwd_stag_kernel (attn_fwd)": "fwd_stag_kernel",
               "bwd_dkdv_kernel (attn_bwd_dkdv)": "bwd_dkdv_kernel",
               "bwd_dq_kernel (attn_bwd_dq_preprocess)": "bwd_dq_kernel",
               "bwd_prep_kernel (attn_bwd_preprocess)": "bwd_prep_kernel"}


def traffic_record(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def measured_traffic(kernel_label, workload):
    """HBM bytes per launch of a kernel from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE record of this workload (already divided by the copy
    calibration), or None when there is no record for the workload or the
    kernel source has changed since the counters were taken."""
    import hashlib
    path = traffic_record(workload)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    k = rec.get("kernels", {}).get(KERNEL_KEYS.get(kernel_label, ""))
    if not k:
        return None
    h = hashlib.sha256()
    for f in k["source_files"]:
        h.update(open(os.path.join(ROOT, "exact_tiled_attention_09_amd", "csrc", f), "rb").read())
    if h.hexdigest() != k["source_sha256"]:
        return None
    return int(k["hbm_read_bytes"] + k["hbm_write_bytes"])


TRAFFIC_SOURCES = {"fwd_stag_kernel": ["fwd_bf16.hip", "miattn_device.h"],
                   "bwd_dq_kernel": ["bwd_bf16.hip", "miattn_device.h"],
                   "bwd_dkdv_kernel": ["bwd_bf16.hip", "miattn_device.h"],
                   "bwd_prep_kernel": ["bwd_bf16.hip", "miattn_device.h"]}


def _counter_means(csv_path, counter):
    """Mean over dispatches of a rocprofv3 counter, per kernel name (the
    counter's rows of one dispatch are summed first)."""
    import csv
    per = {}
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        key = (r["Kernel_Name"], r["Dispatch_Id"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return {name: sum(v) / len(v) for name, v in out.items()}


def write_traffic_record(run_dir, workload, log_fn=print, out_path=None):
    """profiles/traffic_<workload>.json from four rocprofv3 --pmc runs under
    run_dir: fetch/ and write/ (FETCH_SIZE, WRITE_SIZE of this workload's
    bench.py run) and cal_fetch/, cal_write/ (the same counters over the plain
    device copy of --copy-calibration-mib).  Counters are in KiB per
    dispatch; each is divided by what it reads per byte the copy moves."""
    import hashlib
    f = lambda sub: os.path.join(run_dir, sub, "run_counter_collection.csv")
    cal_f, cal_w = _counter_means(f("cal_fetch"), "FETCH_SIZE"), _counter_means(f("cal_write"), "WRITE_SIZE")
    copy_f = [v for n, v in cal_f.items() if "copy" in n.lower()]
    copy_w = [v for n, v in cal_w.items() if "copy" in n.lower()]
    if not copy_f or not copy_w:
        raise SystemExit("no copy kernel in the calibration runs")
    info = json.load(open(os.path.join(run_dir, "calibration.json")))
    nbytes = info["copy_calibration_bytes"]
    ff, fw = copy_f[0] * 1024 / nbytes, copy_w[0] * 1024 / nbytes
    fetch, write = _counter_means(f("fetch"), "FETCH_SIZE"), _counter_means(f("write"), "WRITE_SIZE")
    kernels = {}
    for name, kib in fetch.items():
        key = next((k for k in TRAFFIC_SOURCES if k in name), None)
        if key is None or name not in write:
            continue
        h = hashlib.sha256()
        for src in TRAFFIC_SOURCES[key]:
            h.update(open(os.path.join(ROOT, "exact_tiled_attention_09_amd", "csrc", src), "rb").read())
        kernels[key] = {"instance": name.split("(")[0].replace("void ", "").replace("miattn::", ""),
                        "hbm_read_bytes": int(kib * 1024 / ff), "hbm_write_bytes": int(write[name] * 1024 / fw),
                        "source_sha256": h.hexdigest(), "source_files": TRAFFIC_SOURCES[key]}
    rec = {"workload": workload, "calibration": {"fetch_factor": round(ff, 4), "write_factor": round(fw, 4),
                                                 "copy_bytes": nbytes}, "kernels": kernels}
    out_path = out_path or traffic_record(workload)
    with open(out_path, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    log_fn(f"wrote {out_path}: {sorted(kernels)}")
    return rec


def kernel_bytes(B, H, Hkv, N, d):
    """Algorithmic HBM bytes of each kernel of a bf16 step: every tensor the
    kernel needs read once and every tensor it produces written once (bf16
    Q, K, V, O, dO and gradients; fp32 LSE and D)."""
    eq, ekv, rows = B * H * N * d * 2, B * Hkv * N * d * 2, B * H * N * 4
    return {
        "fwd": eq + 2 * ekv + eq + rows,                        # Q, K, V -> O, LSE
        "dq": 3 * eq + 2 * ekv + rows + eq + rows,              # Q, O, dO, K, V, LSE -> dQ, D
        "dkdv": 2 * eq + 2 * ekv + 2 * rows + 2 * ekv,          # Q, dO, K, V, LSE, D -> dK, dV
        "bwd": 3 * eq + 2 * ekv + rows + eq + 2 * ekv,          # Q, O, dO, K, V, LSE -> dQ, dK, dV
        "prep": 2 * eq + rows,                                  # O, dO -> D
    }


def roofline_entry(kernel, ms, flop, nbytes, traffic):
    """The roofline object of one kernel: HBM-bound (GB/s against 8 TB/s) when
    its arithmetic intensity is below the machine balance, else MFMA-bound
    (TFLOP/s against the bf16 dense peak)."""
    intensity = flop / nbytes
    entry = {"kernel": kernel}
    if intensity < MACHINE_BALANCE:
        a = nbytes / (ms * 1e-3) / 1e9
        entry.update({"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                      "frac": round(a / PEAK_HBM_GBPS, 4)})
    else:
        a = flop / (ms * 1e-3) / 1e12
        entry.update({"bound": "mfma", "achieved": round(a, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(a / PEAK_BF16_TFLOPS, 4)})
    entry.update({"traffic": traffic, "flops_per_launch": flop, "bytes_per_launch": nbytes,
                  "intensity_flop_per_byte": round(intensity, 1), "avg_launch_ms": round(ms, 4)})
    return entry


class no_gc:
    """The timed region runs with Python's garbage collector off: a full
    collection while the host is enqueueing would let the GPU drain its queue
    and idle, and the idle time would land inside one stage's events."""

    def __enter__(self):
        self.was = gc.isenabled()
        gc.collect()
        gc.disable()

    def __exit__(self, *exc):
        if self.was:
            gc.enable()
        return False


def settle(step, stream, ms):
    """Run `step` back to back for `ms` milliseconds before the warm-up.

    Under a steady load the part settles to a lower power state than the one
    it starts a burst in: after even a few milliseconds idle, the next dozen
    steps of the benchmark workload run 5-30% slower than the steps after
    them.  The host stays at most four steps ahead (it waits for the event of
    the step four back), so the queue never drains and the device never idles
    in between."""
    if ms <= 0:
        return
    import torch
    pending = []
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        step()
        e = torch.cuda.Event()
        e.record(stream)
        pending.append(e)
        if len(pending) > 4:
            pending.pop(0).synchronize()


def timed_steps(args, stream, step, n_events):
    """Settle, warm up, then time exactly `args.steps` steps.

    Events are created and the garbage collector is stopped before the
    settle phase, so that between the last warm-up step and the first timed
    one the host only synchronizes: no host work leaves the device idle
    there.  Returns the per-step event lists and the wall time of the timed
    steps."""
    import torch
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_events)] for _ in range(args.steps)]
    log(f"settle {args.settle_ms} ms, warm up {args.warmup} steps, time {args.steps} steps")
    with no_gc():
        settle(step, stream, args.settle_ms)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for ev in events:
            step(ev)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    return events, wall


def host_cores() -> int:
    """Cores this process may run on (its CPU affinity set)."""
    return len(os.sched_getaffinity(0))


class pinned_blas:
    """Runs the oracle with its BLAS threads pinned to the host cores this
    process may use, so that the core count the baseline reports is the one it
    ran on."""

    def __enter__(self):
        from threadpoolctl import threadpool_limits
        self.cores = host_cores()
        self.ctl = threadpool_limits(limits=self.cores, user_api="blas")
        return self

    def __exit__(self, *exc):
        self.ctl.restore_original_limits()
        return False


def cpu_baseline(inp, cfg, scale, budget_s=10.0):
    """The fp64 oracle, forward + backward, on whole (b, h) heads of the same
    inputs, head after head until about ``budget_s`` seconds of host time
    have been spent (at least one head, at most all of them); the rate is
    scaled to the whole batch.  A reported baseline, not a target."""
    from oracle import attention as A
    B, H, N, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
    G = H // cfg.get("Hkv", H)
    heads = 0
    with pinned_blas() as pin:
        threads = pin.cores
        t0 = time.perf_counter()
        while heads < B * H:
            b, h = divmod(heads, H)
            A.head_backward(inp["q"][b, h], inp["k"][b, h // G], inp["v"][b, h // G], inp["do"][b, h], scale,
                            cfg["causal"], **oracle_mask(cfg))
            heads += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
    f_fwd, f_bwd = workload_flops(dict(cfg, B=1, H=1))
    per_head = dt / heads
    return {
        "value": round(heads * (f_fwd + f_bwd) / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{heads} of the {B * H} heads of the workload (fp64, forward+backward) in {dt:.1f} s on the "
                  f"host; whole-job time scales by B*H: {per_head * B * H:.0f} s",
    }


def run_fp8(args, cfg):
    """FP8 forward: one step quantizes Q, K, V (bf16 -> E4M3 codes + scales)
    and runs the FP8 forward.  value: forward FLOPs / whole step time; the
    roofline is the FP8 forward kernel alone against the FP8 dense peak."""
    import torch
    import exact_tiled_attention_09_amd as M
    from attn_inputs import dense_inputs
    B, H, N, d, causal = cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["causal"]
    scale = 1.0 / math.sqrt(d)
    log(f"workload {args.workload}: generating inputs")
    inp = dense_inputs(B, H, N, d, "bf16", seed=0, with_do=False)
    q, k, v = (torch.from_numpy(inp[n]).to(torch.bfloat16).cuda().contiguous() for n in ("q", "k", "v"))
    nb = (N + 63) // 64
    q8, k8 = (torch.empty((B, H, N, d), dtype=torch.uint8, device="cuda") for _ in range(2))
    v8 = torch.empty((B, H, nb, d, 64), dtype=torch.uint8, device="cuda")
    sq, sk = (torch.empty((B, H, nb), dtype=torch.float32, device="cuda") for _ in range(2))
    sv = torch.empty((B, H), dtype=torch.float32, device="cuda")
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        M.attn_quantize_fp8_rows(q, q8, sq, stream)
        M.attn_quantize_fp8_rows(k, k8, sk, stream)
        M.attn_quantize_fp8_vt(v, v8, sv, stream)
        if ev is not None:
            ev[1].record(stream)
        M.attn_fwd_fp8(q8, sq, k8, sk, v8, sv, o, lse, scale, causal, stream)
        if ev is not None:
            ev[2].record(stream)

    events, wall = timed_steps(args, stream, step, 3)
    q_ms = statistics.fmean(ev[0].elapsed_time(ev[1]) for ev in events)
    f_ms = statistics.fmean(ev[1].elapsed_time(ev[2]) for ev in events)
    f_fwd, _ = flops(B, H, N, d, causal)
    ms_step = wall * 1e3 / args.steps
    fwd_tf = f_fwd / (f_ms * 1e-3) / 1e12
    qbytes = 3 * B * H * N * d * 2 + 3 * B * H * N * d + B * H * (2 * nb + 1) * 4
    result = {
        "metric": f"attn fp8 fwd TFLOPS, {args.workload}, 1 MI355X",
        "value": round(f_fwd / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3",
        "data": "synthetic",
        "config": {"workload": f"exact attention FP8 E4M3 forward (with quantization), "
                               f"{'causal' if causal else 'non-causal'} B{B} H{H} N{N} d{d}",
                   "B": B, "H": H, "N": N, "d": d, "causal": causal, "flops_fwd": f_fwd},
        "quantize": {"ms": round(q_ms, 4), "gbps": round(qbytes / (q_ms * 1e-3) / 1e9, 1)},
        "fwd": {"ms": round(f_ms, 4), "tflops": round(fwd_tf, 2),
                "pct_fp8_peak": round(100 * fwd_tf / PEAK_FP8_TFLOPS, 2),
                "pct_bf16_peak": round(100 * fwd_tf / PEAK_BF16_TFLOPS, 2)},
        "roofline": {"kernel": "fwd_fp8_kernel (attn_fwd_fp8)", "bound": "mfma", "achieved": round(fwd_tf, 2),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(fwd_tf / PEAK_FP8_TFLOPS, 4),
                     "traffic": None, "flops_per_launch": f_fwd, "avg_launch_ms": round(f_ms, 4)},
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)
    return 0


def run_prep(args, cfg):
    """The backward's D pre-pass alone: one step is one attn_bwd_preprocess
    call, D = rowsum(dO o O) for every row.  HBM-bound: value is its
    algorithmic bytes (O and dO read once, D written once) per second.  O
    comes from one untimed attn_fwd over the same inputs."""
    import torch
    import exact_tiled_attention_09_amd as M
    from attn_inputs import dense_inputs
    B, H, N, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
    scale = 1.0 / math.sqrt(d)
    log(f"workload {args.workload}: generating inputs")
    inp = dense_inputs(B, H, N, d, "bf16", seed=0)
    q, k, v, do = (torch.from_numpy(inp[n]).to(torch.bfloat16).cuda().contiguous() for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(M.attn_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    M.attn_fwd(q, k, v, o, lse, scale, True, stream)
    # one event pair around the back-to-back launches: for a ~40 us kernel a
    # pair around every launch would add its own few microseconds
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"settle {args.settle_ms} ms, warm up {args.warmup} launches, time {args.steps} launches")
    with no_gc():
        settle(lambda: M.attn_bwd_preprocess(o, do, ws, stream), stream, args.settle_ms)
        for _ in range(args.warmup):
            M.attn_bwd_preprocess(o, do, ws, stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(args.steps):
            M.attn_bwd_preprocess(o, do, ws, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = kernel_bytes(B, H, H, N, d)["prep"]
    flop = 2.0 * B * H * N * d
    label = "bwd_prep_kernel (attn_bwd_preprocess)"
    roofline = roofline_entry(label, ms, flop, nbytes, measured_traffic(label, args.workload))
    result = {
        "metric": f"D pre-pass HBM GB/s, {args.workload}, 1 MI355X",
        "value": roofline["achieved"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"backward D pre-pass D = rowsum(dO o O), B{B} H{H} N{N} d{d} bf16 -> fp32",
                   "B": B, "H": H, "N": N, "d": d, "bytes_per_step": nbytes},
        "prep": {"ms": round(ms, 4), "gbps": roofline["achieved"]},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import attention as A
        o_h = o.float().cpu().numpy()
        with pinned_blas() as pin:
            threads = pin.cores
            t0 = time.perf_counter()
            A.preprocess_d(o_h, inp["do"])
            dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": int(threads),
                                  "kind": "oracle", "sample": f"the whole step (all {B * H * N} rows, fp64) "
                                                              f"in {dt:.2f} s"}
    print(json.dumps(result), flush=True)
    return 0


def run_decode(args, cfg):
    """Decoding against a KV cache: one step is one attn_decode call (split
    pass + merge pass) for all B sequences.  HBM-bound: value is the
    algorithmic bytes (K and V caches once, q, O, LSE) per second."""
    import torch
    import exact_tiled_attention_09_amd as M
    from attn_inputs import decode_inputs
    B, H, Hkv, N, d = cfg["B"], cfg["H"], cfg["Hkv"], cfg["N"], cfg["d"]
    scale = 1.0 / math.sqrt(d)
    log(f"workload {args.workload}: generating inputs")
    inp = decode_inputs(B, H, Hkv, N, d, "bf16", seed=0)
    q, k, v = (torch.from_numpy(inp[n]).to(torch.bfloat16).cuda().contiguous() for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(M.attn_decode_workspace_bytes(B, H, Hkv, N, d), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        M.attn_decode(q, k, v, o, lse, scale, None, ws, stream)
        if ev is not None:
            ev[1].record(stream)

    events, wall = timed_steps(args, stream, step, 2)
    ms = statistics.fmean(e0.elapsed_time(e1) for e0, e1 in events)
    nbytes = 2 * B * Hkv * N * d * 2 + 2 * B * H * d * 2 + B * H * 4
    gbps = nbytes / (ms * 1e-3) / 1e9
    result = {
        "metric": f"decode attention HBM GB/s, {args.workload}, 1 MI355X",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"decoding, one token per sequence, B{B} H{H} H_kv{Hkv} KV cache N{N} d{d} bf16",
                   "B": B, "H": H, "H_kv": Hkv, "N_kv": N, "d": d, "bytes_per_step": nbytes},
        "decode": {"ms": round(ms, 4), "gbps": round(gbps, 1)},
        "roofline": {"kernel": "decode_split_kernel + decode_merge_kernel (attn_decode)", "bound": "hbm",
                     "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None,
                     "bytes_per_launch": nbytes, "avg_launch_ms": round(ms, 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import decode as Dc
        with pinned_blas() as pin:
            threads = pin.cores
            t0 = time.perf_counter()
            Dc.decode_forward(inp["q"], inp["k"], inp["v"], scale)
            dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": int(threads),
                                  "kind": "oracle", "sample": f"the whole step (all {B * H} heads) in {dt:.1f} s"}
    print(json.dumps(result), flush=True)
    return 0


def run_varlen(args, cfg):
    """Packed variable-length sequences with a key-padding mask: one step is
    attn_fwd_varlen then attn_bwd_varlen (its dQ pass, which also forms D, and
    its dK/dV pass).  FLOPs are the dense formulas summed per sequence (N =
    L_s).  The events bracket the forward and the whole backward; the
    roofline object is the forward kernel (the launch bracketed alone)."""
    import numpy as np
    import torch
    import exact_tiled_attention_09_amd as M
    from attn_inputs import left_padding_key_mask, varlen_inputs
    H, d, causal = cfg["H"], cfg["d"], cfg["causal"]
    scale = 1.0 / math.sqrt(d)
    log(f"workload {args.workload}: generating inputs")
    inp = varlen_inputs(cfg["nseq"], cfg["len_lo"], cfg["len_hi"], H, d, "bf16", seed=0)
    cu = inp["cu_seqlens"]
    kv = left_padding_key_mask(cu, cfg["pad"])
    T, maxlen = int(cu[-1]), int(inp["max_seqlen"])
    q, k, v, do = (torch.from_numpy(inp[n]).to(torch.bfloat16).cuda().contiguous() for n in ("q", "k", "v", "do"))
    cu_d = torch.from_numpy(cu).cuda()
    kv_d = torch.from_numpy(kv).cuda()
    M.check_cu_seqlens(cu, T, maxlen, "bench")
    o = torch.empty_like(q)
    lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(M.attn_bwd_varlen_workspace_bytes(T, H, d), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        M.attn_fwd_varlen(q, k, v, o, lse, cu_d, maxlen, scale, causal, kv_d, stream)
        if ev is not None:
            ev[1].record(stream)
        M.attn_bwd_varlen(q, k, v, o, lse, do, dq, dk, dv, cu_d, maxlen, scale, causal, ws, kv_d, stream)
        if ev is not None:
            ev[2].record(stream)

    events, wall = timed_steps(args, stream, step, 3)
    f_ms = statistics.fmean(ev[0].elapsed_time(ev[1]) for ev in events)
    b_ms = statistics.fmean(ev[1].elapsed_time(ev[2]) for ev in events)
    lengths = np.diff(cu).astype(np.float64)
    f_fwd = float(np.sum(4.0 * H * lengths ** 2 * d * (0.5 if causal else 1.0)))
    f_bwd = 2.5 * f_fwd
    ms_step = wall * 1e3 / args.steps
    tf_fwd = f_fwd / (f_ms * 1e-3) / 1e12
    tf_bwd = f_bwd / (b_ms * 1e-3) / 1e12
    by = kernel_bytes(1, H, H, T, d)
    label = "fwd_stag_kernel (attn_fwd_varlen, packed, key padding)"
    roofline = roofline_entry(label, f_ms, f_fwd, by["fwd"] + T, None)
    dead = sum(int(np.sum(np.cumsum(kv[cu[i]:cu[i + 1]]) == 0)) for i in range(len(cu) - 1))
    result = {
        "metric": f"attn fwd+bwd TFLOPS, {args.workload}, 1 MI355X",
        "value": round((f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"exact attention fwd+bwd, packed {len(lengths)} sequences (lengths uniform in "
                               f"[{cfg['len_lo']}, {cfg['len_hi']}], seed 0, {T} tokens), "
                               f"{'causal' if causal else 'non-causal'}, left key padding "
                               f"({dead} fully masked rows), H{H} d{d} bf16",
                   "nseq": len(lengths), "total_tokens": T, "max_seqlen": maxlen, "H": H, "d": d,
                   "causal": causal, "scale": scale, "flops_fwd": f_fwd, "flops_bwd": f_bwd,
                   "fully_masked_rows_per_head": dead},
        "fwd": {"ms": round(f_ms, 4), "tflops": round(tf_fwd, 2),
                "pct_mfma_peak": round(100 * tf_fwd / PEAK_BF16_TFLOPS, 2)},
        "bwd": {"ms": round(b_ms, 4), "tflops": round(tf_bwd, 2),
                "pct_mfma_peak": round(100 * tf_bwd / PEAK_BF16_TFLOPS, 2)},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on one head over every sequence")
        from oracle import attention as A
        with pinned_blas() as pin:
            t0 = time.perf_counter()
            A.varlen_backward(inp["q"], inp["k"], inp["v"], inp["do"], cu, scale, causal, kv, heads=[0])
            dt = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": round((f_fwd + f_bwd) / H / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(pin.cores),
            "kind": "oracle",
            "sample": f"head 0 over all {len(lengths)} sequences (fp64, forward+backward) in {dt:.1f} s on the "
                      f"host; whole-job time scales by H: {dt * H:.0f} s"}
    print(json.dumps(result), flush=True)
    return 0


def run_f32(args, cfg):
    """The fp32 problem: one step is attn_fwd_f32 then attn_bwd_f32.  At 4.2
    MFLOP it is latency-bound (a handful of workgroups), so the line reports
    its time; its parity against the oracle is measured in the CPU-baseline
    leg, which runs the oracle on the same inputs anyway."""
    import numpy as np
    import torch
    import exact_tiled_attention_09_amd as M
    from attn_inputs import dense_inputs
    B, H, N, d, causal = cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["causal"]
    scale = 1.0 / math.sqrt(d)
    inp = dense_inputs(B, H, N, d, "f32", seed=0)
    q, k, v, do = (torch.from_numpy(inp[n]).cuda().contiguous() for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(M.attn_bwd_f32_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        M.attn_fwd_f32(q, k, v, o, lse, scale, causal, stream)
        if ev is not None:
            ev[1].record(stream)
        M.attn_bwd_f32(q, k, v, o, lse, do, dq, dk, dv, scale, causal, ws, stream)
        if ev is not None:
            ev[2].record(stream)

    events, wall = timed_steps(args, stream, step, 3)
    f_ms = statistics.fmean(ev[0].elapsed_time(ev[1]) for ev in events)
    b_ms = statistics.fmean(ev[1].elapsed_time(ev[2]) for ev in events)
    f_fwd, f_bwd = flops(B, H, N, d, causal)
    ms_step = wall * 1e3 / args.steps
    tf = f_fwd / (f_ms * 1e-3) / 1e12
    result = {
        "metric": f"attn fwd+bwd time, {args.workload}, 1 MI355X",
        "value": round(ms_step * 1e3, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"exact attention fwd+bwd fp32, {'causal' if causal else 'non-causal'} "
                               f"B{B} H{H} N{N} d{d}", "B": B, "H": H, "N": N, "d": d, "causal": causal,
                   "scale": scale, "flops_fwd": f_fwd, "flops_bwd": f_bwd},
        "fwd": {"us": round(f_ms * 1e3, 2)},
        "bwd": {"us": round(b_ms * 1e3, 2)},
        "roofline": {"kernel": "fwd_f32_kernel (attn_fwd_f32)", "bound": "mfma", "achieved": round(tf, 4),
                     "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_FP32_MFMA_TFLOPS, 6),
                     "traffic": None, "flops_per_launch": f_fwd, "avg_launch_ms": round(f_ms, 5),
                     "note": "latency-bound: 4 workgroups of 32 query rows on a 256-CU chip"},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import attention as A
        with pinned_blas() as pin:
            t0 = time.perf_counter()
            reps = 0
            while True:
                ref = A.backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal)
                reps += 1
                if time.perf_counter() - t0 >= 1.0:
                    break
            dt = (time.perf_counter() - t0) / reps
        got = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
        err = {n: float(np.max(np.abs(t.cpu().numpy().astype(np.float64) - ref[n]))) for n, t in got.items()}
        result["cpu_baseline"] = {
            "value": round(dt * 1e6, 1), "unit": "us/step", "cores": int(pin.cores), "kind": "oracle",
            "sample": f"the whole step (fp64, forward+backward), mean of {reps} runs",
            "max_abs_err_gpu_vs_oracle": {n: float(f"{e:.3e}") for n, e in err.items()},
            "parity_bar": 1e-5}
    print(json.dumps(result), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=250.0,
                    help="before the warm-up, run the step back to back for this long (host time) so the "
                         "timed steps see the clock the part holds under steady load, not the transient "
                         "after idle; 0 turns it off")
    ap.add_argument("--step-times", metavar="PATH", default=None,
                    help="dense workloads: also write every timed step's per-kernel event times (ms) to PATH "
                         "as JSON")
    ap.add_argument("--workload", default=DEFAULT,
                    choices=sorted(WORKLOADS) + sorted(DECODE_WORKLOADS) + sorted(FP8_WORKLOADS)
                    + sorted(PREP_WORKLOADS) + sorted(VARLEN_WORKLOADS) + sorted(F32_WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (3 times) and exit; its FETCH_SIZE / "
                         "WRITE_SIZE readings calibrate the HBM traffic counters")
    ap.add_argument("--write-traffic", metavar="RUN_DIR", default=None,
                    help="no GPU work: write profiles/traffic_<workload>.json from the rocprofv3 counter runs "
                         "in RUN_DIR (fetch/, write/, cal_fetch/, cal_write/ and calibration.json, the line "
                         "--copy-calibration-mib printed)")
    args = ap.parse_args(argv)
    if args.write_traffic:
        write_traffic_record(args.write_traffic, args.workload, log)
        return 0
    if args.copy_calibration_mib > 0:
        import torch
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 3}))
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); every box here has a single MI355X "
              "and this build has no multi-GPU path", file=sys.stderr)
        return 2
    if args.steps <= 0 or args.warmup < 0 or args.settle_ms < 0:
        print("--steps must be > 0, --warmup and --settle-ms >= 0", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    import exact_tiled_attention_09_amd as M
    from attn_inputs import dense_inputs
    M.load()
    if args.workload in DECODE_WORKLOADS:
        return run_decode(args, DECODE_WORKLOADS[args.workload])
    if args.workload in FP8_WORKLOADS:
        return run_fp8(args, FP8_WORKLOADS[args.workload])
    if args.workload in PREP_WORKLOADS:
        return run_prep(args, PREP_WORKLOADS[args.workload])
    if args.workload in VARLEN_WORKLOADS:
        return run_varlen(args, VARLEN_WORKLOADS[args.workload])
    if args.workload in F32_WORKLOADS:
        return run_f32(args, F32_WORKLOADS[args.workload])

    cfg = WORKLOADS[args.workload]
    B, H, N, d, causal = cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["causal"]
    Hkv = cfg.get("Hkv", H)
    masked = "window" in cfg or "blocks" in cfg
    grouped = Hkv != H or masked   # timed as attn_fwd_* + one backward call
    scale = 1.0 / math.sqrt(d)
    log(f"workload {args.workload}: generating inputs")
    inp = dense_inputs(B, H, N, d, "bf16", seed=0, sigma_qk=cfg["sigma_qk"], kv_heads=Hkv if grouped else None)
    dev = {n: torch.from_numpy(inp[n]).to(torch.bfloat16).cuda().contiguous() for n in ("q", "k", "v", "do")}
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = M.attn_bwd_workspace_bytes(B, H, N, d)
    if "blocks" in cfg:
        mk = oracle_mask(cfg)["blocks"]
        ws_bytes = M.attn_bwd_block_sparse_workspace_bytes(B, H, Hkv, N, d, len(mk[1]))
        row_ptr = torch.from_numpy(mk[0]).cuda()
        col_idx = torch.from_numpy(mk[1]).cuda()
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    fwd_name = "attn_fwd_gqa"

    if "window" in cfg:
        wl, wr = cfg["window"]
        fwd_name = "attn_fwd_window"

        def fwd_call():
            M.attn_fwd_window(q, k, v, o, lse, scale, causal, wl, wr, stream)

        def bwd_call():
            M.attn_bwd_window(q, k, v, o, lse, do, dq, dk, dv, scale, causal, wl, wr, ws, stream)
    elif "blocks" in cfg:
        fwd_name = "attn_fwd_block_sparse"

        def fwd_call():
            M.attn_fwd_block_sparse(q, k, v, o, lse, scale, causal, row_ptr, col_idx, stream)

        def bwd_call():
            M.attn_bwd_block_sparse(q, k, v, o, lse, do, dq, dk, dv, scale, causal, row_ptr, col_idx, ws, stream)
    else:
        def fwd_call():
            M.attn_fwd_gqa(q, k, v, o, lse, scale, causal, stream)

        def bwd_call():
            M.attn_bwd_gqa(q, k, v, o, lse, do, dq, dk, dv, scale, causal, ws, stream)

    def step_grouped(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fwd_call()
        if ev is not None:
            ev[1].record(stream)
        bwd_call()
        if ev is not None:
            ev[3].record(stream)

    def step(ev=None):
        if grouped:
            return step_grouped(ev)
        if ev is not None:
            ev[0].record(stream)
        M.attn_fwd(q, k, v, o, lse, scale, causal, stream)
        if ev is not None:
            ev[1].record(stream)
        # the backward as attn_bwd runs it: the dQ pass (which also stores D),
        # then the dK/dV pass
        M.attn_bwd_dq_preprocess(q, k, v, o, lse, do, dq, scale, causal, ws, stream)
        if ev is not None:
            ev[2].record(stream)
        M.attn_bwd_dkdv(q, k, v, lse, do, dk, dv, scale, causal, ws, stream)
        if ev is not None:
            ev[3].record(stream)

    events, wall = timed_steps(args, stream, step, 4)

    per = {"fwd": [], "bwd_dkdv": [], "bwd_dq": [], "bwd": [], "step": []}
    for ev in events:
        per["fwd"].append(ev[0].elapsed_time(ev[1]))
        per["bwd"].append(ev[1].elapsed_time(ev[3]))
        per["step"].append(ev[0].elapsed_time(ev[3]))
        if not grouped:
            per["bwd_dq"].append(ev[1].elapsed_time(ev[2]))
            per["bwd_dkdv"].append(ev[2].elapsed_time(ev[3]))
    per = {k_: v_ for k_, v_ in per.items() if v_}
    if args.step_times:
        with open(args.step_times, "w") as f:
            json.dump({"settle_ms": args.settle_ms, "warmup": args.warmup, "ms": per}, f)
    mean = {k_: statistics.fmean(v_) for k_, v_ in per.items()}
    med = {k_: statistics.median(v_) for k_, v_ in per.items()}
    low = {k_: min(v_) for k_, v_ in per.items()}

    f_fwd, f_bwd = workload_flops(cfg)
    ms_step = wall * 1e3 / args.steps
    bwd_ms = mean["bwd"]
    f_dkdv, f_dq = 2.0 * f_fwd, 1.5 * f_fwd
    tflops_fwd = f_fwd / (mean["fwd"] * 1e-3) / 1e12
    tflops_bwd = f_bwd / (bwd_ms * 1e-3) / 1e12
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12

    by = kernel_bytes(B, H, Hkv, N, d)
    gbps = lambda nbytes, ms: round(nbytes / (ms * 1e-3) / 1e9, 1)  # noqa: E731
    bwd = {"ms": round(bwd_ms, 4), "ms_median": round(med["bwd"], 4), "ms_min": round(low["bwd"], 4),
           "tflops": round(tflops_bwd, 2),
           "pct_mfma_peak": round(100 * tflops_bwd / PEAK_BF16_TFLOPS, 2), "gbps": gbps(by["bwd"], bwd_ms)}
    # dominant kernel for the roofline: the longest of the MFMA kernels whose
    # launches the events bracket one by one
    kern = {"fwd_stag_kernel (attn_fwd)": (mean["fwd"], f_fwd, by["fwd"])}
    if not grouped:
        tflops_dkdv = f_dkdv / (mean["bwd_dkdv"] * 1e-3) / 1e12
        tflops_dq = f_dq / (mean["bwd_dq"] * 1e-3) / 1e12
        bwd.update({"dkdv_ms": round(mean["bwd_dkdv"], 4), "dkdv_ms_median": round(med["bwd_dkdv"], 4),
                    "dkdv_ms_min": round(low["bwd_dkdv"], 4), "dkdv_tflops": round(tflops_dkdv, 2),
                    "dkdv_gbps": gbps(by["dkdv"], mean["bwd_dkdv"]),
                    "dq_ms": round(mean["bwd_dq"], 4), "dq_ms_median": round(med["bwd_dq"], 4),
                    "dq_ms_min": round(low["bwd_dq"], 4), "dq_tflops": round(tflops_dq, 2),
                    "dq_gbps": gbps(by["dq"], mean["bwd_dq"]), "dq_forms_d": True})
        kern["bwd_dkdv_kernel (attn_bwd_dkdv)"] = (mean["bwd_dkdv"], f_dkdv, by["dkdv"])
        kern["bwd_dq_kernel (attn_bwd_dq_preprocess)"] = (mean["bwd_dq"], f_dq, by["dq"])
    else:
        kern = {f"fwd_stag_kernel ({fwd_name})": (mean["fwd"], f_fwd, by["fwd"])}
    dom = max(kern, key=lambda k_: kern[k_][0])
    dom_ms, dom_flops, dom_bytes = kern[dom]
    roofline = roofline_entry(dom, dom_ms, dom_flops, dom_bytes, measured_traffic(dom, args.workload))

    heads = f"H{H}" + (f" H_kv{Hkv}" if Hkv != H else "")
    mask_desc = ""
    if "window" in cfg:
        mask_desc = f" window{cfg['window']}"
    elif "blocks" in cfg:
        mask_desc = f" block-sparse {cfg['blocks']} ({SPARSE_BLOCK}x{SPARSE_BLOCK} blocks)"
    result = {
        "metric": METRIC if args.workload == DEFAULT else f"attn fwd+bwd TFLOPS, {args.workload}, 1 MI355X",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"exact attention fwd+bwd, {'causal' if causal else 'non-causal'}{mask_desc} "
                               f"B{B} {heads} N{N} d{d} bf16", "B": B, "H": H, "H_kv": Hkv, "N": N, "d": d,
                   "causal": causal, "scale": scale, "flops_fwd": f_fwd, "flops_bwd": f_bwd,
                   "visible_pairs_per_head": visible_pairs(cfg) if masked else None},
        "fwd": {"ms": round(mean["fwd"], 4), "ms_median": round(med["fwd"], 4), "ms_min": round(low["fwd"], 4),
                "tflops": round(tflops_fwd, 2),
                "pct_mfma_peak": round(100 * tflops_fwd / PEAK_BF16_TFLOPS, 2),
                "gbps": gbps(by["fwd"], mean["fwd"])},
        "bwd": bwd,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on one head")
        result["cpu_baseline"] = cpu_baseline(inp, cfg, scale)
    del np
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
