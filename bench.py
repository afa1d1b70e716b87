#!/usr/bin/env python3
"""Benchmark of the Block AttnRes stack forward on one MI355X.

Workload (default): Block AttnRes two-phase prefill, L = 48 sublayers, S = 8
(6 blocks, at most 7 sources), B = 8, T = 2048 (R = 16384 token rows),
D = 4096, bf16, seeded synthetic inputs already resident in HBM. A step is one
attnres_block_stack_forward: the query fold, 6 Phase-1 passes, 42 Phase-2
merges, 6 block closes and the final aggregate. Sublayer outputs come from a
resident table (the built-in table callback), so the timed region holds only
AttnRes work.

Prints ONE JSON line: tokens/s (value), the whole forward's algorithmic HBM
GB/s, a roofline entry for the dominant kernel (Phase 2: algorithmic bytes per
launch over its HIP-event-timed average duration, against 8 TB/s), and the
fp64 CPU oracle timed on a bounded row sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_HBM_GBPS = 8000.0
METRIC = "tokens/s and achieved HBM GB/s (% of peak) for Block AttnRes stack forward"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "phase2_block_L48_S8_traffic.json")


def kernels_digest() -> str:
    h = hashlib.sha256()
    for rel in ("depth_wise_attention_rms_amd/csrc/kernels.hip", "depth_wise_attention_rms_amd/csrc/device.hpp"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per Phase-2 launch from the committed counter summary, or None
    when it is absent, for another workload, or older than the kernels."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("kernels_sha256") != kernels_digest():
        return None
    return t.get("traffic_bytes_per_launch")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="block_L48_S8")
    ap.add_argument("--cpu-rows", type=int, default=6144,
                    help="token rows of the CPU-oracle baseline sample (0 disables it)")
    ap.add_argument("--calibration-copy-gib", type=float, default=0.0,
                    help="before the steps, copy a tensor of this many GiB with torch (a plain "
                         "copy kernel of known size, read once and written once) so hardware "
                         "counters of the same run can be scaled to bytes")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the AttnRes path shards token rows with no exchange, so per-GPU work is this "
              "single-GPU figure", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from depth_wise_attention_rms_amd import binding
    from depth_wise_attention_rms_amd import inputs
    from depth_wise_attention_rms_amd.workload import DeviceStack

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    wl = inputs.WORKLOADS[args.workload]
    assert wl.kind == "stack" and not wl.ring, "the benchmark times a resident-table stack workload"
    ds = DeviceStack(wl)
    nb = ds.nb
    stream = torch.cuda.current_stream()

    if args.calibration_copy_gib > 0:
        n = int(args.calibration_copy_gib * (1 << 30)) // 2
        src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        ds.forward()
    torch.cuda.synchronize()

    launches_per_step = 1 + wl.L + 2 * nb + 1
    binding.attnres_timing_enable(args.steps * launches_per_step + 16)
    binding.attnres_timing_reset()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        ds.forward()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / args.steps
    gpu_ms = ev0.elapsed_time(ev1) / args.steps
    kinds = {}
    for k in ("phase1", "phase2", "aggregate", "close", "fold"):
        n, ms, byts = binding.attnres_timing_read(k)
        if n:
            kinds[k] = {"launches_per_step": n / args.steps, "avg_us": 1e3 * ms / n,
                        "ms_per_step": ms / args.steps,
                        "bytes_per_launch": byts / n, "GBps": byts / (ms * 1e6)}
    binding.attnres_timing_enable(0)

    fwd_bytes = sum(v["bytes_per_launch"] * v["launches_per_step"] for k, v in kinds.items() if k != "fold")
    ms_per_step = wall_ms
    tokens_per_s = wl.R / (ms_per_step / 1e3)
    fwd_gbps = fwd_bytes / (ms_per_step * 1e6)

    dom = kinds["phase2"]
    traffic = measured_traffic(wl.name)
    roofline = {"bound": "hbm", "kernel": "phase2_kernel", "achieved": round(dom["GBps"], 1),
                "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(dom["GBps"] / PEAK_HBM_GBPS, 4),
                "traffic": traffic, "bytes_per_launch": dom["bytes_per_launch"],
                "avg_launch_us": round(dom["avg_us"], 2)}

    cpu = None
    if args.cpu_rows > 0:
        import oracle
        from depth_wise_attention_rms_amd.workload import EPS
        rows = np.sort(np.random.default_rng(0).choice(wl.R, size=min(args.cpu_rows, wl.R), replace=False))
        xr, vr = ds.host_rows(rows)
        cores = max(1, min(16, len(os.sched_getaffinity(0))))
        oracle.build() if not os.path.exists(oracle.LIBRARY) else None
        c0 = time.perf_counter()
        oracle.block_stack(xr, vr, ds.W_host, wl.S, eps=EPS, want_h=False, nthreads=cores)
        c1 = time.perf_counter()
        cpu = {"value": round(len(rows) / (c1 - c0), 1), "unit": "tokens/s", "cores": cores,
               "kind": "oracle",
               "sample": f"{len(rows)} of {wl.R} token rows (seed 0), full 48-sublayer naive "
                         f"forward in fp64, {c1 - c0:.2f} s wall"}

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "gpu_ms_per_step": round(gpu_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based normals; inputs resident in HBM)",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "D": wl.D, "L": wl.L, "S": wl.S,
                   "blocks": nb, "global_batch": wl.B, "seq_len": wl.T, "parallelism": "single GPU"},
        "achieved_GBps": round(fwd_gbps, 1),
        "hbm_frac": round(fwd_gbps / PEAK_HBM_GBPS, 4),
        "bytes_per_step": fwd_bytes,
        "roofline": roofline,
        "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kinds.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
