"""Benchmark: serving-scale quantized Delta-rule decode on one MI355X.

Workload: 1024 requests x 32 GDN heads, 128x128 states packed at 8/6/4 bits by head
lifetime quartile (6.0 nominal code bits), one decode step per launch. A "step" is one
pass of the whole hot path (dequantize, gated delta update, readout, scale refit,
requantize, pack) over all 32,768 (request, head) states.

Prints ONE JSON line (see the keys below). ``value`` = state-updates/s over the timed
region (inputs already resident in HBM); ``roofline`` prices the step kernel's
algorithmic bytes per launch against MI355X's 8 TB/s HBM peak, from HIP events around
every timed launch on the launch stream; ``cpu_baseline`` times the scalar CPU oracle
on host threads over a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "state-updates/s (req x head) and % of HBM roofline, 1024-req mixed 6-bit"
HBM_PEAK_GBPS = 8000.0
# non-packed fp32 VALU issue rate of MI355X: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
VALU_PEAK_LANE_OPS = 256 * 4 * 16 * 2.4e9
PROFILE = os.path.join(ROOT, "profiles", "k_step_gdn_serving_1024x32.md")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(layout, n_unit: int, gate: int) -> int:
    """Bytes the step must move per launch: packed codes read + written, key-row and
    value-column scales read + written (fp32), q/k/v read, a and b read, o written."""
    codes = 2 * layout.packed_bytes
    scales = 2 * 2 * n_unit * 128 * 4
    qkv = 3 * n_unit * 128 * 4
    gates = n_unit * 4 * (128 if gate == 1 else 1) + n_unit * 4
    out = n_unit * 128 * 4
    return codes + scales + qkv + gates + out


def profile_record():
    """Machine-readable lines of the committed rocprofv3 summary of the step kernel, or {}
    when they were taken on a different kernel source than the one built here."""
    from quantized_delta_rule_03_amd import rocprof_summary

    try:
        rec = {}
        with open(PROFILE) as f:
            for line in f:
                k, sep, v = line.partition(": ")
                if sep and k.replace("_", "").isalnum() and " " not in k:
                    rec[k] = v.strip()
    except OSError:
        return {}
    if rec.get("kernel_source_sha256") != rocprof_summary.kernel_source_sha256(ROOT):
        return {}
    return rec


def cpu_baseline(w, bits, threads: int, n_req: int, steps: int):
    import oracle
    from quantized_delta_rule_03_amd import workloads as wl

    pool = oracle.Pool(n_req, w.n_head, bits)
    pool.quantize(np.zeros((n_req, w.n_head, 128, 128), np.float32))
    inputs = [wl.step_inputs(w, t, n_req=n_req) for t in range(steps)]
    t0 = time.perf_counter()
    for inp in inputs:
        pool.step_threads(w.gate, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"],
                          threads=threads)
    dt = time.perf_counter() - t0
    updates = n_req * w.n_head * steps
    return {"value": updates / dt, "unit": "state-updates/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{steps} steps x {n_req} requests x {w.n_head} heads "
                      f"({updates} state updates) of the same workload, oracle on "
                      f"{threads} host threads, {dt:.2f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-requests", type=int, default=1024)
    ap.add_argument("--cpu-steps", type=int, default=8)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the decode step has "
              "no cross-GPU exchange; run one process per GPU on its own requests.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from quantized_delta_rule_03_amd import qdr
    from quantized_delta_rule_03_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = wl.WORKLOADS[3]
    bits = qdr.assign_bits(w.gate, wl.halflives(w, args.seed))
    pool = qdr.StatePool(w.n_req, w.n_head, w.gate, bits, device=dev)
    L = pool.layout
    n_unit = w.n_unit
    a = torch.from_numpy(wl.static_gate(w, args.seed)).to(dev)
    total = args.warmup + args.steps
    log(f"generating {total} steps of inputs on the device")
    inputs = [wl.device_step_inputs(w, t, dev, args.seed) for t in range(total)]
    o = torch.empty((w.n_req, w.n_head, 128), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def launch(inp):
        pool.step(inp["q"], inp["k"], inp["v"], a, inp["b"], o, stream=stream)

    for t in range(args.warmup):
        launch(inputs[t])
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps); timing {args.steps} steps")

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        launch(inputs[args.warmup + i])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = np.array([s.elapsed_time(e) for s, e in ev])
    avg_kern_s = float(kern_ms.mean()) / 1e3
    ms_per_step = wall * 1e3 / args.steps
    value = n_unit / (wall / args.steps)
    nbytes = algorithmic_bytes(L, n_unit, w.gate)
    achieved = nbytes / avg_kern_s / 1e9
    log(f"step kernel: mean {kern_ms.mean()*1e3:.1f} us, median {np.median(kern_ms)*1e3:.1f} us; "
        f"{achieved:.0f} GB/s algorithmic ({100*achieved/HBM_PEAK_GBPS:.1f}% of 8 TB/s)")

    prof = profile_record()
    traffic = float(prof["traffic_bytes_per_launch"]) if "traffic_bytes_per_launch" in prof else None
    valu = None
    if "SQ_INSTS_VALU" in prof:
        lane_ops = float(prof["SQ_INSTS_VALU"]) * 64
        valu = {"lane_ops_per_launch": lane_ops, "achieved": lane_ops / avg_kern_s,
                "peak": VALU_PEAK_LANE_OPS, "unit": "lane-ops/s",
                "frac": lane_ops / avg_kern_s / VALU_PEAK_LANE_OPS}

    cpu = None
    if not args.no_cpu_baseline:
        threads = min(16, os.cpu_count() or 1)
        log(f"cpu baseline: oracle on {threads} threads, {args.cpu_requests} requests x "
            f"{args.cpu_steps} steps")
        cpu = cpu_baseline(w, bits, threads, args.cpu_requests, args.cpu_steps)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "n_req": w.n_req, "n_head": w.n_head, "dk": 128,
                   "dv": 128, "gate": "GDN scalar, half-life log-uniform [1, 4096]",
                   "bits": "8/6/4 by head lifetime quartile (6.0 code bits/value)",
                   "steps_per_launch": 1, "parallelism": "single GPU"},
        "hbm_gbps": achieved,
        "pct_hbm_roofline": 100.0 * achieved / HBM_PEAK_GBPS,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": "k_step<GDN>", "bytes_per_launch": nbytes,
                     "avg_launch_us": avg_kern_s * 1e6},
        "valu": valu,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
