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

``--workload window`` and ``--workload chunk`` time the windowed serving shape (256
requests x 32 KDA heads, 8-bit, windows of 64 tokens) in window mode (one call per
token) and in chunk mode (one call per window) instead; ``--workload comp`` times chunk
mode with 16 compensator tokens per state.
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
BF16_MFMA_PEAK = 2.5e15  # dense bf16 matrix FLOP/s of MI355X
# non-packed fp32 VALU issue rate of MI355X: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
VALU_PEAK_LANE_OPS = 256 * 4 * 16 * 2.4e9
PROFILE = os.path.join(ROOT, "profiles", "k_step_gdn_serving_1024x32.md")
PROFILE_CHUNK = os.path.join(ROOT, "profiles", "k_chunk_kda_256x32_t64.md")
PROFILE_COMP = os.path.join(ROOT, "profiles", "k_chunk_comp16_kda_256x32_t64.md")
PROFILE_WINDOW = os.path.join(ROOT, "profiles", "k_window_kda_256x32_w64.md")
CLOCK_TRACE_PERIOD_S = 10e-6  # clock-trace sample spacing beside the timed launches
COMP_TOKENS = 16  # compensator tokens per unit in the --workload comp line


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


def profile_record(path=PROFILE):
    """Machine-readable lines of a committed rocprofv3 summary (default: the step kernel),
    or {} when they were taken on a different kernel source than the one built here."""
    from quantized_delta_rule_03_amd import rocprof_summary

    try:
        rec = {}
        with open(path) as f:
            for line in f:
                k, sep, v = line.partition(": ")
                if sep and k.replace("_", "").isalnum() and " " not in k:
                    rec[k] = v.strip()
    except OSError:
        return {}
    kernels = "damp" if "damp" in os.path.basename(path) else "k_step<"
    if rec.get("kernel_source_sha256") != rocprof_summary.kernel_source_sha256(ROOT, kernels):
        return {}
    return rec


def window_algorithmic_bytes(tile_bytes: int, n_unit: int, W: int) -> int:
    """Bytes one window (W tokens + fold) must move: per token the fixed packed state and
    its scales, q/k/v, the per-channel gate and b, o; the buffered (key, w) pairs of the
    earlier tokens read, the new pair appended, the cumulative gate and the keys' decay
    since their base read and written; at the last token the buffered keys written back
    decayed (the base moves there; on this workload no gate product falls low enough to
    move it earlier); at the end the buffer and state read once more and the requantized
    state and scales written."""
    per_unit = 0
    for t in range(W):
        per_unit += tile_bytes + 2 * 512      # packed state + key-row and value-column scales
        per_unit += 3 * 512 + 512 + 4 + 512   # q, k, v, a (per channel), b; o
        per_unit += 1024 * t                  # buffer read (keys, deltas)
        per_unit += 1024 + 2 * ((512 if t else 0) + 512)  # append (k, w); g and h read + written
        if t == W - 1:
            per_unit += 512 * t               # decayed keys written (the base moves)
    per_unit += tile_bytes + 1024 + 1024 * W + 512  # fold: state, scales, buffer, gate read
    per_unit += tile_bytes + 1024                   # requantized state and scales written
    return per_unit * n_unit


def bench_window(args, torch, qdr, wl, dev):
    """Window mode (config: 256 requests x 32 KDA heads, 8-bit, W = 64): time whole windows
    of W token launches (the last one with the fold)."""
    w = wl.WORKLOADS[4]
    bits = wl.uniform_bits(w.n_head, 8)
    W = w.window
    pool = qdr.StatePool(w.n_req, w.n_head, w.gate, bits, window=W, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    pool.quantize(0.1 * torch.randn((w.n_req, w.n_head, 128, 128), generator=g, device=dev))
    a = torch.from_numpy(wl.static_gate(w, args.seed)).to(dev)
    n_win = max(1, args.steps // W)
    log(f"generating {W} tokens of inputs on the device")
    inputs = [wl.device_step_inputs(w, t, dev, args.seed) for t in range(W)]
    o = torch.empty((w.n_req, w.n_head, 128), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def window():
        for t in range(W):
            x = inputs[t]
            pool.window_token(t, x["q"], x["k"], x["v"], a, x["b"], o, stream=stream)

    window()
    torch.cuda.synchronize()
    log(f"warmup window done; timing {n_win} windows of {W} tokens")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_win)]
    t0 = time.perf_counter()
    for i in range(n_win):
        ev[i][0].record(stream)
        window()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    win_s = float(np.mean([s.elapsed_time(e) for s, e in ev])) / 1e3
    n_unit = w.n_unit
    nbytes = window_algorithmic_bytes(pool.layout.packed_bytes // w.n_req // w.n_head, n_unit, W)
    achieved = nbytes / win_s / 1e9
    tokens = n_win * W
    log(f"window: {win_s * 1e6 / W:.1f} us per token (fold included); {achieved:.0f} GB/s "
        f"algorithmic ({100 * achieved / HBM_PEAK_GBPS:.1f}% of 8 TB/s)")
    # HBM bytes per window (W token dispatches and the fold) from the committed counters
    prof = profile_record(PROFILE_WINDOW)
    traffic = float(prof["traffic_bytes_per_call"]) if "traffic_bytes_per_call" in prof else None
    return {
        "metric": "token-updates/s (req x head), window mode W=64, 256-req KDA 8-bit",
        "value": n_unit * tokens / wall,
        "unit": "token-updates/s",
        "n_gpus": 1, "steps": tokens, "warmup": W, "ms_per_step": wall * 1e3 / tokens,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "n_req": w.n_req, "n_head": w.n_head, "dk": 128,
                   "dv": 128, "gate": "KDA per-channel, half-life log-uniform [1, 8192]",
                   "bits": "8 (uniform)", "window": W, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": "k_window_token<KDA> + k_window_fold<KDA>",
                     "bytes_per_window": nbytes, "avg_window_us": win_s * 1e6},
        "cpu_baseline": None,
    }


def chunk_algorithmic_bytes(tile_bytes: int, n_unit: int, T: int, m: int = 0) -> int:
    """Bytes one chunk call (T tokens) must move: the packed state and its scales read
    once and written once; per token q, k, v, the per-channel gate and b read and o
    written; with m compensator tokens, their index (2 B) and value (4 B) read and
    written."""
    per_unit = 2 * (tile_bytes + 2 * 512) + T * (3 * 512 + 512 + 4 + 512) + 2 * 6 * m
    return per_unit * n_unit


def chunk_method_flops(n_unit: int, T: int) -> float:
    """The matrix products the chunked form of the method needs per call, counted once (2
    FLOPs per multiply-add): per unit and sub-block of C = 16 tokens, S_r(gam k) and
    S_r(gam q) (2 x 128 x 128 x C), the two C x C Gram matrices over the 128 key channels,
    the readout term B delta (C x C x 128) and the state update S += sum_t delta_t k_t^T
    (128 x 128 x C)."""
    n_sub = -(-T // 16)
    C = 16
    per_sub = 2 * (2 * 128 * 128 * C + 2 * C * C * 128 + C * C * 128 + 128 * 128 * C)
    return float(n_unit) * n_sub * per_sub


def chunk_issued_flops(n_unit: int, T: int) -> float:
    """Matrix-core FLOPs as the kernel issues them: per unit and 16-token sub-block, 624
    v_mfma_f32_16x16x32_bf16 (each fp32 operand split into three bf16 parts, six part
    products per operand pair) and 32 v_mfma_f32_16x16x4_f32."""
    n_sub = -(-T // 16)
    return float(n_unit) * n_sub * (624 * 16 * 16 * 32 * 2 + 32 * 16 * 16 * 4 * 2)


def bench_chunk(args, torch, qdr, wl, dev, m=0):
    """Chunk mode on the windowed serving shape (256 requests x 32 KDA heads, 8-bit): one
    qdr_decode_chunk call takes the window's T = 64 tokens at once. m > 0: the same with
    m compensator tokens per state (qdr_comp_chunk)."""
    w = wl.WORKLOADS[4]
    bits = wl.uniform_bits(w.n_head, 8)
    T = w.window
    pool = qdr.StatePool(w.n_req, w.n_head, w.gate, bits, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    S0 = 0.1 * torch.randn((w.n_req, w.n_head, 128, 128), generator=g, device=dev)
    if m:
        pool.comp_quantize(S0, m)
    else:
        pool.quantize(S0)
    del S0
    a1 = torch.from_numpy(wl.static_gate(w, args.seed)).to(dev)
    n_chunk = max(16, args.steps // T)  # at least 16 calls (about 13 ms) in the timed region
    log(f"generating {T} tokens of inputs on the device")
    toks = [wl.device_step_inputs(w, t, dev, args.seed) for t in range(T)]
    x = {k: torch.stack([t[k] for t in toks]).contiguous() for k in toks[0]}
    a = a1.unsqueeze(0).expand((T,) + tuple(a1.shape)).contiguous()
    del toks
    o = torch.empty((T, w.n_req, w.n_head, 128), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def chunk():
        if m:
            pool.comp_chunk(x["q"], x["k"], x["v"], a, x["b"], o, stream=stream)
        else:
            pool.chunk(x["q"], x["k"], x["v"], a, x["b"], o, stream=stream)

    for _ in range(max(1, args.warmup)):
        chunk()
    torch.cuda.synchronize()
    log(f"warmup done; timing {n_chunk} chunks of {T} tokens")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_chunk)]
    t0 = time.perf_counter()
    for i in range(n_chunk):
        ev[i][0].record(stream)
        chunk()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    chunk_s = float(np.mean([s.elapsed_time(e) for s, e in ev])) / 1e3
    n_unit = w.n_unit
    nbytes = chunk_algorithmic_bytes(pool.layout.packed_bytes // w.n_req // w.n_head, n_unit, T,
                                     m)
    achieved = nbytes / chunk_s / 1e9
    tokens = n_chunk * T
    log(f"chunk (m={m}): {chunk_s * 1e6:.1f} us per {T}-token call, {chunk_s * 1e6 / T:.2f} us "
        f"per token; {achieved:.0f} GB/s algorithmic "
        f"({100 * achieved / HBM_PEAK_GBPS:.1f}% of 8 TB/s)")
    prof = profile_record(PROFILE_COMP if m else PROFILE_CHUNK)
    traffic = float(prof["traffic_bytes_per_launch"]) if "traffic_bytes_per_launch" in prof else None
    flops = chunk_method_flops(n_unit, T)
    issued = chunk_issued_flops(n_unit, T)
    mfma = {"method_flops_per_call": flops, "achieved": flops / chunk_s,
            "peak": BF16_MFMA_PEAK, "unit": "FLOP/s", "frac": flops / chunk_s / BF16_MFMA_PEAK,
            "issued_flops_per_call": issued,
            "issued_frac": issued / chunk_s / BF16_MFMA_PEAK}
    valu = None
    if "SQ_INSTS_VALU" in prof:
        lane_ops = float(prof["SQ_INSTS_VALU"]) * 64
        valu = {"lane_ops_per_launch": lane_ops, "achieved": lane_ops / chunk_s,
                "peak": VALU_PEAK_LANE_OPS, "unit": "lane-ops/s",
                "frac": lane_ops / chunk_s / VALU_PEAK_LANE_OPS}
    comp = f", {m} compensator tokens" if m else ""
    return {
        "metric": f"token-updates/s (req x head), chunk mode T=64{comp}, 256-req KDA 8-bit",
        "value": n_unit * tokens / wall,
        "unit": "token-updates/s",
        "n_gpus": 1, "steps": tokens, "warmup": max(1, args.warmup) * T,
        "ms_per_step": wall * 1e3 / tokens,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name + (" (chunk, compensator tokens)" if m else " (chunk)"),
                   "n_req": w.n_req, "n_head": w.n_head,
                   "dk": 128, "dv": 128, "gate": "KDA per-channel, half-life log-uniform [1, 8192]",
                   "bits": "8 (uniform)", "tokens_per_call": T, "compensator_tokens": m,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": "k_chunk<KDA>", "bytes_per_call": nbytes,
                     "avg_call_us": chunk_s * 1e6},
        "mfma": mfma,
        "valu": valu,
        "cpu_baseline": None,
    }


def bench_compare(args, torch, qdr, wl, dev):
    """The decode step under each scale rule on the serving shape (1024 requests x 32 GDN
    heads): STEPQuant at the lifetime map (the default line) and at 8 bits, and the
    per-key-row and per-tensor INT8 baselines (8 bits). Same kernel skeleton; the rules
    differ only in the refit."""
    w = wl.WORKLOADS[3]
    mixed = qdr.assign_bits(w.gate, wl.halflives(w, args.seed))
    b8 = wl.uniform_bits(w.n_head, 8)
    settings = [("step_mixed", mixed, qdr.RULE_STEP), ("step_8bit", b8, qdr.RULE_STEP),
                ("keyrow_int8", b8, qdr.RULE_KEYROW), ("tensor_int8", b8, qdr.RULE_TENSOR)]
    a = torch.from_numpy(wl.static_gate(w, args.seed)).to(dev)
    n_in = 8
    inputs = [wl.device_step_inputs(w, t, dev, args.seed) for t in range(n_in)]
    o = torch.empty((w.n_req, w.n_head, 128), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    steps = max(16, args.steps)
    rules = {}
    for name, bits, rule in settings:
        pool = qdr.StatePool(w.n_req, w.n_head, w.gate, bits, device=dev, rule=rule)
        for t in range(max(3, args.warmup)):
            x = inputs[t % n_in]
            pool.step(x["q"], x["k"], x["v"], a, x["b"], o, stream=stream)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for i in range(steps):
            x = inputs[i % n_in]
            ev[i][0].record(stream)
            pool.step(x["q"], x["k"], x["v"], a, x["b"], o, stream=stream)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        us = float(np.mean([s_.elapsed_time(e_) for s_, e_ in ev])) * 1e3
        nbytes = algorithmic_bytes(pool.layout, w.n_unit, w.gate)
        rules[name] = {"us_per_step": us, "state_updates_per_s": w.n_unit / (us / 1e6),
                       "gbps": nbytes / (us / 1e6) / 1e9, "bytes_per_step": nbytes}
        log(f"{name}: {us:.1f} us per step, {rules[name]['gbps']:.0f} GB/s algorithmic")
        del pool
    ref = rules["step_8bit"]
    return {
        "metric": "decode-step time per scale rule, 1024-req GDN (STEPQuant vs INT8 baselines)",
        "value": ref["state_updates_per_s"], "unit": "state-updates/s (STEPQuant 8-bit)",
        "n_gpus": 1, "steps": steps, "warmup": max(3, args.warmup), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name + " (rules)", "n_req": w.n_req, "n_head": w.n_head},
        "rules": rules,
    }


def bench_layers(args, torch, qdr, wl, dev):
    """The decode step on the two layer configurations: the GDN layer (64 requests x 32
    heads, 8/6/4-bit heads, from the zero state) and the KDA layer (256 requests x 32
    heads, 8/6/4-bit key channels per head, from a seeded Gaussian state with outlier rows
    and columns: the timing does not depend on the values). Their working sets (58.7 MB
    and 239 MB) fit the 256 MB last-level cache, so these lines are flagged cache-resident
    (the GDN one is also close to launch-bound): not HBM measurements."""
    out = []
    for wid in (1, 2):
        w = wl.WORKLOADS[wid]
        bits = qdr.assign_bits(w.gate, wl.halflives(w, args.seed))
        pool = qdr.StatePool(w.n_req, w.n_head, w.gate, bits, device=dev)
        if wid == 2:
            g = torch.Generator(device=dev)
            g.manual_seed(args.seed)
            S0 = torch.randn((w.n_req, w.n_head, 128, 128), generator=g, device=dev)
            S0[:, :, :, ::97] *= 10.0
            S0[:, :, ::89, :] *= 10.0
            pool.quantize(S0)
            del S0
        a = torch.from_numpy(wl.static_gate(w, args.seed)).to(dev)
        n_in = 8
        inputs = [wl.device_step_inputs(w, t, dev, args.seed) for t in range(n_in)]
        o = torch.empty((w.n_req, w.n_head, 128), dtype=torch.float32, device=dev)
        stream = torch.cuda.current_stream()
        for t in range(max(3, args.warmup)):
            x = inputs[t % n_in]
            pool.step(x["q"], x["k"], x["v"], a, x["b"], o, stream=stream)
        torch.cuda.synchronize()
        steps = max(20, args.steps)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            x = inputs[i % n_in]
            ev[i][0].record(stream)
            pool.step(x["q"], x["k"], x["v"], a, x["b"], o, stream=stream)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        us = float(np.mean([s_.elapsed_time(e_) for s_, e_ in ev])) * 1e3
        nbytes = algorithmic_bytes(pool.layout, w.n_unit, w.gate)
        gbps = nbytes / (us / 1e6) / 1e9
        log(f"{w.name}: {us:.1f} us per step (kernel), {wall * 1e6 / steps:.1f} us wall; "
            f"{gbps:.0f} GB/s algorithmic (cache-resident working set {nbytes / 1e6:.1f} MB)")
        out.append({"workload": w.name, "n_req": w.n_req, "n_head": w.n_head,
                    "units": w.n_unit, "us_per_step_kernel": us,
                    "us_per_step_wall": wall * 1e6 / steps,
                    "state_updates_per_s": w.n_unit / (wall / steps),
                    "gbps_algorithmic": gbps, "bytes_per_step": nbytes,
                    "cache_resident": True, "steps": steps})
        del pool, inputs
    return {
        "metric": "decode-step time on the GDN and KDA layer configurations (cache-resident)",
        "value": out[0]["state_updates_per_s"], "unit": "state-updates/s (GDN layer)",
        "n_gpus": 1, "steps": out[0]["steps"], "warmup": max(3, args.warmup),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "gdn_32h_b64_mixed + kda_32h_b256_mixed_prewarm (layers)"},
        "layers": out,
    }


PROFILE_DAMP = os.path.join(ROOT, "profiles", "k_damp_step_gdn_serving_1024x32.md")


def damp_algorithmic_bytes(n_unit: int, gate: int) -> int:
    """Bytes one DAMP-variant step must move per launch: binary16 channels, codes and
    key-row ranges read and written, q/k/v, a and b read, o written."""
    state = 128 * 16 * 2 + 128 * 112 + 112 * 4
    return n_unit * (2 * state + 3 * 512 + 4 * (128 if gate == 1 else 1) + 4 + 512)


def bench_damp(args, torch, qdr, wl, dev):
    """The DAMP-style storage variant (16 binary16 + 112 INT8 key channels per head,
    stochastic rounding) on the serving shape, one step per launch."""
    w = wl.WORKLOADS[3]
    sel = qdr.damp_select(w.gate, wl.halflives(w, args.seed), w.n_head)
    st = qdr.DampState(w.n_req, w.n_head, w.gate, sel, seed=args.seed, device=dev)
    a = torch.from_numpy(wl.static_gate(w, args.seed)).to(dev)
    n_in = 8
    inputs = [wl.device_step_inputs(w, t, dev, args.seed) for t in range(n_in)]
    o = torch.empty((w.n_req, w.n_head, 128), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for t in range(args.warmup):
        x = inputs[t % n_in]
        st.step(x["q"], x["k"], x["v"], a, x["b"], o, step=t, stream=stream)
    torch.cuda.synchronize()
    steps = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        x = inputs[i % n_in]
        ev[i][0].record(stream)
        st.step(x["q"], x["k"], x["v"], a, x["b"], o, step=args.warmup + i, stream=stream)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_s = float(np.mean([s_.elapsed_time(e_) for s_, e_ in ev])) / 1e3
    nbytes = damp_algorithmic_bytes(w.n_unit, w.gate)
    achieved = nbytes / kern_s / 1e9
    log(f"damp step: {kern_s * 1e6:.1f} us per launch; {achieved:.0f} GB/s algorithmic "
        f"({100 * achieved / HBM_PEAK_GBPS:.1f}% of 8 TB/s)")
    prof = profile_record(PROFILE_DAMP)
    traffic = float(prof["traffic_bytes_per_launch"]) if "traffic_bytes_per_launch" in prof else None
    return {
        "metric": "state-updates/s (req x head), DAMP-style variant, 1024-req GDN",
        "value": w.n_unit / (wall / steps), "unit": "state-updates/s",
        "n_gpus": 1, "steps": steps, "warmup": args.warmup, "ms_per_step": wall * 1e3 / steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name + " (damp)", "n_req": w.n_req, "n_head": w.n_head,
                   "bits": "16 binary16 + 112 INT8 (stochastic rounding) key channels per head"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": "k_damp_step<GDN>", "bytes_per_launch": nbytes,
                     "avg_launch_us": kern_s * 1e6},
        "cpu_baseline": None,
    }


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
                      f"{threads} host thread{'s' if threads > 1 else ''}, {dt:.2f} s wall"}


def host_threads() -> int:
    """Host threads for the multi-threaded baseline: the CPUs this process may run on,
    capped at 16 (one GPU's share of a shared GPU host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baselines(w, bits, args):
    """The oracle timed twice on the host: one thread over a small sample, and all usable
    host threads over the larger one. The multi-threaded figure is the reported value."""
    threads = host_threads()
    log(f"cpu baseline: oracle on 1 thread, {args.cpu1_requests} requests x "
        f"{args.cpu1_steps} steps")
    one = cpu_baseline(w, bits, 1, args.cpu1_requests, args.cpu1_steps)
    log(f"cpu baseline: oracle on {threads} threads, {args.cpu_requests} requests x "
        f"{args.cpu_steps} steps")
    many = cpu_baseline(w, bits, threads, args.cpu_requests, args.cpu_steps)
    many["nproc"] = os.cpu_count()
    many["single_thread"] = one
    return many


def probe_clock_mhz(torch, qdr, dev, iters=40000, n_block=None):
    """Engine clock: shader-clock cycles over constant-rate ticks while work-groups run a
    dependent fp32 fma chain. Default: 8 work-groups per CU (full VALU load); n_block=1
    samples the clock the chip is running at (one CU, about 15 us)."""
    if n_block is None:
        n_block = 8 * torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.zeros((n_block, 4), dtype=torch.int64, device=dev)
    qdr.probe_clock(out, iters)
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    return float(o[:, 0].sum() / o[:, 1].sum() * qdr.probe_wall_rate() / 1e6)


def clock_trace_summary(tr, wall_hz: float, kern_s: float) -> dict:
    """Engine clock from a clock trace ([n][2]: shader-clock counter, constant-rate
    counter): over the whole trace, its first and last fifth, and the lowest 0.5 ms
    window; coverage = trace span over the summed timed launch durations."""
    cyc = np.diff(tr[:, 0].astype(np.float64))
    tick = np.diff(tr[:, 1].astype(np.float64))
    mhz = lambda c, t: float(c.sum() / t.sum() * wall_hz / 1e6)
    n = len(cyc)
    f = max(1, n // 5)
    win = max(1, int(round(0.5e-3 * wall_hz / max(1.0, float(np.median(tick))))))
    lows = [mhz(cyc[i:i + win], tick[i:i + win]) for i in range(0, max(1, n - win + 1), win)]
    return {"mean": mhz(cyc, tick), "first_fifth": mhz(cyc[:f], tick[:f]),
            "last_fifth": mhz(cyc[-f:], tick[-f:]), "min_0p5ms": min(lows),
            "coverage": float(tick.sum() / wall_hz / kern_s), "samples": n + 1}


def probe_copy_gbps(torch, qdr, dev, nbytes: int, reps: int = 20):
    """Achievable HBM read+write bandwidth: a streaming copy of nbytes (read nbytes, write
    nbytes) on the probe kernel, mean over reps timed copies after two untimed ones."""
    n = (nbytes // 16) * 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        qdr.probe_copy(src, dst, stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for s_, e_ in ev:
        s_.record(stream)
        qdr.probe_copy(src, dst, stream)
        e_.record(stream)
    torch.cuda.synchronize()
    t = float(np.mean([s_.elapsed_time(e_) for s_, e_ in ev])) / 1e3
    del src, dst
    return 2.0 * n * 4 / t / 1e9


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    # untimed launches before the timed region; 50 decode steps (about 13 ms of work) let
    # the GPU clocks settle, so the timed launches measure the steady serving rate
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-requests", type=int, default=1024)
    ap.add_argument("--cpu-steps", type=int, default=24)
    ap.add_argument("--cpu1-requests", type=int, default=128)
    ap.add_argument("--cpu1-steps", type=int, default=8)
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the clock and copy-bandwidth probes")
    ap.add_argument("--workload",
                    choices=["serving", "window", "chunk", "comp", "compare", "damp", "layers"],
                    default="serving",
                    help="serving: the decode-step metric (default); window: window mode "
                         "(one call per token); chunk: chunk mode (one call per window); "
                         "comp: chunk mode with compensator tokens; "
                         "compare: the decode step under each scale rule; damp: the "
                         "DAMP-style storage variant; layers: the GDN and KDA layer "
                         "configurations (cache-resident working sets)")
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
    if args.workload == "window":
        print(json.dumps(bench_window(args, torch, qdr, wl, dev)), flush=True)
        return
    if args.workload == "chunk":
        print(json.dumps(bench_chunk(args, torch, qdr, wl, dev)), flush=True)
        return
    if args.workload == "comp":
        print(json.dumps(bench_chunk(args, torch, qdr, wl, dev, m=COMP_TOKENS)), flush=True)
        return
    if args.workload == "compare":
        print(json.dumps(bench_compare(args, torch, qdr, wl, dev)), flush=True)
        return
    if args.workload == "damp":
        print(json.dumps(bench_damp(args, torch, qdr, wl, dev)), flush=True)
        return
    if args.workload == "layers":
        print(json.dumps(bench_layers(args, torch, qdr, wl, dev)), flush=True)
        return
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

    wev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.warmup)]
    for t in range(args.warmup):
        wev[t][0].record(stream)
        launch(inputs[t])
        wev[t][1].record(stream)
    torch.cuda.synchronize()
    warm_us = [s_.elapsed_time(e_) * 1e3 for s_, e_ in wev]
    log(f"warmup done ({args.warmup} steps); timing {args.steps} steps")
    trace = mon = None
    if not args.no_probes:
        # the engine clock while the timed steps run: one sampling wave on a second stream
        # (it fits beside the step's three work-groups per CU and sleeps between samples),
        # sized to end within the timed region even if every timed launch is as fast as the
        # fastest warm-up launch
        wall_hz = qdr.probe_wall_rate()
        period = max(1, int(round(wall_hz * CLOCK_TRACE_PERIOD_S)))
        est_us = min(warm_us) if warm_us else 200.0
        n_sample = max(2, min(1 << 20, int(0.8 * est_us * args.steps * 1e-6 * wall_hz / period)))
        trace = torch.zeros((n_sample, 2), dtype=torch.int64, device=dev)
        mon = torch.cuda.Stream(device=dev)

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    if trace is not None:
        qdr.probe_clock_trace(trace, period, mon)
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
    probes = None
    if not args.no_probes:
        clock = clock_trace_summary(trace.cpu().numpy(), wall_hz, float(kern_ms.sum()) / 1e3)
        if clock["coverage"] > 1.0:
            log("warning: the clock trace outlasted the timed launches; wall time includes it")
        # the remaining probes run after the timed region, so they cannot change it
        clock_load = probe_clock_mhz(torch, qdr, dev)
        del inputs
        copy_gbps = probe_copy_gbps(torch, qdr, dev, nbytes // 2)
        probes = {"copy_gbps": copy_gbps, "frac_of_copy": achieved / copy_gbps,
                  "copy_bytes_each_way": (nbytes // 2 // 16) * 16,
                  "clock_mhz_timed": clock, "clock_mhz_full_valu_load": clock_load,
                  "warmup_launch_us": [round(x, 1) for x in warm_us]}
        log(f"probes: streaming copy {copy_gbps:.0f} GB/s (step at {100*achieved/copy_gbps:.1f}% "
            f"of it); engine clock during the timed steps {clock['mean']:.0f} MHz (first "
            f"fifth {clock['first_fifth']:.0f}, last fifth {clock['last_fifth']:.0f}, lowest "
            f"0.5 ms {clock['min_0p5ms']:.0f}) over {100*clock['coverage']:.0f}% of the timed "
            f"kernel time; {clock_load:.0f} MHz under full VALU load")

    prof = profile_record()
    traffic = float(prof["traffic_bytes_per_launch"]) if "traffic_bytes_per_launch" in prof else None
    valu = None
    if "SQ_INSTS_VALU" in prof:
        lane_ops = float(prof["SQ_INSTS_VALU"]) * 64
        valu = {"lane_ops_per_launch": lane_ops, "achieved": lane_ops / avg_kern_s,
                "peak": VALU_PEAK_LANE_OPS, "unit": "lane-ops/s",
                "frac": lane_ops / avg_kern_s / VALU_PEAK_LANE_OPS,
                "lane_ops_per_entry": lane_ops / (n_unit * 128 * 128)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baselines(w, bits, args)

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
                     "avg_launch_us": avg_kern_s * 1e6,
                     "median_launch_us": float(np.median(kern_ms)) * 1e3,
                     # what holds the kernel below this bound: the VALU issue of its exact
                     # arithmetic (the "valu" object), not HBM (calibrated traffic equals
                     # the algorithmic bytes)
                     "limiter": "valu-issue"},
        "probes": probes,
        "valu": valu,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
