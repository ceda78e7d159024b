"""Summarise rocprofv3 CSV output for one kernel (default: the decode step) as a short
markdown file.

Inputs (all written by rocprofv3 ``--output-format csv`` into one directory):
  <dir>/trace_kernel_stats.csv            --kernel-trace --stats of bench.py
  <dir>/fetch_counter_collection.csv      --pmc FETCH_SIZE of bench.py
  <dir>/write_counter_collection.csv      --pmc WRITE_SIZE of bench.py
  <dir>/cfetch_counter_collection.csv     --pmc FETCH_SIZE of copy_calibration.py
  <dir>/cwrite_counter_collection.csv     --pmc WRITE_SIZE of copy_calibration.py
  <dir>/p*_counter_collection.csv         optional extra counter passes of bench.py

HBM traffic per launch = FETCH_SIZE x f_fetch + WRITE_SIZE x f_write, where each
factor is (bytes the calibration copy really moves) / (what the counter reports for
it). The summary ends with machine-readable ``key: value`` lines that bench.py reads.
"""
import argparse
import csv
import hashlib
import os
import statistics
from collections import defaultdict

KIB = 1024.0


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def counters(path, match):
    """{counter: [value per dispatch]} for kernels whose name contains `match`."""
    out = defaultdict(list)
    for r in _rows(path):
        if match(r["Kernel_Name"]):
            out[r["Counter_Name"]].append(float(r["Counter_Value"]))
    return out


KERNELS = ("k_step<",)


def is_step(name):
    return any(k in name for k in KERNELS)


def is_copy(name):
    return "elementwise" in name and "MulFunctor" in name


def kernel_sources(kernels):
    """The source files whose code a summary of `kernels` (name fragments) depends on: the
    DAMP-style variant's kernels live in qdr_damp.hip, every other kernel in qdr_kernels.hip;
    both include qdr_internal.h."""
    main = "qdr_damp.hip" if "damp" in kernels else "qdr_kernels.hip"
    return (f"quantized_delta_rule_03_amd/csrc/{main}", "quantized_delta_rule_03_amd/csrc/qdr_internal.h")


def kernel_source_sha256(root, kernels="k_step<"):
    """Hash of the code of the sources that `kernels` are built from: line comments,
    trailing blanks and blank lines are left out, so a summary stays valid across
    comment-only edits and goes stale on any change to that code."""
    h = hashlib.sha256()
    for rel in kernel_sources(kernels):
        with open(os.path.join(root, rel), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode("utf-8") + b"\n")
    return h.hexdigest()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("dir")
    ap.add_argument("--copy-bytes", type=float, default=None,
                    help="bytes read (= bytes written) per calibration dispatch")
    ap.add_argument("--kernels", default="k_step<",
                    help="comma-separated kernel-name fragments to summarise")
    ap.add_argument("--cmd", action="append", default=[], help="command lines, for the record")
    ap.add_argument("--title", default="k_step, serving workload")
    ap.add_argument("--bench-log", default=None,
                    help="stderr of the traced bench run: its [bench] lines are quoted")
    ap.add_argument("--per-call", default=None,
                    help="kernel-name fragment whose dispatches mark one call of a multi-kernel "
                         "sequence (e.g. the fold ending each window): traffic is then also "
                         "given per call, all matched dispatches' bytes over that count")
    args = ap.parse_args()
    global KERNELS
    KERNELS = tuple(args.kernels.split(","))
    d = args.dir
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    label = " + ".join(k.rstrip("<") for k in KERNELS)

    lines = [f"# {args.title}", "", "Commands (run from the repository root):", ""]
    lines += [f"    {c}" for c in args.cmd]
    lines.append("")

    if args.bench_log:
        with open(args.bench_log) as f:
            quoted = [ln.rstrip() for ln in f if ln.startswith("[bench]")]
        if quoted:
            lines.append("Traced run, as bench.py reported it (HIP events on the launch stream):")
            lines.append("")
            lines += [f"    {ln}" for ln in quoted]
            lines.append("")
    stats = [r for r in _rows(os.path.join(d, "trace_kernel_stats.csv")) if is_step(r["Name"])]
    lines.append("## Kernel trace (rocprofv3 --kernel-trace --stats)")
    lines.append("")
    lines.append("| kernel | calls | avg us | min us | max us |")
    lines.append("|---|---|---|---|---|")
    avg_ns = None
    for r in stats:
        name = r["Name"].replace("qdr::(anonymous namespace)::", "").split("(")[0]
        avg_ns = float(r["AverageNs"])
        lines.append(f"| {name} | {r['Calls']} | {avg_ns / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    lines.append("")

    if not os.path.exists(os.path.join(d, "fetch_counter_collection.csv")):
        lines.append("## Machine-readable")
        lines.append("")
        lines.append(f"kernel_source_sha256: {kernel_source_sha256(root, args.kernels)}")
        print("\n".join(lines))
        return
    fetch = counters(os.path.join(d, "fetch_counter_collection.csv"), is_step)["FETCH_SIZE"]
    write = counters(os.path.join(d, "write_counter_collection.csv"), is_step)["WRITE_SIZE"]
    per_call = None
    if args.per_call:
        marks = lambda n: args.per_call in n
        n_calls = len(counters(os.path.join(d, "fetch_counter_collection.csv"), marks)["FETCH_SIZE"])
        per_call = (n_calls, sum(fetch), sum(write))
    cf = counters(os.path.join(d, "cfetch_counter_collection.csv"), is_copy)["FETCH_SIZE"]
    cw = counters(os.path.join(d, "cwrite_counter_collection.csv"), is_copy)["WRITE_SIZE"]
    f_fetch = args.copy_bytes / (statistics.mean(cf) * KIB)
    f_write = args.copy_bytes / (statistics.mean(cw) * KIB)
    fetch_b = statistics.mean(fetch) * KIB * f_fetch
    write_b = statistics.mean(write) * KIB * f_write
    lines.append("## HBM traffic (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE)")
    lines.append("")
    lines.append("| | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch |")
    lines.append("|---|---|---|")
    lines.append(f"| calibration copy ({args.copy_bytes / 2**20:.0f} MiB read + written) | "
                 f"{statistics.mean(cf):.0f} | {statistics.mean(cw):.0f} |")
    lines.append(f"| {label} (mean of {len(fetch)} / {len(write)} dispatches) | "
                 f"{statistics.mean(fetch):.0f} | {statistics.mean(write):.0f} |")
    lines.append("")
    lines.append(f"Scale factors (known bytes / counter bytes of the copy): fetch {f_fetch:.3f}, "
                 f"write {f_write:.3f}.")
    lines.append(f"{label} HBM traffic per launch: {fetch_b / 1e6:.1f} MB read + "
                 f"{write_b / 1e6:.1f} MB written = {(fetch_b + write_b) / 1e6:.1f} MB.")
    call_b = None
    if per_call:
        n_calls, fsum, wsum = per_call
        call_f = fsum * KIB * f_fetch / n_calls
        call_w = wsum * KIB * f_write / n_calls
        call_b = call_f + call_w
        lines.append(f"Per call ({n_calls} calls, each ending with one {args.per_call} "
                     f"dispatch; all {len(fetch)} dispatches counted): {call_f / 1e6:.1f} MB "
                     f"read + {call_w / 1e6:.1f} MB written = {call_b / 1e6:.1f} MB.")
    lines.append("")

    extra = sorted(f for f in os.listdir(d) if f.startswith("p") and f.endswith("_counter_collection.csv"))
    means = {}
    for f in extra:
        for name, vals in counters(os.path.join(d, f), is_step).items():
            means[name] = statistics.mean(vals)
    if means:
        lines.append(f"## Other counters (mean per {label} dispatch)")
        lines.append("")
        for name in sorted(means):
            lines.append(f"- {name}: {means[name]:.4g}")
        lines.append("")

    lines.append("## Machine-readable")
    lines.append("")
    if avg_ns is not None:
        lines.append(f"avg_launch_ns: {avg_ns:.0f}")
    lines.append(f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}")
    if call_b is not None:
        lines.append(f"traffic_bytes_per_call: {call_b:.0f}")
    lines.append(f"fetch_scale: {f_fetch:.4f}")
    lines.append(f"write_scale: {f_write:.4f}")
    for name in sorted(means):
        lines.append(f"{name}: {means[name]:.0f}")
    lines.append(f"kernel_source_sha256: {kernel_source_sha256(root, args.kernels)}")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
