"""Counter calibration workload: a plain HBM-to-HBM copy of known size.

Run under ``rocprofv3 --pmc FETCH_SIZE`` (and separately ``WRITE_SIZE``): one
elementwise kernel reads ``--mib`` MiB and writes the same amount, on every CU. The
ratio of the known byte count to what each counter reports for that kernel is the
scale applied to the same counter on the decode-step kernel (see
``rocprof_summary.py``).
"""
import argparse

import torch


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=1024)
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args()
    n = args.mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.reps):
        torch.mul(src, 1.0, out=dst)  # one elementwise kernel: n*4 bytes read, n*4 written
    torch.cuda.synchronize()
    print(f"copy_calibration: {args.reps} x {n * 4} bytes read and written", flush=True)


if __name__ == "__main__":
    main()
