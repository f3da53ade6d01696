"""Calibration run for HBM traffic counters: a plain device-to-device copy
of a known size (torch's copy kernel), repeated a few times.

    python -m consumer_gemm_chain_amd.copy_probe [MiB] [repeats]

Under ``rocprofv3 --pmc FETCH_SIZE`` (then ``WRITE_SIZE``) each copy
dispatch should read and write MiB mebibytes; the ratio of that size to
what the counter reports is the factor that turns the counter readings of
the chain's kernels into bytes.
"""
from __future__ import annotations

import sys


def main() -> None:
    import torch
    mib = int(sys.argv[1]) if len(sys.argv) > 1 else 1024
    reps = int(sys.argv[2]) if len(sys.argv) > 2 else 3
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB x {reps}")


if __name__ == "__main__":
    main()
