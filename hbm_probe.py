"""Plain device-to-device copy of a known size, for calibrating HBM byte counters.

    python hbm_probe.py [MiB] [repeats]

Copies a MiB-sized buffer `repeats` times with torch's copy kernel; a
rocprofv3 --pmc run over it gives FETCH_SIZE / WRITE_SIZE per dispatch for
exactly MiB MiB read and written, the scale used to turn the same counters on
the scoring kernels into bytes.
"""
import sys

import torch


def main():
    mib = int(sys.argv[1]) if len(sys.argv) > 1 else 256
    reps = int(sys.argv[2]) if len(sys.argv) > 2 else 5
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB x {reps}", flush=True)


if __name__ == "__main__":
    main()
