"""A plain device copy of known size, run under rocprofv3 --pmc to calibrate
the FETCH_SIZE / WRITE_SIZE counters (bytes the counters report for a copy
that moves exactly N bytes each way).

    python -m block_diffusion_decoding_attn_amd.copy_probe [MiB] [reps]
"""
import sys

import torch


def main():
    mib = int(sys.argv[1]) if len(sys.argv) > 1 else 1024
    reps = int(sys.argv[2]) if len(sys.argv) > 2 else 4
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB x {reps}", flush=True)


if __name__ == "__main__":
    main()
