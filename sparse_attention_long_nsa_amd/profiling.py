"""Profiling helpers: a plain device copy of known size, used to calibrate
rocprofv3's memory counters (FETCH_SIZE / WRITE_SIZE) before they are read
for the layer's kernels.

  python -m sparse_attention_long_nsa_amd.profiling copy --mib 1024 --reps 3
"""
from __future__ import annotations

import argparse
import sys


def copy_probe(mib: int, reps: int) -> None:
    import torch
    n = mib * 1024 * 1024 // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB x {reps}: each dispatch reads {mib * 1024} KiB and writes {mib * 1024} KiB",
          flush=True)


def main(argv=None) -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=3)
    a = ap.parse_args(argv)
    if a.cmd == "copy":
        copy_probe(a.mib, a.reps)


if __name__ == "__main__":
    main(sys.argv[1:])
