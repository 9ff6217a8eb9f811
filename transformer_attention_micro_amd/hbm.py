"""HBM bandwidth sweep: triad, copy, read-only and write-only kernels.

    python -m transformer_attention_micro_amd.hbm [--sizes-mib 64 256 1024 2048 4096]
                                                  [--blocks 64 128 256 512 1024] [--iters 50]

The TileOPs benchmarks/hardware page ("HBM Bandwidth", "Methodology")
measures the triad a[i] = b[i] + s c[i] next to copy, read-only and
write-only kernels with 128-bit accesses, sweeps the working-set size and
the block size, and reports the best bandwidth over the block sweep.  This
does the same on one MI355X through kb_bench_triad / kb_bench_stream: for
each kind and working set (the total size of the arrays the kernel touches)
it prints the best GB/s over the block sizes and the block that gave it.
Working sets below the 256 MB Infinity Cache are served partly from it.
"""
from __future__ import annotations

import argparse
import json
import sys

import numpy as np

ARRAYS = {"triad": 3, "copy": 2, "read": 1, "write": 1}  # arrays each kind touches


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--sizes-mib", type=int, nargs="+", default=[64, 256, 1024, 2048, 4096])
    ap.add_argument("--blocks", type=int, nargs="+", default=[64, 128, 256, 512, 1024])
    ap.add_argument("--iters", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--json", action="store_true", help="also print one JSON line per row")
    return ap.parse_args(argv)


def best_gbs(kb, torch, kind, mib, blocks, stream, warmup, iters):
    """Best GB/s over `blocks` for `kind` with a `mib` MiB working set."""
    n = (mib << 20) // (4 * ARRAYS[kind])
    n -= n % 4
    a = torch.empty(n, dtype=torch.float32, device="cuda")
    b = torch.rand(n, dtype=torch.float32, device="cuda")
    c = torch.rand(n, dtype=torch.float32, device="cuda") if kind == "triad" else None
    best = (0.0, 0)
    for block in blocks:
        if kind == "triad":
            per, _ = kb.kb_bench_triad(a.data_ptr(), b.data_ptr(), c.data_ptr(), 1.5, n, block, stream, warmup,
                                       iters)
        else:
            s = float("nan") if kind == "read" else 1.5
            per, _ = kb.kb_bench_stream(kind, a.data_ptr(), b.data_ptr(), s, n, block, stream, warmup, iters)
        gbs = kb.STREAM_BYTES[kind] * n / (float(np.median(per)) * 1e-3) / 1e9
        if gbs > best[0]:
            best = (gbs, block)
    del a, b, c
    torch.cuda.empty_cache()
    return best


def main(argv=None) -> int:
    args = parse(argv)
    import torch

    import transformer_attention_micro_amd as kb

    if not torch.cuda.is_available():
        print("the sweep needs a GPU", file=sys.stderr)
        return 1
    kb.lib()
    torch.cuda.set_device(0)
    stream = int(torch.cuda.current_stream().cuda_stream)
    rows = []
    for mib in args.sizes_mib:
        row = {"working_set_mib": mib}
        for kind in ARRAYS:
            gbs, block = best_gbs(kb, torch, kind, mib, args.blocks, stream, args.warmup, args.iters)
            row[kind] = {"gbs": round(gbs, 1), "block": block}
        rows.append(row)
    print(f"best over blocks {args.blocks}, median of {args.iters} launches; GB/s (block)")
    print()
    print("| working set (MiB) | triad | copy | read | write |")
    print("|---|---|---|---|---|")
    for r in rows:
        cells = " | ".join(f"{r[k]['gbs']:.0f} ({r[k]['block']})" for k in ARRAYS)
        print(f"| {r['working_set_mib']} | {cells} |")
    if args.json:
        for r in rows:
            print(json.dumps(r))
    return 0


if __name__ == "__main__":
    sys.exit(main())
