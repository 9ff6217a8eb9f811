"""HBM bandwidth sweep: triad, copy, read-only and write-only kernels.

    python -m transformer_attention_micro_amd.hbm [--sizes-mib 64 256 1024 2048 4096]
                                                  [--blocks 64 128 256 512 1024] [--iters 50]
    python -m transformer_attention_micro_amd.hbm --calibrate [--profile-out mi355x.json]

The TileOPs benchmarks/hardware page ("HBM Bandwidth", "Methodology")
measures the triad a[i] = b[i] + s c[i] next to copy, read-only and
write-only kernels with 128-bit accesses, sweeps the working-set size and
the block size, and reports the best bandwidth over the block sweep.  This
does the same on one MI355X through kb_bench_triad / kb_bench_stream: for
each kind and working set (the total size of the arrays the kernel touches)
it prints the best GB/s over the block sizes and the block that gave it.
Working sets below the 256 MB Infinity Cache are served partly from it.

--calibrate runs the page's calibration protocol ("Methodology"): a 2 GB
working set, 100 warmup launches per configuration, then 200 launches x 5
runs, best and median reported, the calibration being the best triad
bandwidth over the block sweep divided by the datasheet figure ("Output",
"Adding a new GPU profile").  --profile-out writes the device profile: the
datasheet ceilings this library measures against and the measured
calibration (clocks are not locked here: that needs root).
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
    ap.add_argument("--calibrate", action="store_true",
                    help="run the calibration protocol (2 GB, 100 warmup, 200 x 5 runs, best and median)")
    ap.add_argument("--profile-out", default=None, help="with --calibrate: write the device profile JSON here")
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


# MI355X datasheet figures (the ceilings every fraction in this package is
# taken against).
MI355X = {
    "name": "mi355x", "arch": "gfx950", "compute_units": 256, "xcds": 8, "peak_sclk_mhz": 2400,
    "hbm_gbs": 8000.0, "hbm_capacity_gb": 288, "lds_per_cu_kib": 160, "l2_per_xcd_mb": 4,
    "infinity_cache_mb": 256,
    "mfma_dense_tflops": {"bf16": 2516.6, "fp16": 2516.6, "fp8": 5033.2, "fp32": 157.3, "fp64": 78.6},
    "vector_fp32_tflops": 157.3,
}


def protocol(fn, nbytes, warmup=100, runs=5, iters=200):
    """The page's timing protocol for one configuration: `warmup` untimed
    launches, then `runs` runs of `iters` timed launches; `fn(warmup, iters)`
    returns the per-launch times (ms).  Returns the best and the median over
    the runs of each run's mean bandwidth."""
    per_run = []
    for r in range(runs):
        per = fn(warmup if r == 0 else 0, iters)
        per_run.append(nbytes / (float(np.mean(per)) * 1e-3) / 1e9)
    return {"best_gbs": round(max(per_run), 1), "median_gbs": round(float(np.median(per_run)), 1),
            "runs_gbs": [round(x, 1) for x in per_run]}


def calibrate(kb, torch, stream, mib=2048, blocks=(64, 128, 256, 512, 1024), warmup=100, runs=5, iters=200,
              kinds=("triad", "copy", "read", "write")):
    """Every kind at a `mib` MiB working set over the block sweep with the
    protocol above; the calibration is the best triad bandwidth over the
    blocks divided by the datasheet HBM figure."""
    out = {"working_set_mib": mib, "protocol": {"warmup": warmup, "runs": runs, "iters": iters},
           "blocks": list(blocks)}
    for kind in kinds:
        n = (mib << 20) // (4 * ARRAYS[kind])
        n -= n % 4
        a = torch.empty(n, dtype=torch.float32, device="cuda")
        b = torch.rand(n, dtype=torch.float32, device="cuda")
        c = torch.rand(n, dtype=torch.float32, device="cuda") if kind == "triad" else None
        rows = {}
        for block in blocks:
            if kind == "triad":
                fn = lambda w, it: kb.kb_bench_triad(a.data_ptr(), b.data_ptr(), c.data_ptr(), 1.5, n, block,
                                                     stream, w, it)[0]
            else:
                s = float("nan") if kind == "read" else 1.5
                fn = lambda w, it: kb.kb_bench_stream(kind, a.data_ptr(), b.data_ptr(), s, n, block, stream, w,
                                                      it)[0]
            rows[block] = protocol(fn, kb.STREAM_BYTES[kind] * n, warmup, runs, iters)
        best_block = max(rows, key=lambda k: rows[k]["best_gbs"])
        out[kind] = {"bytes_per_launch": kb.STREAM_BYTES[kind] * n, "best_block": best_block,
                     "best_gbs": rows[best_block]["best_gbs"], "median_gbs": rows[best_block]["median_gbs"],
                     "per_block": {str(k): v for k, v in rows.items()}}
        del a, b, c
        torch.cuda.empty_cache()
    out["calibration"] = round(out["triad"]["best_gbs"] / MI355X["hbm_gbs"], 4)
    return out


def profile(cal, device):
    """The device profile: datasheet ceilings plus the measured calibration."""
    return {"gpu": MI355X["name"], "theoretical": MI355X, "device": device,
            "hbm": {"calibration": cal["calibration"], "measured_triad_gbs": cal["triad"]["best_gbs"],
                    "measured_triad_median_gbs": cal["triad"]["median_gbs"], "triad_block": cal["triad"]["best_block"],
                    "working_set_mib": cal["working_set_mib"], "protocol": cal["protocol"],
                    "reference_kernels_gbs": {k: cal[k]["best_gbs"] for k in ("copy", "read", "write") if k in cal}},
            "clocks_locked": False,
            "command": "python -m transformer_attention_micro_amd.hbm --calibrate --profile-out <file>"}


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
    if args.calibrate:
        cal = calibrate(kb, torch, stream, blocks=tuple(args.blocks))
        t = cal["triad"]
        print(f"Measured peak (triad vec4): {t['best_gbs']:.2f} GB/s (block {t['best_block']}, "
              f"median of runs {t['median_gbs']:.2f})")
        print(f"Theoretical: {MI355X['hbm_gbs']:.1f} GB/s")
        print(f"Calibration: {cal['calibration']:.4f}")
        for k in ("copy", "read", "write"):
            print(f"  {k}: best {cal[k]['best_gbs']:.1f} GB/s (block {cal[k]['best_block']}), "
                  f"median {cal[k]['median_gbs']:.1f}")
        if args.profile_out:
            with open(args.profile_out, "w") as f:
                json.dump(profile(cal, kb.kb_device_info()), f, indent=1)
                f.write("\n")
            print(f"wrote {args.profile_out} (hbm.calibration: {cal['calibration']:.4f})")
        return 0
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
