"""Sequence-length sweep of the three variants (the kbench page's study).

    python -m transformer_attention_micro_amd.sweep [--dtype f32|bf16] [--causal]
                                                    [--seqs 128 256 ... 32768] [--budget-ms 400]
                                                    [--heads 16] [--dim 64] [--iters 20]

The kbench page ("Running", "Expected results") sweeps the sequence length at
16 heads and head dimension 64 and compares the naive, fused and flash
kernels by relative latency (naive = 1.0) and by where each sits on the
roofline: naive streams the S x S scores through DRAM and stays near the
bandwidth ceiling, flash keeps them on chip and climbs toward the compute
ceiling as S grows.  This runs that sweep on one MI355X with the same
seeded inputs as the tests and prints one Markdown table (and, with --json,
one JSON line per row).

Per row: median hipEvent time per launch of each variant, its algorithmic
TFLOP/s (4 d per visible query/key pair), naive's algorithmic HBM GB/s
(Q, K, V read, O written, plus 16 bytes per score: written, read and
rewritten by the softmax, read by P V), flash's compulsory GB/s, and the
latency of fused and flash relative to naive.  Each variant gets as many
timed launches as fit in about --budget-ms (at least 3, at most --iters).

Below the table, the reading the page's "Expected results" asks for: the
relative latencies at S = 2048 beside the page's 1.0x / ~2.2x / ~4.7x, the
first S at which naive's algorithmic bandwidth reaches 90 % of the triad
measured in the same run (its DRAM ceiling), and the S at which flash's
compulsory bandwidth peaks, i.e. from where on it falls while its TFLOP/s
keep rising.
"""
from __future__ import annotations

import argparse
import json
import sys

import numpy as np


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--dtype", choices=("f32", "bf16"), default="f32")
    ap.add_argument("--causal", action="store_true")
    ap.add_argument("--seqs", type=int, nargs="+",
                    default=[128, 256, 512, 1024, 2048, 4096, 8192, 16384, 32768])
    ap.add_argument("--budget-ms", type=float, default=400.0, help="timed launches per variant and S")
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--heads", type=int, default=16)
    ap.add_argument("--dim", type=int, default=64)
    ap.add_argument("--iters", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--json", action="store_true", help="also print one JSON line per row")
    return ap.parse_args(argv)


def main(argv=None) -> int:
    args = parse(argv)
    import torch

    import transformer_attention_micro_amd as kb
    from transformer_attention_micro_amd import inputs

    if not torch.cuda.is_available():
        print("the sweep needs a GPU", file=sys.stderr)
        return 1
    kb.lib()
    torch.cuda.set_device(0)
    stream = int(torch.cuda.current_stream().cuda_stream)
    dt = kb.KB_BF16 if args.dtype == "bf16" else kb.KB_F32
    esize = 2 if args.dtype == "bf16" else 4
    rows = []
    for S in args.seqs:
        p = inputs.make_problem(args.batch, args.heads, S, args.dim, args.dtype, causal=args.causal, seed=S)
        dev = []
        for a in p.device_arrays():
            t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16) \
                if a.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(a))
            dev.append(t.cuda())
        o = torch.empty((p.BH, S, args.dim), dtype=torch.float32, device="cuda")
        ptrs = (dev[0].data_ptr(), dev[1].data_ptr(), dev[2].data_ptr(), o.data_ptr())
        cfg = kb.make_cfg(p.B, p.H, S, args.dim, args.causal, dt)
        ws = torch.empty(kb.kb_attention_workspace_size(cfg, "naive"), dtype=torch.uint8, device="cuda")
        ncfg = kb.make_cfg(p.B, p.H, S, args.dim, args.causal, dt, 0.0, ws.data_ptr(), ws.numel())
        flops = kb.attention_flops(p.B, p.H, S, args.dim, args.causal)
        comp = kb.attention_bytes(p.B, p.H, S, args.dim, esize)
        ms = {}
        for name, c in (("naive", ncfg), ("fused", cfg), ("flash", cfg)):
            first, _ = kb.kb_bench_attention(c, *ptrs, name, stream, 1, 1)
            iters = int(min(args.iters, max(3, args.budget_ms / max(first[0], 1e-3))))
            per, _ = kb.kb_bench_attention(c, *ptrs, name, stream, args.warmup if iters > 3 else 0, iters)
            ms[name] = float(np.median(per))
        print(f"[sweep] S={S}: naive {ms['naive']:.4f} fused {ms['fused']:.4f} flash {ms['flash']:.4f} ms",
              file=sys.stderr, flush=True)
        row = {"B": p.B, "H": p.H, "S": S, "d": args.dim, "dtype": args.dtype, "causal": args.causal}
        for name in ("naive", "fused", "flash"):
            row[f"{name}_ms"] = round(ms[name], 5)
            row[f"{name}_tflops"] = round(flops / (ms[name] * 1e-3) / 1e12, 3)
        row["naive_hbm_gbs_algorithmic"] = round((comp + 16 * p.BH * S * S) / (ms["naive"] * 1e-3) / 1e9, 1)
        row["flash_hbm_gbs_compulsory"] = round(comp / (ms["flash"] * 1e-3) / 1e9, 1)
        row["fused_speedup_vs_naive"] = round(ms["naive"] / ms["fused"], 2)
        row["flash_speedup_vs_naive"] = round(ms["naive"] / ms["flash"], 2)
        rows.append(row)
        del dev, o, ws
        torch.cuda.empty_cache()

    from transformer_attention_micro_amd.hbm import best_gbs
    triad, _ = best_gbs(kb, torch, "triad", 2048, (64, 256, 1024), stream, 20, 50)
    mask = "causal" if args.causal else "non-causal"
    print(f"B={args.batch} H={args.heads} d={args.dim} {args.dtype} {mask}; median of 3 to {args.iters} launches "
          f"(as many as fit in ~{args.budget_ms:.0f} ms)")
    print()
    print("| S | naive ms | fused ms | flash ms | naive TFLOP/s | fused TFLOP/s | flash TFLOP/s | "
          "naive GB/s (algorithmic) | flash GB/s (compulsory) | fused vs naive | flash vs naive |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['S']} | {r['naive_ms']:.4f} | {r['fused_ms']:.4f} | {r['flash_ms']:.4f} | "
              f"{r['naive_tflops']:.2f} | {r['fused_tflops']:.2f} | {r['flash_tflops']:.2f} | "
              f"{r['naive_hbm_gbs_algorithmic']:.0f} | {r['flash_hbm_gbs_compulsory']:.0f} | "
              f"{r['fused_speedup_vs_naive']:.2f}x | {r['flash_speedup_vs_naive']:.2f}x |")
    print()
    print(reading(rows, triad))
    if args.json:
        for r in rows:
            print(json.dumps(r))
    return 0


def reading(rows, triad_gbs):
    """The page's expected-results reading of a sweep (rows sorted by S)."""
    out = [f"Triad (same run, 2 GiB, best of blocks 64/256/1024): {triad_gbs:.0f} GB/s."]
    at = {r["S"]: r for r in rows}
    if 2048 in at:
        r = at[2048]
        out.append(f"Relative latency at S=2048 (naive = 1.0x): fused {r['fused_speedup_vs_naive']:.2f}x, "
                   f"flash {r['flash_speedup_vs_naive']:.2f}x faster (the page: ~2.2x and ~4.7x).")
    pinned = [r["S"] for r in rows if r["naive_hbm_gbs_algorithmic"] >= 0.9 * triad_gbs]
    out.append("naive reaches 90% of the triad from S=" + str(pinned[0]) if pinned else
               "naive stays below 90% of the triad at every S of the sweep (best "
               f"{max(r['naive_hbm_gbs_algorithmic'] for r in rows) / triad_gbs:.2f} of it).")
    if rows:
        peak = max(rows, key=lambda r: r["flash_hbm_gbs_compulsory"])
        later = [r for r in rows if r["S"] > peak["S"]]
        if later:
            out.append(f"flash's compulsory bandwidth peaks at S={peak['S']} ({peak['flash_hbm_gbs_compulsory']:.0f} "
                       f"GB/s) and falls after it (to {later[-1]['flash_hbm_gbs_compulsory']:.0f} GB/s at "
                       f"S={later[-1]['S']}) while its TFLOP/s go from {peak['flash_tflops']:.1f} to "
                       f"{later[-1]['flash_tflops']:.1f}.")
        else:
            out.append(f"flash's compulsory bandwidth still rises at the largest S ({peak['S']}).")
    return "\n".join(out)


if __name__ == "__main__":
    sys.exit(main())
