"""Benchmark: SDPA forward throughput of attn_flash on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one attention forward pass (kb_attention, variant flash) over the
workload B=2, H=32, S=8192, d=128, bf16 inputs, causal mask, fp32 output,
with Q, K, V already resident in HBM.  The default warmup (200 launches,
~0.2 s) outlasts the clock transient of an MI355X coming out of idle (a few
fast launches, a dip of up to ~30 %, then ~0.1 s of recovery), so the timed
steps measure sustained throughput.  The K timed steps are bracketed by
torch.cuda.synchronize() on both sides; inside, kb_bench_attention records a
hipEvent between consecutive launches on the launch stream, which gives the
per-launch kernel time used for the roofline fraction.

The JSON line also carries:
  roofline      achieved TFLOP/s per launch vs the MI355X dense bf16 MFMA
                peak (2516.6 TFLOP/s), and HBM bytes per launch from the
                rocprofv3 FETCH_SIZE / WRITE_SIZE summary committed under
                profiles/ (null if the kernel changed since it was taken);
  cpu_baseline  the fp64 oracle timed on this host's cores on a bounded,
                seeded sample of the same workload's query rows (also used
                to check the GPU output on those rows); small_configs: the
                oracle on every row of each workload with S <= 2048, on all
                threads and on one, beside the GPU's time and its error;
  triad         the HBM triad calibration (best of a block-size sweep);
  hbm_reference copy, read-only and write-only kernels at the same 2 GiB
                working set (best of the same sweep);
  variants      naive and fused on the same workload (a few timed calls);
  per_config    flash on every configured workload (the metric is quoted per
                (B, H, S, d), causal or not), each warmed up for ~0.3 s:
                mean hipEvent time per launch, TFLOP/s and the fraction of
                the dtype's MFMA peak;
  ceilings      sustained compute ceilings (kb_bench_ceiling: bf16 and fp32
                MFMA, fp32 FMA, exp) with the shader clock the probe ran at,
                the compute analogue of the triad.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SDPA forward TFLOP/s + % of MFMA peak per (B,H,S,d), causal/non-causal"
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}  # MI355X dense MFMA
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="b2h32s8192d128_bf16_causal")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-extras", action="store_true", help="skip triad and the naive/fused variants")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the flash table over every configured workload")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the compute-ceiling probes")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed steps, run a plain device copy of this many MiB three times "
                         "(a kernel of known traffic, used to scale the rocprofv3 byte counters)")
    ap.add_argument("--traffic-kib", type=float, nargs=2, metavar=("FETCH", "WRITE"), default=None,
                    help="rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the flash kernel, "
                         "already scaled by the copy-kernel calibration")
    return ap.parse_args()


def device_tensors(p, torch):
    out = []
    for a in p.device_arrays():
        if a.dtype == np.uint16:
            out.append(torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda())
        else:
            out.append(torch.from_numpy(a).cuda())
    return out


def cpu_baseline(p, o_gpu, budget_s, seed=1234):
    """Time the fp64 oracle on distinct seeded query rows (a random order of
    all rows, taken in growing chunks) until ~budget_s seconds."""
    import oracle
    rng = np.random.default_rng(seed)
    order = rng.permutation(p.BH * p.S).astype(np.int64)
    nthreads = oracle.default_threads()
    flops = 0
    rows_done = []
    errs = []
    t_used = 0.0
    chunk = 256
    pos = 0
    while t_used < budget_s and pos < order.size:
        rows = order[pos:pos + chunk]
        pos += rows.size
        t0 = time.perf_counter()
        ref = oracle.sdpa(p.q, p.k, p.v, causal=p.causal, rows=rows, nthreads=nthreads)
        t_used += time.perf_counter() - t0
        i = rows % p.S
        vis = (i + 1) if p.causal else np.full_like(i, p.S)
        flops += int(4 * p.d * vis.sum())
        rows_done.append(rows)
        errs.append(float(np.max(np.abs(o_gpu[rows] - ref))))
        if t_used > 0.5 * budget_s and chunk < 4096:
            chunk *= 2
    n = int(sum(len(r) for r in rows_done))
    return {
        "value": flops / t_used / 1e12,
        "unit": "TFLOP/s",
        "cores": nthreads,
        "kind": "oracle",
        "sample": f"{n} distinct seeded query rows (of {p.BH * p.S}) of the same workload, fp64, "
                  f"{t_used:.1f} s; throughput scaled by the rows' algorithmic FLOPs",
        "max_abs_err_vs_gpu_on_sample": max(errs),
    }


def cpu_small_configs(kb, torch, inputs, stream):
    """The fp64 oracle on every row of the small workloads (S <= 2048), with
    all the host threads and with one, beside one flash launch on the GPU of
    the same inputs: oracle time, its FLOP rate, the GPU's kernel time and
    speed-up, and the max-abs and relative-L2 error of the GPU output."""
    import oracle
    out = []
    for name, spec in inputs.WORKLOADS.items():
        if spec["S"] > 2048:
            continue
        p = inputs.workload(name)
        q, k, v = device_tensors(p, torch)
        o = torch.empty((p.BH, p.S, p.d), dtype=torch.float32, device="cuda")
        dt = kb.KB_BF16 if p.dtype == inputs.BF16 else kb.KB_F32
        cfg = kb.make_cfg(p.B, p.H, p.S, p.d, p.causal, dt)
        per, _ = kb.kb_bench_attention(cfg, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), "flash",
                                       stream, 20, 20)
        got = o.cpu().numpy().astype(np.float64)
        flops = kb.attention_flops(p.B, p.H, p.S, p.d, p.causal)
        row = {"workload": name, "gpu_kernel_ms_median": round(float(np.median(per)), 4)}
        for label, nt in (("all_threads", oracle.default_threads()), ("one_thread", 1)):
            t0 = time.perf_counter()
            ref = oracle.sdpa(p.q, p.k, p.v, causal=p.causal, nthreads=nt)
            sec = time.perf_counter() - t0
            row[label] = {"threads": nt, "seconds": round(sec, 4), "gflops": round(flops / sec / 1e9, 2)}
        row["gpu_speedup_vs_all_threads"] = round(row["all_threads"]["seconds"] * 1e3 / row["gpu_kernel_ms_median"], 1)
        row["max_abs_err"] = float(np.max(np.abs(got - ref)))
        row["rel_l2_err"] = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        out.append(row)
        del q, k, v, o
        torch.cuda.empty_cache()
    return out


def per_config_table(kb, torch, inputs, stream, cache, iters=20, warm_ms=300.0):
    """Flash on every configured workload (seeded inputs per the recipe; the
    S=8192 workload also without the mask), each warmed up for at least
    warm_ms so the row is not measured inside a clock transient."""
    rows = []
    for name in inputs.WORKLOADS:
        p = cache[name] if name in cache else inputs.workload(name)
        q, k, v = device_tensors(p, torch)
        o = torch.empty((p.BH, p.S, p.d), dtype=torch.float32, device="cuda")
        dt = kb.KB_BF16 if p.dtype == inputs.BF16 else kb.KB_F32
        for causal in ([True, False] if name == "b2h32s8192d128_bf16_causal" else [p.causal]):
            cfg = kb.make_cfg(p.B, p.H, p.S, p.d, causal, dt)
            ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr())
            first, _ = kb.kb_bench_attention(cfg, *ptrs, "flash", stream, 0, 1)
            warm = max(3, int(np.ceil(warm_ms / max(first[0], 1e-3))))
            per, _ = kb.kb_bench_attention(cfg, *ptrs, "flash", stream, warm, iters)
            ms = float(np.mean(per))
            fl = kb.attention_flops(p.B, p.H, p.S, p.d, causal)
            tf = fl / (ms * 1e-3) / 1e12
            rows.append({"workload": name, "B": p.B, "H": p.H, "S": p.S, "d": p.d, "causal": causal,
                         "dtype": p.dtype, "kernel_ms_mean": round(ms, 4), "tflops": round(tf, 2),
                         "frac_of_peak": round(tf / PEAK_TFLOPS[p.dtype], 4)})
        del q, k, v, o
        torch.cuda.empty_cache()
    return rows


# Datasheet peaks the ceilings are compared with (TFLOP/s; the fp32 vector
# figure counts packed FMA, which the probe does not use, so its non-packed
# bound is half of it) and the work per clock per CU of each probe.
CEIL_PEAK = {"mfma_bf16": 2516.6, "mfma_f32": 157.3, "fma_f32": 157.3 / 2, "exp_f32": None, "mfma_bf16_data": 2516.6}
CEIL_PER_CLK_CU = {"mfma_bf16": 4096, "mfma_f32": 256, "fma_f32": 128, "exp_f32": None, "mfma_bf16_data": 4096}
CEIL_MEMORY = ("lds_read", "l1_read", "l2_read")  # read-bandwidth probes, bytes per launch


def ceilings(kb, torch, stream, target_ms=40.0):
    """Each probe sized to ~target_ms per launch, one warmup launch (so the
    clock settles under load), then three timed ones."""
    work = torch.empty(kb.kb_ceiling_work_size(), dtype=torch.uint8, device="cuda")
    cus = kb.kb_device_info()["compute_units"]
    out = {}
    for kind in kb.CEILINGS:
        per, _, _ = kb.kb_bench_ceiling(kind, 2000, work.data_ptr(), work.numel(), stream, 1, 1)
        iters = max(1, int(2000 * target_ms / max(per[0], 1e-3)))
        per, ops, mhz = kb.kb_bench_ceiling(kind, iters, work.data_ptr(), work.numel(), stream, 1, 3)
        ms = float(np.median(per))
        if kind in CEIL_MEMORY:
            gbs = ops / (ms * 1e-3) / 1e9
            row = {"unit": "GB/s", "value": round(gbs, 1), "clock_mhz": round(mhz, 0), "ms_per_launch": round(ms, 3),
                   "iters": iters}
            if mhz > 0:
                row["bytes_per_clk_per_cu"] = round(gbs * 1e9 / (cus * mhz * 1e6), 1)
            out[kind] = row
            continue
        rate = ops / (ms * 1e-3) / 1e12
        row = {"unit": "Texp/s" if kind == "exp_f32" else "TFLOP/s", "value": round(rate, 2),
               "clock_mhz": round(mhz, 0), "ms_per_launch": round(ms, 3), "iters": iters}
        if CEIL_PEAK[kind]:
            row["frac_of_datasheet_peak"] = round(rate / CEIL_PEAK[kind], 4)
        if CEIL_PER_CLK_CU[kind] and mhz > 0:
            row["peak_at_measured_clock"] = round(CEIL_PER_CLK_CU[kind] * cus * mhz * 1e6 / 1e12, 1)
        out[kind] = row
    del work
    return out


def measured_traffic(workload):
    """HBM bytes per flash launch from the committed rocprofv3 counter summary,
    or None when there is none for this workload or the kernel source changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"flash_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(ROOT, rec["source"])
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if not sha.startswith(rec["source_sha256_prefix"]):
        return None
    return int(rec["hbm_bytes_per_launch"])


def triad_calibration(kb, torch, stream):
    n = 2048 * 1024 * 1024 // 12  # 2048 MiB working set over a, b, c
    n -= n % 4
    a = torch.empty(n, dtype=torch.float32, device="cuda")
    b = torch.rand(n, dtype=torch.float32, device="cuda")
    c = torch.rand(n, dtype=torch.float32, device="cuda")
    best = None
    for block in (64, 128, 256, 512, 1024):
        per, _ = kb.kb_bench_triad(a.data_ptr(), b.data_ptr(), c.data_ptr(), 1.5, n, block, stream, 20, 50)
        ms = float(np.median(per))
        gbs = 12.0 * n / (ms * 1e-3) / 1e9
        if best is None or gbs > best["gbs"]:
            best = {"gbs": gbs, "block": block, "median_ms": ms}
    del a, b, c
    torch.cuda.empty_cache()
    return {"best_gbs": round(best["gbs"], 1), "block": best["block"], "bytes": 12 * n,
            "calibration_vs_8000": round(best["gbs"] / HBM_PEAK_GBS, 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this library has no "
              f"multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        return 2
    import torch

    import transformer_attention_micro_amd as kb
    from transformer_attention_micro_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    kb.lib()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    p = inputs.workload(args.workload)
    q, k, v = device_tensors(p, torch)
    o = torch.empty((p.BH, p.S, p.d), dtype=torch.float32, device="cuda")
    dt = kb.KB_BF16 if p.dtype == inputs.BF16 else kb.KB_F32
    cfg = kb.make_cfg(p.B, p.H, p.S, p.d, p.causal, dt)
    stream = int(torch.cuda.current_stream().cuda_stream)
    flops = kb.attention_flops(p.B, p.H, p.S, p.d, p.causal)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr())

    for _ in range(args.warmup):
        kb.kb_attention(cfg, *ptrs, "flash", stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    per, total_ms = kb.kb_bench_attention(cfg, *ptrs, "flash", stream, 0, args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    kern_ms = float(np.mean(per))
    achieved = flops / (kern_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[p.dtype]
    traffic = measured_traffic(args.workload)
    if args.traffic_kib:
        traffic = int((args.traffic_kib[0] + args.traffic_kib[1]) * 1024)

    result = {
        "metric": METRIC,
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "B": p.B, "H": p.H, "S": p.S, "d": p.d,
                   "causal": p.causal, "variant": "flash", "out": "f32", "flops_per_step": flops,
                   "seed": p.seed, "inputs_sha256": p.sha256()},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel_ms_mean": round(kern_ms, 4), "kernel_ms_min": round(float(np.min(per)), 4),
                     "kernel_ms_p50": round(float(np.median(per)), 4),
                     "kernel_ms_p99": round(float(np.percentile(per, 99)), 4)},
    }

    # Right after the main measurement, before the HBM-bound legs heat the
    # GPU (a heat-soaked MI355X runs the same flash launch up to ~17% slower).
    if not args.no_configs:
        result["per_config"] = per_config_table(kb, torch, inputs, stream, {args.workload: p})

    if args.copy_mib > 0:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = {"read": 4 * n, "write": 4 * n}
        del src, dst

    if not args.no_extras:
        extras = {}
        ws = torch.empty(kb.kb_attention_workspace_size(cfg, "naive"), dtype=torch.uint8, device="cuda")
        ncfg = kb.make_cfg(p.B, p.H, p.S, p.d, p.causal, dt, 0.0, ws.data_ptr(), ws.numel())
        for name, c in (("naive", ncfg), ("fused", cfg)):
            try:
                pv, _ = kb.kb_bench_attention(c, *ptrs, name, stream, 1, 3)
                ms = float(np.median(pv))
                extras[name] = {"ms": round(ms, 3), "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
                if name == "naive":
                    nbytes = 16 * p.BH * p.S * p.S + kb.attention_bytes(p.B, p.H, p.S, p.d, 2 if dt else 4)
                    extras[name]["hbm_gbs_algorithmic"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
            except kb.KbError as e:
                extras[name] = {"error": str(e)}
        del ws
        torch.cuda.empty_cache()
        result["variants"] = extras
        result["triad"] = triad_calibration(kb, torch, stream)
        from transformer_attention_micro_amd.hbm import best_gbs
        ref = {}
        for kind in ("copy", "read", "write"):
            gbs, block = best_gbs(kb, torch, kind, 2048, (64, 128, 256, 512, 1024), stream, 10, 30)
            ref[kind] = {"gbs": round(gbs, 1), "block": block, "frac_of_8000": round(gbs / HBM_PEAK_GBS, 4)}
        result["hbm_reference"] = ref

    if not args.no_ceilings:
        result["ceilings"] = ceilings(kb, torch, stream)

    if not args.no_cpu:
        kb.kb_attention(cfg, *ptrs, "flash", stream)
        torch.cuda.synchronize()
        o_host = o.cpu().numpy().reshape(p.BH * p.S, p.d).astype(np.float64)
        result["cpu_baseline"] = cpu_baseline(p, o_host, args.cpu_seconds)
        result["cpu_baseline"]["small_configs"] = cpu_small_configs(kb, torch, inputs, stream)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
