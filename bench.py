"""Benchmark: SDPA forward throughput of attn_flash on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one attention forward pass (kb_attention, variant flash) over the
workload B=2, H=32, S=8192, d=128, bf16 inputs, causal mask, fp32 output,
with Q, K, V already resident in HBM.  W untimed launches, then the K timed
steps, bracketed by torch.cuda.synchronize() on both sides; inside,
kb_bench_attention records a hipEvent between consecutive launches on the
launch stream, which gives the per-launch kernel time used for the roofline
fraction.  The default warmup (200 launches, ~0.2 s) outlasts the clock
transient of an MI355X coming out of idle (a few fast launches, a dip of up
to ~30 %, then ~0.1 s of recovery); a short warmup leaves the timed steps
inside it, and the line says so (`protocol` and `per_config` below are
always measured warm).

The JSON line also carries:
  roofline      achieved TFLOP/s per launch vs the MI355X dense bf16 MFMA
                peak (2516.6 TFLOP/s), and HBM bytes per launch from the
                rocprofv3 FETCH_SIZE / WRITE_SIZE summary committed under
                profiles/ (null if the kernel changed since it was taken);
  protocol      the headline launch under the HBM page's timing protocol
                (100 warmup launches, then 200 launches x 5 runs; best and
                median of the runs' mean times);
  per_config    every configured workload (and the S=8192 one without the
                mask) x every variant (flash, naive, fused): min / p50 / p99
                / mean kernel time, TFLOP/s and the fraction of the dtype's
                MFMA peak, algorithmic GB/s and the fraction of 8 TB/s, the
                shader clock right before and right after the timed launches
                (a short clock probe), and the max-abs / relative-L2 error against the
                oracle (filled in by the CPU leg; every row for S <= 2048,
                the tile-edge rows plus 64 seeded rows per head above);
                a variant that cannot run a workload says why;
  hbm           the triad calibration and the copy / read-only / write-only
                reference kernels at a 2 GiB working set under the same
                protocol, best over a block-size sweep;
  ceilings      sustained compute and on-chip bandwidth ceilings
                (kb_bench_ceiling) with the shader clock each probe ran at;
  cpu_baseline  the fp64 oracle timed on this host's cores on a bounded,
                seeded sample of the headline workload's query rows (also
                used to check the GPU output on those rows), with the host's
                physical core count and SMT state; small_configs: the oracle
                on every row of each workload with S <= 2048, on all threads
                and on one, beside the GPU's time and its error.
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SDPA forward TFLOP/s + % of MFMA peak per (B,H,S,d), causal/non-causal"
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}  # MI355X dense MFMA
HBM_PEAK_GBS = 8000.0
HEADLINE = "b2h32s8192d128_bf16_causal"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-extras", action="store_true", help="skip the HBM calibration and the protocol block")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the table over every configured workload and variant")
    ap.add_argument("--flash-only", action="store_true", help="the per-config table for the flash variant only")
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


# ---------------------------------------------------------------- clocks

class ClockProbe:
    """The shader clock right before and right after a measurement, from a
    ~40 us launch of the fp32-FMA ceiling probe (its waves time themselves
    with s_memtime against the 100 MHz s_memrealtime; kb_bench_ceiling).
    The SMU's own metrics (amdsmi) refresh about once a second, too slowly
    for rows that run a fraction of a second, so they give only the socket
    power of the last refresh."""

    def __init__(self, kb, torch, stream, iters: int = 2000):
        self.kb, self.stream, self.iters = kb, stream, iters
        self.work = torch.empty(kb.kb_ceiling_work_size(), dtype=torch.uint8, device="cuda")
        self.smu = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self.amdsmi = amdsmi
            self.smu = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception:  # no SMU access: report the probe clocks only
            self.smu = None

    def mhz(self):
        _, _, mhz = self.kb.kb_bench_ceiling("fma_f32", self.iters, self.work.data_ptr(), self.work.numel(),
                                             self.stream, 0, 1)
        return round(mhz, 0)

    def smu_power(self):
        if self.smu is None:
            return None
        try:
            pw = self.amdsmi.amdsmi_get_gpu_metrics_info(self.smu).get("current_socket_power")
            return float(pw) if isinstance(pw, (int, float)) else None
        except Exception:
            return None

    def around(self, fn):
        """Runs fn() between two probe launches; returns (fn's result, clocks)."""
        before = self.mhz()
        out = fn()
        after = self.mhz()
        return out, {"shader_mhz_before": before, "shader_mhz_after": after, "smu_socket_power_w": self.smu_power()}


# ---------------------------------------------------------------- timing helpers

def time_stats(per):
    a = np.asarray(per, dtype=np.float64)
    return {"n": int(a.size), "min": round(float(a.min()), 4), "p50": round(float(np.median(a)), 4),
            "p99": round(float(np.percentile(a, 99)), 4), "mean": round(float(a.mean()), 4)}


def sample_rows(S: int, BH: int, seed: int = 0, per_head: int = 64):
    """Flat row ids bh * S + i: the tile-edge rows of every head plus seeded
    rows (the rows the oracle checks when it cannot afford all of them)."""
    edges = {0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 511, 512, S // 2, S - 2, S - 1}
    rng = np.random.default_rng(seed)
    rows = []
    for bh in range(BH):
        r = {e for e in edges if 0 <= e < S}
        r |= set(rng.integers(0, S, size=per_head).tolist())
        rows.extend(bh * S + i for i in sorted(r))
    return np.array(rows, dtype=np.int64)


def algorithmic_bytes(kb, p, variant):
    """Compulsory bytes (Q, K, V read once, fp32 O written once) plus, for
    naive, the fp32 score matrix written, read and rewritten by the softmax
    and read by P V (16 bytes per score)."""
    comp = kb.attention_bytes(p.B, p.H, p.S, p.d, 2 if p.dtype == "bf16" else 4)
    return comp + (16 * p.BH * p.S * p.S if variant == "naive" else 0)


# Rows whose median launch is shorter than this also get a batched mean
# (iters launches back to back between two events): at a few microseconds
# per launch the events recorded between launches are a large part of the
# per-launch times.
BATCHED_BELOW_MS = 1.0


def per_config_table(kb, torch, inputs, stream, cache, clocks, checks, variants=("flash", "naive", "fused"),
                     flash_iters=100, warm_ms=300.0, budget_ms=600.0):
    """Every configured workload x variant x mask.  flash first (each row
    warmed for >= warm_ms, so none sits in a clock transient; before the
    HBM-bound variants heat the GPU), then naive and fused (one warm launch,
    then as many timed launches as fit in ~budget_ms, at least 3).  Each
    row keeps the output rows the oracle will check in `checks`."""
    rows = []
    free = torch.cuda.mem_get_info()[0]
    for vpass in (("flash",), tuple(v for v in variants if v != "flash")):
        for name in inputs.WORKLOADS:
            if not vpass:
                break
            p = cache[name] if name in cache else inputs.workload(name)
            q, k, v = device_tensors(p, torch)
            o = torch.empty((p.BH, p.S, p.d), dtype=torch.float32, device="cuda")
            dt = kb.KB_BF16 if p.dtype == inputs.BF16 else kb.KB_F32
            rid = None if p.S <= 2048 else sample_rows(p.S, p.BH)
            for causal in ([True, False] if name == HEADLINE else [p.causal]):
                for variant in vpass:
                    row = {"workload": name, "B": p.B, "H": p.H, "S": p.S, "d": p.d, "causal": causal,
                           "dtype": p.dtype, "variant": variant}
                    ws = None
                    try:
                        cfg = kb.make_cfg(p.B, p.H, p.S, p.d, causal, dt)
                        if variant == "naive":
                            need = kb.kb_attention_workspace_size(cfg, "naive")
                            if need > free - (8 << 30):
                                raise kb.KbError(3, "workspace", f"{need} bytes do not fit in device memory")
                            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
                            cfg = kb.make_cfg(p.B, p.H, p.S, p.d, causal, dt, 0.0, ws.data_ptr(), need)
                        ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr())
                        first, _ = kb.kb_bench_attention(cfg, *ptrs, variant, stream, 0, 1)
                        t1 = max(first[0], 1e-3)
                        if variant == "flash":
                            warm, iters = max(3, int(np.ceil(warm_ms / t1))), flash_iters
                        else:
                            warm, iters = 1, int(min(100, max(3, budget_ms / t1)))
                        kb.kb_bench_attention(cfg, *ptrs, variant, stream, warm, 1)
                        (per, _), clk = clocks.around(
                            lambda: kb.kb_bench_attention(cfg, *ptrs, variant, stream, 0, iters))
                        st = time_stats(per)
                        fl = kb.attention_flops(p.B, p.H, p.S, p.d, causal)
                        nb = algorithmic_bytes(kb, p, variant)
                        tf = fl / (st["p50"] * 1e-3) / 1e12
                        gbs = nb / (st["p50"] * 1e-3) / 1e9
                        row.update({"kernel_ms": st, "tflops": round(tf, 2),
                                    "frac_of_peak": round(tf / PEAK_TFLOPS[p.dtype], 4),
                                    "tflops_at_mean": round(fl / (st["mean"] * 1e-3) / 1e12, 2),
                                    "algorithmic_bytes": nb, "gbs": round(gbs, 1),
                                    "frac_of_hbm": round(gbs / HBM_PEAK_GBS, 4), "clock": clk,
                                    "max_abs_err": None, "rel_l2_err": None})
                        if st["p50"] < BATCHED_BELOW_MS:
                            # Launch-scale rows: the same launches back to back with
                            # only an outer event pair (no event between launches).
                            _, tot = kb.kb_bench_attention(cfg, *ptrs, variant, stream, 0, iters,
                                                           per_launch=False)
                            bm = tot / iters
                            tb = fl / (bm * 1e-3) / 1e12
                            row.update({"batched_ms": round(bm, 5), "tflops_batched": round(tb, 2),
                                        "frac_of_peak_batched": round(tb / PEAK_TFLOPS[p.dtype], 4)})
                        torch.cuda.synchronize()
                        got = o.cpu().numpy().reshape(p.BH * p.S, p.d)
                        checks.append((row, name, causal, rid, got if rid is None else got[rid].copy()))
                    except kb.KbError as e:
                        row["status"] = str(e)
                    rows.append(row)
                    print(f"[per_config] {name} {'c' if causal else 'nc'} {variant}: "
                          f"{row.get('kernel_ms', {}).get('p50', row.get('status'))}", file=sys.stderr,
                          flush=True)
                    del ws
                    torch.cuda.empty_cache()
            del q, k, v, o
            torch.cuda.empty_cache()
    return rows


def headline_protocol(kb, cfg, ptrs, stream, flops, peak, warmup=100, runs=5, iters=200):
    """The HBM page's timing protocol ("Methodology") applied to the headline
    launch: `warmup` launches, then `runs` runs of `iters` timed launches;
    the best and the median of the runs' mean times."""
    means = []
    for r in range(runs):
        per, _ = kb.kb_bench_attention(cfg, *ptrs, "flash", stream, warmup if r == 0 else 0, iters)
        means.append(float(np.mean(per)))
    best, med = min(means), float(np.median(means))
    return {"warmup": warmup, "runs": runs, "iters": iters, "run_mean_ms": [round(m, 4) for m in means],
            "best_ms": round(best, 4), "median_ms": round(med, 4),
            "tflops_best": round(flops / (best * 1e-3) / 1e12, 2), "tflops_median": round(flops / (med * 1e-3) / 1e12, 2),
            "frac_best": round(flops / (best * 1e-3) / 1e12 / peak, 4),
            "frac_median": round(flops / (med * 1e-3) / 1e12 / peak, 4)}


# ---------------------------------------------------------------- CPU leg (the oracle)

def host_cpu():
    """Physical cores, SMT threads per core and the model name (lscpu), and
    the CPUs this process may use."""
    info = {"affinity_cpus": len(os.sched_getaffinity(0))}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        kv = {}
        for line in out.splitlines():
            if ":" in line:
                a, b = line.split(":", 1)
                kv[a.strip()] = b.strip()
        sockets = int(kv.get("Socket(s)", "0") or 0)
        cps = int(kv.get("Core(s) per socket", "0") or 0)
        tpc = int(kv.get("Thread(s) per core", "0") or 0)
        info.update({"physical_cores": sockets * cps or None, "sockets": sockets or None,
                     "smt_threads_per_core": tpc or None, "smt_on": (tpc > 1) if tpc else None,
                     "logical_cpus": int(kv.get("CPU(s)", "0") or 0) or None, "model": kv.get("Model name")})
    except Exception as e:
        info["lscpu_error"] = f"{type(e).__name__}: {e}"
    return info


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
    cpu = host_cpu()
    return {
        "value": flops / t_used / 1e12,
        "unit": "TFLOP/s",
        "cores": nthreads,
        "kind": "oracle",
        "sample": f"{n} distinct seeded query rows (of {p.BH * p.S}) of the same workload, fp64, "
                  f"{t_used:.1f} s on {nthreads} threads ({cpu.get('physical_cores')} physical cores, "
                  f"{cpu.get('smt_threads_per_core')} threads per core); throughput scaled by the rows' "
                  f"algorithmic FLOPs",
        "host": cpu,
        "max_abs_err_vs_gpu_on_sample": max(errs),
    }


def fill_errors(checks, inputs, cache):
    """The oracle on the rows each per-config row kept; one oracle evaluation
    per (workload, mask), shared by the variants."""
    import oracle
    refs = {}
    for row, name, causal, rid, got in checks:
        key = (name, causal)
        if key not in refs:
            p = cache[name] if name in cache else inputs.workload(name)
            want = oracle.sdpa(p.q, p.k, p.v, causal=causal, rows=rid)
            refs[key] = want.reshape(-1, p.d)
        want = refs[key]
        g = np.asarray(got, dtype=np.float64)
        row["max_abs_err"] = float(np.max(np.abs(g - want)))
        row["rel_l2_err"] = float(np.linalg.norm(g - want) / np.linalg.norm(want))
        row["rows_checked"] = "all" if rid is None else int(len(rid))


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


# ---------------------------------------------------------------- ceilings

# Datasheet peaks the ceilings are compared with (TFLOP/s; the fp32 vector
# figure counts packed FMA, which the probe does not use, so its non-packed
# bound is half of it) and the work per clock per CU of each probe.
CEIL_PEAK = {"mfma_bf16": 2516.6, "mfma_f32": 157.3, "fma_f32": 157.3 / 2, "exp_f32": None, "mfma_bf16_data": 2516.6,
             "mfma_bf16_fma3": 2516.6, "mfma_bf16_exp3": 2516.6, "mfma_bf16_exp4": 2516.6, "mfma_bf16_lds": 2516.6}
CEIL_PER_CLK_CU = {"mfma_bf16": 4096, "mfma_f32": 256, "fma_f32": 128, "exp_f32": None, "mfma_bf16_data": 4096,
                   "mfma_bf16_fma3": 4096, "mfma_bf16_exp3": 4096, "mfma_bf16_exp4": 4096, "mfma_bf16_lds": 4096}
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
            row["frac_of_peak_at_measured_clock"] = round(rate / row["peak_at_measured_clock"], 4)
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
    clocks = ClockProbe(kb, torch, stream)  # after the timed steps: the probe must not warm them
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
                     "kernel_ms_p99": round(float(np.percentile(per, 99)), 4),
                     "shader_mhz_after": clocks.mhz()},
    }
    if args.warmup < 100:
        result["roofline"]["note"] = (f"{args.warmup} warmup launches leave the timed ones inside the clock "
                                      f"transient of a GPU coming out of idle; 'protocol' and 'per_config' "
                                      f"are measured warm")

    if not args.no_extras:
        result["protocol"] = headline_protocol(kb, cfg, ptrs, stream, flops, peak)

    checks = []
    cache = {args.workload: p}
    if not args.no_configs:
        variants = ("flash",) if args.flash_only else ("flash", "naive", "fused")
        result["per_config"] = per_config_table(kb, torch, inputs, stream, cache, clocks, checks, variants)

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
        from transformer_attention_micro_amd import hbm
        cal = hbm.calibrate(kb, torch, stream)
        result["hbm"] = {"calibration_vs_8000": cal["calibration"],
                         "protocol": cal["protocol"], "working_set_mib": cal["working_set_mib"],
                         **{kind: {x: cal[kind][x] for x in ("best_gbs", "median_gbs", "best_block")}
                            for kind in ("triad", "copy", "read", "write")}}

    if not args.no_ceilings:
        result["ceilings"] = ceilings(kb, torch, stream)

    if not args.no_cpu:
        kb.kb_attention(cfg, *ptrs, "flash", stream)
        torch.cuda.synchronize()
        o_host = o.cpu().numpy().reshape(p.BH * p.S, p.d).astype(np.float64)
        result["cpu_baseline"] = cpu_baseline(p, o_host, args.cpu_seconds)
        result["cpu_baseline"]["small_configs"] = cpu_small_configs(kb, torch, inputs, stream)
        if checks:
            fill_errors(checks, inputs, cache)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
