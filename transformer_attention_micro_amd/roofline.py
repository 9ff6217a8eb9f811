"""Hierarchical instruction roofline of the attention kernels on one MI355X.

The GPU-Roofline-Python page ("Metrics Used", "How to use the roofline
tool", "Bandwidth Ceilings"), after Ding and Williams' instruction roofline:
a kernel is placed by its instruction count, its transaction count at each
level of the memory hierarchy and its run time, against an instruction
issue ceiling and one bandwidth ceiling per level.

    python -m transformer_attention_micro_amd.roofline run [--workload W] [--variants flash naive fused]
    python -m transformer_attention_micro_amd.roofline ceilings --out FILE.json
    python -m transformer_attention_micro_amd.roofline passes DIR        # the rocprofv3 commands
    python -m transformer_attention_micro_amd.roofline report DIR [--svg FILE]

`run` is the program the profiler wraps: each variant warmed up (at least
`--warmup` launches and `--warmup-ms` of them), then `--launches` timed
launches at the workload; then calibration kernels whose bytes are known (the HBM read
and write kernels over 1 GiB each, the LDS, L1 and L2 read probes).
`passes` prints one kernel-trace run and four counter passes of it, each
within the per-pass counter limits.  `ceilings` measures the bandwidth
ceilings and the vector issue rate.  `report` reads the five result folders
and the ceilings, and prints the roofline as Markdown: per-kernel metrics,
ridge points, which ceiling binds, and a text plot per kernel.

Metrics (the page's definitions, read for wave64 hardware):
  instructions  SQ_INSTS_* count wave instructions: one per instruction a
                64-lane wave issues, i.e. the per-thread count divided by
                the 64 lanes of a wave (the page divides by the 32 of a
                warp).  The plotted count is the vector ALU class (MFMA
                included, SQ_INSTS_VALU): on CDNA a CU issues at most one
                wave VALU instruction per clock, while the other classes
                issue beside it.
  transactions  64-byte units at every level:
    LDS   SQ_INSTS_LDS_LOAD_BANDWIDTH + SQ_INSTS_LDS_STORE_BANDWIDTH (in 64 B
          by definition; loads that go straight from global memory into
          LDS are vector-memory instructions and are not in them)
    L1    TCP_TOTAL_CACHE_ACCESSES x bytes per access (calibrated on the
          L1 probe, whose bytes are known)
    L2    (TCC_READ_SECTORS + TCC_WRITE_SECTORS) x 32 B
    HBM   FETCH_SIZE and WRITE_SIZE (KiB), each scaled by what it reads for
          the 1 GiB read and write kernels
  performance   wave instructions / (1e9 x kernel time)  [GIPS]
  intensity     wave instructions / transactions at that level
"""
from __future__ import annotations

import argparse
import csv
import json
import math
import os
import re
import sys
from collections import defaultdict

import numpy as np

PASSES = {
    "inst": ["SQ_INSTS", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_SALU", "SQ_INSTS_SMEM", "SQ_INSTS_LDS",
             "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR"],
    "mem": ["SQ_INSTS_LDS_LOAD_BANDWIDTH", "SQ_INSTS_LDS_STORE_BANDWIDTH", "SQ_VALU_MFMA_BUSY_CYCLES",
            "TCP_TOTAL_CACHE_ACCESSES_sum", "TCP_TCC_READ_REQ_sum", "TCP_TCC_WRITE_REQ_sum", "TCC_READ_SECTORS_sum",
            "TCC_WRITE_SECTORS_sum"],
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
}
LEVELS = ("LDS", "L1", "L2", "HBM")
TXN = 64  # bytes per transaction at every level
CALIB_BYTES = 1 << 30  # the read and write calibration kernels move 1 GiB each
NOMINAL_MHZ = 2400.0
DATASHEET_HBM_GBS = 8000.0

# Kernel-name patterns (demangled or mangled) -> label, in report order.
KERNELS = [
    (r"flash_(bf16|f32_split|f32_tile)_kernel", "flash"),
    (r"fused_kernel", "fused"),
    (r"scores_(bf16|f32)_kernel", "naive 1/3 scores"),
    (r"softmax_(vec|any)_kernel", "naive 2/3 softmax"),
    (r"pv_(bf16|f32)_kernel", "naive 3/3 P.V"),
    (r"read_vec_kernel", "HBM read 1 GiB"),
    (r"write_vec_kernel", "HBM write 1 GiB"),
    (r"ceiling_kernel(<4>|ILi4E)", "LDS read probe"),
    (r"ceiling_kernel(<5>|ILi5E)", "L1 read probe"),
    (r"ceiling_kernel(<6>|ILi6E)", "L2 read probe"),
]
CALIBRATION = {"HBM read 1 GiB", "HBM write 1 GiB", "LDS read probe", "L1 read probe", "L2 read probe"}
PROBE_ITERS = {"lds_read": 4000, "l1_read": 2000, "l2_read": 500}


def label_of(name: str):
    for pat, lab in KERNELS:
        if re.search(pat, name):
            return lab
    return None


# ---------------------------------------------------------------- run (GPU)

def cmd_run(args) -> int:
    import torch

    import transformer_attention_micro_amd as kb
    from transformer_attention_micro_amd import inputs

    if not torch.cuda.is_available():
        print("roofline run needs a GPU", file=sys.stderr)
        return 1
    kb.lib()
    torch.cuda.set_device(0)
    stream = int(torch.cuda.current_stream().cuda_stream)
    p = inputs.workload(args.workload)
    dev = []
    for a in p.device_arrays():
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16) \
            if a.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(a))
        dev.append(t.cuda())
    o = torch.empty((p.BH, p.S, p.d), dtype=torch.float32, device="cuda")
    ptrs = (dev[0].data_ptr(), dev[1].data_ptr(), dev[2].data_ptr(), o.data_ptr())
    dt = kb.KB_BF16 if p.dtype == inputs.BF16 else kb.KB_F32
    cfg = kb.make_cfg(p.B, p.H, p.S, p.d, p.causal, dt)
    for variant in args.variants:
        ws = None
        c = cfg
        if variant == "naive":
            ws = torch.empty(kb.kb_attention_workspace_size(cfg, "naive"), dtype=torch.uint8, device="cuda")
            c = kb.make_cfg(p.B, p.H, p.S, p.d, p.causal, dt, 0.0, ws.data_ptr(), ws.numel())
        # Warm up for at least --warmup-ms: after an idle spell the clock
        # boosts for a few launches, dips, and takes ~0.2 s of sustained load
        # to settle where a long run stays.
        first, _ = kb.kb_bench_attention(c, *ptrs, variant, stream, 0, 1)
        warm = max(args.warmup, int(math.ceil(args.warmup_ms / max(first[0], 1e-3))))
        per, _ = kb.kb_bench_attention(c, *ptrs, variant, stream, warm, args.launches)
        print(f"[run] {variant} {args.workload}: {warm + 1} warmup and {args.launches} timed launches, "
              f"mean {np.mean(per):.3f} ms", flush=True)
        del ws
        torch.cuda.empty_cache()
    del dev, o
    torch.cuda.empty_cache()
    if args.no_calibration:
        return 0
    n = CALIB_BYTES // 4
    a = torch.empty(n, dtype=torch.float32, device="cuda")
    b = torch.rand(n, dtype=torch.float32, device="cuda")
    kb.kb_bench_stream("read", a.data_ptr(), b.data_ptr(), float("nan"), n, 256, stream, 0, 1)
    kb.kb_bench_stream("write", a.data_ptr(), b.data_ptr(), 1.5, n, 256, stream, 0, 1)
    del a, b
    work = torch.empty(kb.kb_ceiling_work_size(), dtype=torch.uint8, device="cuda")
    known = {}
    for kind, iters in PROBE_ITERS.items():
        _, nbytes, _ = kb.kb_bench_ceiling(kind, iters, work.data_ptr(), work.numel(), stream, 0, 1)
        known[kind] = nbytes
    print("[run] calibration " + json.dumps({"read_bytes": CALIB_BYTES, "write_bytes": CALIB_BYTES,
                                             "probe_bytes": known, "warmup": args.warmup,
                                             "launches": args.launches}), flush=True)
    torch.cuda.synchronize()
    return 0


# ----------------------------------------------------------- ceilings (GPU)

def cmd_ceilings(args) -> int:
    import torch

    import transformer_attention_micro_amd as kb
    from transformer_attention_micro_amd.hbm import best_gbs

    if not torch.cuda.is_available():
        print("roofline ceilings needs a GPU", file=sys.stderr)
        return 1
    kb.lib()
    torch.cuda.set_device(0)
    stream = int(torch.cuda.current_stream().cuda_stream)
    cus = kb.kb_device_info()["compute_units"]
    work = torch.empty(kb.kb_ceiling_work_size(), dtype=torch.uint8, device="cuda")
    out = {"compute_units": cus, "nominal_mhz": NOMINAL_MHZ, "levels": {}}
    for kind, level in (("lds_read", "LDS"), ("l1_read", "L1"), ("l2_read", "L2"), ("fma_f32", "VALU")):
        per, _, _ = kb.kb_bench_ceiling(kind, 1000, work.data_ptr(), work.numel(), stream, 1, 1)
        iters = max(1, int(1000 * args.target_ms / max(per[0], 1e-3)))
        per, ops, mhz = kb.kb_bench_ceiling(kind, iters, work.data_ptr(), work.numel(), stream, 1, 3)
        ms = float(np.median(per))
        if level == "VALU":
            gips = ops / 128.0 / (ms * 1e-3) / 1e9  # 128 flops per wave v_fma_f32
            out["valu_gips_measured"] = round(gips, 1)
            out["valu_clock_mhz"] = round(mhz, 0)
        else:
            out["levels"][level] = {"gbs": round(ops / (ms * 1e-3) / 1e9, 1), "clock_mhz": round(mhz, 0)}
        print(f"[ceilings] {kind}: {ms:.3f} ms at {mhz:.0f} MHz", flush=True)
    del work
    torch.cuda.empty_cache()
    # HBM: the best of the read-only, write-only and copy kernels (2 GiB
    # working set, best block size), each kept beside it.
    hbm = {"datasheet_gbs": DATASHEET_HBM_GBS}
    for kind in ("read", "write", "copy"):
        gbs, block = best_gbs(kb, torch, kind, 2048, (64, 128, 256, 512, 1024), stream, 10, 30)
        hbm[kind] = {"gbs": round(gbs, 1), "block": block}
    hbm["gbs"] = max(hbm[k]["gbs"] for k in ("read", "write", "copy"))
    out["levels"]["HBM"] = hbm
    out["valu_gips_nominal"] = round(cus * NOMINAL_MHZ * 1e6 / 1e9, 1)
    text = json.dumps(out, indent=1)
    if args.out:
        os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
        with open(args.out, "w") as f:
            f.write(text + "\n")
    print(text)
    return 0


# ------------------------------------------------------------ passes (text)

def pass_commands(outdir: str, workload: str) -> list:
    prog = f"python3 -m transformer_attention_micro_amd.roofline run --workload {workload}"
    cmds = [f"rocprofv3 --kernel-trace --stats --output-format csv -d {outdir}/trace -o p -- {prog}"]
    for name, counters in PASSES.items():
        cmds.append(f"rocprofv3 --pmc {' '.join(counters)} --output-format csv -d {outdir}/{name} -o p -- {prog}")
    return cmds


def cmd_passes(args) -> int:
    for c in pass_commands(args.dir, args.workload):
        print(c)
    return 0


# ------------------------------------------------------------ report (CPU)

def _find(d: str, suffix: str):
    for root, _, files in os.walk(d):
        for f in sorted(files):
            if f.endswith(suffix):
                return os.path.join(root, f)
    return None


def load_trace(d: str) -> dict:
    """Kernel label -> list of dispatch durations (ns), in dispatch order."""
    path = _find(d, "kernel_trace.csv")
    if path is None:
        raise FileNotFoundError(f"no kernel_trace.csv under {d}")
    out = defaultdict(list)
    for r in csv.DictReader(open(path)):
        lab = label_of(r["Kernel_Name"])
        if lab:
            out[lab].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return out


def load_counters(d: str) -> dict:
    """Kernel label -> counter -> list of per-dispatch values, in dispatch order."""
    path = _find(d, "counter_collection.csv")
    if path is None:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    per = defaultdict(lambda: defaultdict(float))
    names = {}
    for r in csv.DictReader(open(path)):
        lab = label_of(r["Kernel_Name"])
        if lab:
            key = int(r["Dispatch_Id"])
            per[key][r["Counter_Name"]] += float(r["Counter_Value"])
            names[key] = lab
    out = defaultdict(lambda: defaultdict(list))
    for key in sorted(per):
        for c, v in per[key].items():
            out[names[key]][c].append(v)
    return out


def _typical(vals: list, timed: int) -> float:
    """Mean over the last `timed` dispatches (the warmup launches before them
    run on cold caches and a ramping clock); all of them if there are fewer."""
    v = vals[-timed:] if 0 < timed < len(vals) else vals
    return float(np.mean(v))


def _counter(passes: dict, lab: str, name: str, timed: int = 0) -> float:
    for p in passes.values():
        if lab in p:
            for key in (name, name.replace("_sum", "")):
                if key in p[lab]:
                    return _typical(p[lab][key], timed)
    return float("nan")


def metrics(trace: dict, passes: dict, calib: dict, timed: int = 0, cus: int = 256,
            mhz: float = NOMINAL_MHZ) -> dict:
    """Per-kernel instruction, transaction and time metrics, each the mean
    over the last `timed` dispatches of the kernel (all if 0)."""
    out = {}
    for _, lab in KERNELS:
        if lab not in trace:
            continue
        t_ns = _typical(trace[lab], timed)
        c = lambda n: _counter(passes, lab, n, timed)  # noqa: E731
        tx = {
            "LDS": c("SQ_INSTS_LDS_LOAD_BANDWIDTH") + c("SQ_INSTS_LDS_STORE_BANDWIDTH"),
            "L1": c("TCP_TOTAL_CACHE_ACCESSES_sum") * calib["l1_bytes_per_access"] / TXN,
            "L2": (c("TCC_READ_SECTORS_sum") + c("TCC_WRITE_SECTORS_sum")) * 32 / TXN,
            "HBM": (c("FETCH_SIZE") * calib["fetch_scale"] + c("WRITE_SIZE") * calib["write_scale"]) * 1024 / TXN,
        }
        m = {"time_us": t_ns / 1e3, "dispatches": len(trace[lab]), "insts": c("SQ_INSTS"),
             "valu": c("SQ_INSTS_VALU"), "mfma": c("SQ_INSTS_MFMA"), "salu": c("SQ_INSTS_SALU"),
             "lds_insts": c("SQ_INSTS_LDS"), "vmem_rd": c("SQ_INSTS_VMEM_RD"), "vmem_wr": c("SQ_INSTS_VMEM_WR"),
             "tx": tx}
        m["gips_valu"] = m["valu"] / (t_ns * 1e-9) / 1e9
        # Matrix-pipe clocks summed over the SIMDs, measured; without that
        # counter, 32 per MFMA (the bf16 32x32x16 form; a 16x16x32 takes 16).
        busy = c("SQ_VALU_MFMA_BUSY_CYCLES")
        m["mfma_busy_measured"] = not math.isnan(busy)
        if not m["mfma_busy_measured"]:
            busy = m["mfma"] * 32
        m["mfma_pipe"] = busy / (4 * cus * mhz * 1e6 * t_ns * 1e-9)
        m["gips_all"] = m["insts"] / (t_ns * 1e-9) / 1e9
        m["intensity"] = {lv: (m["valu"] / tx[lv] if tx[lv] > 0 else math.inf) for lv in LEVELS}
        m["gbs"] = {lv: tx[lv] * TXN / (t_ns * 1e-9) / 1e9 for lv in LEVELS}
        out[lab] = m
    return out


def calibrate(passes: dict, run_log: dict) -> dict:
    """Counter units from the calibration kernels, whose bytes are known."""
    c = lambda lab, n: _counter(passes, lab, n)  # noqa: E731
    probe = run_log.get("probe_bytes", {})
    cal = {"fetch_scale": CALIB_BYTES / (c("HBM read 1 GiB", "FETCH_SIZE") * 1024),
           "write_scale": CALIB_BYTES / (c("HBM write 1 GiB", "WRITE_SIZE") * 1024),
           "l1_bytes_per_access": probe.get("l1_read", math.nan) / c("L1 read probe", "TCP_TOTAL_CACHE_ACCESSES_sum")}
    checks = {
        "LDS probe: LDS counter bytes / known": c("LDS read probe", "SQ_INSTS_LDS_LOAD_BANDWIDTH") * TXN /
        probe.get("lds_read", math.nan),
        "L2 probe: L2 sector bytes / known": c("L2 read probe", "TCC_READ_SECTORS_sum") * 32 / probe.get("l2_read", math.nan),
        "HBM read: L2 sector bytes / known": c("HBM read 1 GiB", "TCC_READ_SECTORS_sum") * 32 / CALIB_BYTES,
        "HBM write: L2 sector bytes / known": c("HBM write 1 GiB", "TCC_WRITE_SECTORS_sum") * 32 / CALIB_BYTES,
        "HBM read: FETCH_SIZE bytes / known": 1.0 / cal["fetch_scale"],
        "HBM write: WRITE_SIZE bytes / known": 1.0 / cal["write_scale"],
        "L1 probe: bytes per TCP cache access": cal["l1_bytes_per_access"],
    }
    return cal, checks


def ceiling_table(ceil: dict) -> dict:
    """GIPS ceiling (nominal and measured) and per-level bandwidth ceilings in
    transactions per second."""
    bw = {lv: ceil["levels"][lv]["gbs"] * 1e9 / TXN for lv in LEVELS}
    return {"gips_nominal": ceil["valu_gips_nominal"], "gips_measured": ceil["valu_gips_measured"], "tps": bw,
            "ridge": {lv: ceil["valu_gips_measured"] * 1e9 / bw[lv] for lv in LEVELS}}


def binding(m: dict, ct: dict):
    """The lowest attainable GIPS over the ceilings at this kernel's
    intensities, and which ceiling it is."""
    best = ("VALU issue", ct["gips_measured"])
    for lv in LEVELS:
        att = ct["tps"][lv] * m["intensity"][lv] / 1e9
        if att < best[1]:
            best = (lv, att)
    return best


def text_plot(lab: str, m: dict, ct: dict, width: int = 64, height: int = 16) -> str:
    """Log-log text plot: x = VALU instructions per 64-byte transaction,
    y = GIPS.  Ceilings drawn with their level's letter (= for the issue
    ceiling), the kernel's point at each level with '*' (labelled below)."""
    x0, x1, y0, y1 = -3.0, 3.0, 0.0, 3.0  # decades
    grid = [[" "] * width for _ in range(height)]
    sym = {"LDS": "s", "L1": "1", "L2": "2", "HBM": "h"}

    def cell(lx, ly):
        cx = int(round((lx - x0) / (x1 - x0) * (width - 1)))
        cy = int(round((y1 - ly) / (y1 - y0) * (height - 1)))
        return cx, cy

    for cx in range(width):
        lx = x0 + (x1 - x0) * cx / (width - 1)
        top = math.log10(ct["gips_measured"])
        for lv in LEVELS:
            ly = math.log10(ct["tps"][lv] / 1e9) + lx
            if ly < top:
                _, cy = cell(lx, ly)
                if 0 <= cy < height:
                    grid[cy][cx] = sym[lv]
        _, cy = cell(lx, top)
        if 0 <= cy < height and all(math.log10(ct["tps"][lv] / 1e9) + lx >= top for lv in LEVELS):
            grid[cy][cx] = "="
    notes = []
    for lv in LEVELS:
        it = m["intensity"][lv]
        if not (it > 0 and math.isfinite(it)) or m["gips_valu"] <= 0:
            continue
        cx, cy = cell(min(max(math.log10(it), x0), x1), min(max(math.log10(m["gips_valu"]), y0), y1))
        grid[cy][cx] = "*"
        notes.append(f"{lv} {it:.3g}")
    lines = [f"{lab}: GIPS (VALU, log) vs VALU instructions per 64 B transaction (log, 1e-3 .. 1e3)"]
    for i, row in enumerate(grid):
        yv = y1 - (y1 - y0) * i / (height - 1)
        lines.append(f"{10 ** yv:7.0f} |" + "".join(row))
    lines.append("        +" + "-" * width)
    lines.append("         1e-3" + " " * (width // 2 - 9) + "1" + " " * (width // 2 - 9) + "1e3")
    lines.append(f"         ceilings: = VALU issue, s LDS, 1 L1, 2 L2, h HBM;  * points at {', '.join(notes)}")
    return "\n".join(lines)


def render(met: dict, ct: dict, ceil: dict, checks: dict, cal: dict, cmds: list, title: str) -> str:
    L = [f"# Hierarchical instruction roofline: {title}", ""]
    L.append("Commands (from the repository root, on one MI355X):")
    L.append("")
    L.append("```")
    L.extend(cmds)
    L.append("```")
    L.append("")
    L.append("## Ceilings")
    L.append("")
    L.append(f"VALU issue: {ct['gips_nominal']:.1f} GIPS nominal (one wave VALU instruction per CU per clock, "
             f"{ceil['compute_units']} CUs at {ceil['nominal_mhz']:.0f} MHz); {ct['gips_measured']:.1f} GIPS "
             f"measured (fp32 FMA probe at {ceil['valu_clock_mhz']:.0f} MHz).")
    L.append("")
    L.append("| Level | Measured GB/s | G transactions/s (64 B) | Ridge (VALU instr / transaction) | Probe |")
    L.append("|---|---|---|---|---|")
    hb = ceil["levels"]["HBM"]
    hbm_kinds = ", ".join(f"{k} {hb[k]['gbs']:.0f}" for k in ("read", "write", "copy") if k in hb)
    probe = {"LDS": "ds_read_b128, 64 KiB window per CU", "L1": "16 KiB slice per CU",
             "L2": "2 MiB region per XCD",
             "HBM": f"best of the HBM kernels at 2 GiB ({hbm_kinds}; datasheet 8000 GB/s)"}
    for lv in LEVELS:
        L.append(f"| {lv} | {ceil['levels'][lv]['gbs']:.0f} | {ct['tps'][lv] / 1e9:.1f} | {ct['ridge'][lv]:.3g} | "
                 f"{probe[lv]} |")
    L.append("")
    L.append("## Counter units (calibration kernels of known bytes, same runs)")
    L.append("")
    L.append("| Check | Value |")
    L.append("|---|---|")
    for k, v in checks.items():
        L.append(f"| {k} | {v:.3f} |")
    L.append("")
    L.append(f"Scales used: FETCH_SIZE x {cal['fetch_scale']:.3f}, WRITE_SIZE x {cal['write_scale']:.3f}, "
             f"{cal['l1_bytes_per_access']:.1f} bytes per TCP cache access.")
    L.append("")
    L.append("## Kernels")
    L.append("")
    L.append("Instruction counts are wave instructions per dispatch; GIPS over the kernel-trace time.")
    L.append("")
    L.append("MFMA pipe: the fraction of the SIMDs' matrix-pipe clocks (at the nominal clock) the kernel's MFMAs "
             "occupy (SQ_VALU_MFMA_BUSY_CYCLES; where that counter is absent, 32 clocks per MFMA).")
    L.append("")
    L.append("| Kernel | Time (us) | Wave instr | VALU (MFMA) | LDS instr | VMEM rd/wr | GIPS all | GIPS VALU | "
             "MFMA pipe |")
    L.append("|---|---|---|---|---|---|---|---|---|")
    for lab, m in met.items():
        L.append(f"| {lab} | {m['time_us']:.1f} | {m['insts']:.3e} | {m['valu']:.3e} ({m['mfma']:.2e}) | "
                 f"{m['lds_insts']:.2e} | {m['vmem_rd']:.2e}/{m['vmem_wr']:.2e} | {m['gips_all']:.1f} | "
                 f"{m['gips_valu']:.1f} | {m['mfma_pipe']:.2f} |")
    L.append("")
    L.append("| Kernel | LDS GB/s | L1 GB/s | L2 GB/s | HBM GB/s | Intensity LDS / L1 / L2 / HBM | Binding ceiling "
             "(attainable GIPS) | Achieved / attainable |")
    L.append("|---|---|---|---|---|---|---|---|")
    for lab, m in met.items():
        lv, att = binding(m, ct)
        its = " / ".join(f"{m['intensity'][x]:.3g}" for x in LEVELS)
        g = m["gbs"]
        L.append(f"| {lab} | {g['LDS']:.0f} | {g['L1']:.0f} | {g['L2']:.0f} | {g['HBM']:.0f} | {its} | "
                 f"{lv} ({att:.0f}) | {m['gips_valu'] / att:.2f} |")
    L.append("")
    L.append("## Plots")
    L.append("")
    for lab, m in met.items():
        if lab in CALIBRATION:
            continue
        L.append("```")
        L.append(text_plot(lab, m, ct))
        L.append("```")
        L.append("")
    return "\n".join(L)


def svg_plot(met: dict, ct: dict, path: str) -> None:
    import matplotlib
    matplotlib.use("Agg")
    import matplotlib.pyplot as plt
    plt.rcParams["svg.fonttype"] = "none"
    labs = [lab for lab in met if lab not in CALIBRATION]
    fig, axes = plt.subplots(1, len(labs), figsize=(4.2 * len(labs), 4), squeeze=False)
    xs = np.logspace(-3, 3, 200)
    colors = {"LDS": "tab:green", "L1": "tab:orange", "L2": "tab:purple", "HBM": "tab:blue"}
    for ax, lab in zip(axes[0], labs):
        m = met[lab]
        for lv in LEVELS:
            ax.plot(xs, np.minimum(ct["tps"][lv] * xs / 1e9, ct["gips_measured"]), color=colors[lv], lw=1, label=lv)
            it = m["intensity"][lv]
            if math.isfinite(it) and it > 0:
                ax.plot([it], [m["gips_valu"]], "o", color=colors[lv])
            ax.axvline(ct["ridge"][lv], color=colors[lv], lw=0.5, ls=":")
        ax.axhline(ct["gips_nominal"], color="k", lw=0.8, ls="--")
        ax.set_xscale("log")
        ax.set_yscale("log")
        ax.set_ylim(1, 2e3)
        ax.set_title(lab, fontsize=9)
        ax.set_xlabel("VALU instr / 64 B transaction")
    axes[0][0].set_ylabel("GIPS (VALU)")
    axes[0][0].legend(fontsize=7)
    fig.tight_layout()
    fig.savefig(path)


def cmd_report(args) -> int:
    d = args.dir
    trace = load_trace(os.path.join(d, "trace"))
    passes = {name: load_counters(os.path.join(d, name)) for name in PASSES}
    run_log = {}
    log = os.path.join(d, "run.log")
    if os.path.exists(log):
        for line in open(log):
            if line.startswith("[run] calibration "):
                run_log = json.loads(line[len("[run] calibration "):])
    ceil = json.load(open(args.ceilings or os.path.join(d, "ceilings.json")))
    cal, checks = calibrate(passes, run_log)
    met = metrics(trace, passes, cal, int(run_log.get("launches", 0)), int(ceil["compute_units"]),
                  float(ceil["nominal_mhz"]))
    ct = ceiling_table(ceil)
    # The kernel-trace run goes first, on a GPU that has not just been heated
    # by the ceiling probes: a hot MI355X runs the same flash launch up to
    # ~30% slower.
    cmds = [c + f" > {d}/run.log" if i == 0 else c for i, c in enumerate(pass_commands(d, args.workload))]
    cmds.insert(1, f"python3 -m transformer_attention_micro_amd.roofline ceilings --out {d}/ceilings.json")
    cmds.append(f"python3 -m transformer_attention_micro_amd.roofline report {d} --workload {args.workload}")
    print(render(met, ct, ceil, checks, cal, cmds, args.title or args.workload))
    if args.svg:
        svg_plot(met, ct, args.svg)
    if args.json:
        with open(args.json, "w") as f:
            json.dump({"ceilings": ct, "calibration": cal, "checks": checks,
                       "kernels": {k: {kk: vv for kk, vv in v.items()} for k, v in met.items()}}, f, indent=1,
                      default=float)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", default="b2h32s8192d128_bf16_causal")
    r.add_argument("--variants", nargs="+", default=["flash", "naive", "fused"])
    r.add_argument("--warmup", type=int, default=10)
    r.add_argument("--warmup-ms", type=float, default=300.0)
    r.add_argument("--launches", type=int, default=3)
    r.add_argument("--no-calibration", action="store_true")
    c = sub.add_parser("ceilings")
    c.add_argument("--out", default=None)
    c.add_argument("--target-ms", type=float, default=30.0)
    p = sub.add_parser("passes")
    p.add_argument("dir")
    p.add_argument("--workload", default="b2h32s8192d128_bf16_causal")
    rp = sub.add_parser("report")
    rp.add_argument("dir")
    rp.add_argument("--workload", default="b2h32s8192d128_bf16_causal")
    rp.add_argument("--ceilings", default=None)
    rp.add_argument("--svg", default=None)
    rp.add_argument("--json", default=None)
    rp.add_argument("--title", default=None)
    args = ap.parse_args(argv)
    return {"run": cmd_run, "ceilings": cmd_ceilings, "passes": cmd_passes, "report": cmd_report}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())
