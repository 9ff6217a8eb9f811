"""Host logic of the hierarchical roofline report: synthetic rocprofv3 result
folders with known counters go in, the metrics the instruction-roofline
method defines (instructions / transactions, instructions / time) come out."""
import csv
import json
import math
import os

import pytest

from transformer_attention_micro_amd import roofline as rl

FLASH = "void (anonymous namespace)::flash_bf16_kernel<128, true, 8>(bool _Accum const*, _S, _P, void, int, float)"
SOFTMAX = "_ZN12_GLOBAL__N_118softmax_vec_kernelEPfii"
READ = "(anonymous namespace)::read_vec_kernel(float*, HIP_vector_type<float, 4u> const*, float, unsigned long)"
WRITE = "(anonymous namespace)::write_vec_kernel(HIP_vector_type<float, 4u>*, float, unsigned long)"
LDSP = "void (anonymous namespace)::ceiling_kernel<4>(int, float, unsigned long long*, float*, unsigned char const*)"
L1P = "_ZN12_GLOBAL__N_114ceiling_kernelILi5EEEvifPyPfPKh"
L2P = "void (anonymous namespace)::ceiling_kernel<6>(int, float, unsigned long long*, float*, unsigned char const*)"
GIB = 1 << 30


def _write_trace(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "p_kernel_trace.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        t = 1000
        for i, (name, ns) in enumerate(rows):
            w.writerow(["KERNEL_DISPATCH", i + 1, name, t, t + ns])
            t += ns + 10


def _write_counters(d, rows):
    """rows: (dispatch id, kernel name, {counter: value})"""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for disp, name, vals in rows:
            for c, v in vals.items():
                w.writerow([disp, name, c, v])


@pytest.fixture()
def result_dir(tmp_path):
    """Flash and the softmax pass: one warmup dispatch (garbage values that
    must be ignored) and two timed ones each; then the calibration kernels."""
    d = str(tmp_path)
    probe = {"lds_read": 64e9, "l1_read": 32e9, "l2_read": 8e9}
    # kernels in dispatch order: flash x3, softmax x3, read, write, 3 probes
    names = [FLASH] * 3 + [SOFTMAX] * 3 + [READ, WRITE, LDSP, L1P, L2P]
    times = [5_000_000, 1_000_000, 1_000_000, 9_000_000, 2_000_000, 2_000_000, 200_000, 150_000, 500_000, 900_000,
             250_000]
    _write_trace(os.path.join(d, "trace"), list(zip(names, times)))
    inst = {FLASH: {"SQ_INSTS": 3e8, "SQ_INSTS_VALU": 2e8, "SQ_INSTS_MFMA": 3e7, "SQ_INSTS_LDS": 5e7},
            SOFTMAX: {"SQ_INSTS": 1e9, "SQ_INSTS_VALU": 8e8, "SQ_INSTS_MFMA": 0.0, "SQ_INSTS_LDS": 3e7}}
    # flash: LDS 64 B x 2e8, L1 accesses 1e8 (x 64 B), L2 sectors 2e8 (x 32 B), HBM 1e6 KiB fetched (x2), 2.5e5 written
    mem = {FLASH: {"SQ_INSTS_LDS_LOAD_BANDWIDTH": 1.5e8, "SQ_INSTS_LDS_STORE_BANDWIDTH": 5e7,
                   "SQ_VALU_MFMA_BUSY_CYCLES": 3e7 * 30,
                   "TCP_TOTAL_CACHE_ACCESSES_sum": 1e8, "TCC_READ_SECTORS_sum": 1.5e8, "TCC_WRITE_SECTORS_sum": 5e7},
           SOFTMAX: {"SQ_INSTS_LDS_LOAD_BANDWIDTH": 1e7, "SQ_INSTS_LDS_STORE_BANDWIDTH": 0.0,
                     "TCP_TOTAL_CACHE_ACCESSES_sum": 4e8, "TCC_READ_SECTORS_sum": 4e8, "TCC_WRITE_SECTORS_sum": 4e8}}
    fetch = {FLASH: {"FETCH_SIZE": 1e6}, SOFTMAX: {"FETCH_SIZE": 6.25e6}}
    write = {FLASH: {"WRITE_SIZE": 2.5e5}, SOFTMAX: {"WRITE_SIZE": 1.25e7}}
    calib = {READ: {"FETCH_SIZE": GIB / 1024 / 2, "TCC_READ_SECTORS_sum": GIB / 32, "TCC_WRITE_SECTORS_sum": 0.0},
             WRITE: {"WRITE_SIZE": GIB / 1024, "TCC_READ_SECTORS_sum": 0.0, "TCC_WRITE_SECTORS_sum": GIB / 32},
             LDSP: {"SQ_INSTS_LDS_LOAD_BANDWIDTH": probe["lds_read"] / 64},
             L1P: {"TCP_TOTAL_CACHE_ACCESSES_sum": probe["l1_read"] / 64},
             L2P: {"TCC_READ_SECTORS_sum": probe["l2_read"] / 32}}
    for sub, table in (("inst", inst), ("mem", mem), ("fetch", fetch), ("write", write)):
        rows = []
        for i, name in enumerate(names):
            vals = dict(table.get(name, {}))
            for c, v in calib.get(name, {}).items():
                if any(c in cs for cs in [rl.PASSES[sub]]):
                    vals[c] = v
            if not vals:
                continue
            if i in (0, 3):  # warmup dispatches: values that must not be used
                vals = {c: v * 17.0 + 1e9 for c, v in vals.items()}
            rows.append((i + 1, name, vals))
        _write_counters(os.path.join(d, sub), rows)
    with open(os.path.join(d, "run.log"), "w") as f:
        f.write("[run] flash: 2 launches\n")
        f.write("[run] calibration " + json.dumps({"read_bytes": GIB, "write_bytes": GIB, "probe_bytes": probe,
                                                   "warmup": 1, "launches": 2}) + "\n")
    ceil = {"compute_units": 256, "nominal_mhz": 2400.0, "valu_gips_measured": 500.0, "valu_clock_mhz": 2380.0,
            "valu_gips_nominal": 614.4,
            "levels": {"LDS": {"gbs": 128000.0}, "L1": {"gbs": 32000.0}, "L2": {"gbs": 32000.0},
                       "HBM": {"gbs": 6400.0}}}
    with open(os.path.join(d, "ceilings.json"), "w") as f:
        json.dump(ceil, f)
    return d


def _load(d):
    trace = rl.load_trace(os.path.join(d, "trace"))
    passes = {n: rl.load_counters(os.path.join(d, n)) for n in rl.PASSES}
    run_log = json.loads(open(os.path.join(d, "run.log")).read().split("[run] calibration ")[1])
    return trace, passes, run_log


def test_kernel_names_map_to_labels():
    assert rl.label_of(FLASH) == "flash"
    for fp32 in ("void (anonymous namespace)::flash_f32_split_kernel<64, false, 8>(float const*, float const*, "
                 "float const*, void*, int, int, int, int, float)",
                 "_ZN12_GLOBAL__N_121flash_f32_tile_kernelILi64ELb1EEEvPKfS2_S2_Pviiiif"):
        assert rl.label_of(fp32) == "flash", fp32
    assert rl.label_of(SOFTMAX) == "naive 2/3 softmax"
    assert rl.label_of(L1P) == "L1 read probe"
    assert rl.label_of(LDSP) == "LDS read probe"
    assert rl.label_of("some_other_kernel") is None


def test_calibration_recovers_counter_units(result_dir):
    trace, passes, run_log = _load(result_dir)
    cal, checks = rl.calibrate(passes, run_log)
    assert cal["fetch_scale"] == pytest.approx(2.0)
    assert cal["write_scale"] == pytest.approx(1.0)
    assert cal["l1_bytes_per_access"] == pytest.approx(64.0)
    assert checks["LDS probe: LDS counter bytes / known"] == pytest.approx(1.0)
    assert checks["L2 probe: L2 sector bytes / known"] == pytest.approx(1.0)


def test_metrics_follow_the_definitions(result_dir):
    trace, passes, run_log = _load(result_dir)
    cal, _ = rl.calibrate(passes, run_log)
    met = rl.metrics(trace, passes, cal, timed=run_log["launches"])
    f = met["flash"]
    assert f["time_us"] == pytest.approx(1000.0)  # the 5 ms warmup dispatch is left out
    assert f["valu"] == pytest.approx(2e8)  # so are its counters
    # transactions in 64-byte units
    assert f["tx"]["LDS"] == pytest.approx(2e8)
    assert f["tx"]["L1"] == pytest.approx(1e8)
    assert f["tx"]["L2"] == pytest.approx(2e8 * 32 / 64)
    assert f["tx"]["HBM"] == pytest.approx((2e6 + 2.5e5) * 1024 / 64)
    # intensity = VALU wave instructions / transactions; GIPS = instructions / ns
    for lv in rl.LEVELS:
        assert f["intensity"][lv] == pytest.approx(2e8 / f["tx"][lv])
    assert f["gips_valu"] == pytest.approx(2e8 / 1e6)
    assert f["gips_all"] == pytest.approx(3e8 / 1e6)
    # measured matrix-pipe clocks when the counter is there, else 32 per MFMA
    assert f["mfma_busy_measured"]
    assert f["mfma_pipe"] == pytest.approx(3e7 * 30 / (4 * 256 * 2.4e9 * 1e-3))
    assert not met["naive 2/3 softmax"]["mfma_busy_measured"]
    s = met["naive 2/3 softmax"]
    assert s["gbs"]["HBM"] == pytest.approx((6.25e6 * 2 + 1.25e7) * 1024 / 2e-3 / 1e9)


def test_ceilings_ridges_and_binding(result_dir):
    trace, passes, run_log = _load(result_dir)
    cal, _ = rl.calibrate(passes, run_log)
    met = rl.metrics(trace, passes, cal, timed=2)
    ceil = json.load(open(os.path.join(result_dir, "ceilings.json")))
    ct = rl.ceiling_table(ceil)
    assert ct["tps"]["HBM"] == pytest.approx(6400e9 / 64)
    assert ct["ridge"]["HBM"] == pytest.approx(500e9 / (6400e9 / 64))
    # flash: far right of every ridge -> the issue ceiling binds
    lv, att = rl.binding(met["flash"], ct)
    assert lv == "VALU issue" and att == pytest.approx(500.0)
    # softmax: 25e6 KiB of HBM traffic = 4e8 transactions for 8e8 instructions: intensity 2,
    # attainable 100e9 transactions/s x 2 = 200 GIPS, below the 500 GIPS issue ceiling
    s = met["naive 2/3 softmax"]
    assert s["intensity"]["HBM"] == pytest.approx(8e8 / 4e8)
    lv, att = rl.binding(s, ct)
    assert lv == "HBM" and att == pytest.approx(ct["tps"]["HBM"] * 2.0 / 1e9)


def test_text_plot_and_report(result_dir, capsys):
    assert rl.main(["report", result_dir]) == 0
    out = capsys.readouterr().out
    assert "## Ceilings" in out and "Ridge" in out and "| flash |" in out
    assert out.count("GIPS (VALU, log)") == 2  # one plot per attention kernel, none for calibration kernels
    trace, passes, run_log = _load(result_dir)
    cal, _ = rl.calibrate(passes, run_log)
    met = rl.metrics(trace, passes, cal, timed=2)
    ct = rl.ceiling_table(json.load(open(os.path.join(result_dir, "ceilings.json"))))
    plot = rl.text_plot("flash", met["flash"], ct, width=40, height=10)
    body = [ln for ln in plot.splitlines() if "|" in ln]
    assert len(body) == 10 and all(len(ln.split("|", 1)[1]) == 40 for ln in body)
    assert sum(ln.count("*") for ln in body) >= 1
    assert math.isfinite(met["flash"]["intensity"]["HBM"])


def test_pass_commands_respect_counter_limits():
    """Each counter pass stays within one run's per-block limits (8 SQ, 4 TCC
    with FETCH_SIZE counting 3 and WRITE_SIZE 2, 4 TCP)."""
    tcc_cost = {"FETCH_SIZE": 3, "WRITE_SIZE": 2}
    for name, counters in rl.PASSES.items():
        sq = sum(c.startswith("SQ_") for c in counters)
        tcp = sum(c.startswith("TCP_") for c in counters)
        tcc = sum(tcc_cost.get(c, 1) for c in counters if c.startswith("TCC_") or c in tcc_cost)
        assert sq <= 8 and tcp <= 4 and tcc <= 4, name
    cmds = rl.pass_commands("out", "b2h32s8192d128_bf16_causal")
    assert len(cmds) == 1 + len(rl.PASSES)
    assert all("-- python3 -m transformer_attention_micro_amd.roofline run" in c for c in cmds)
    assert "--kernel-trace" in cmds[0] and all("--pmc" in c for c in cmds[1:])
