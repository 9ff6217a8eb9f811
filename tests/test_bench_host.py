"""Host-side helpers of bench.py (no GPU): timing statistics, the rows the
oracle checks, algorithmic bytes per variant, the host CPU description and
the clock probe around a measured call."""
import numpy as np

import bench
import transformer_attention_micro_amd as kb
from transformer_attention_micro_amd import inputs


def test_time_stats():
    st = bench.time_stats([1.0, 2.0, 3.0, 4.0, 100.0])
    assert st["n"] == 5 and st["min"] == 1.0 and st["p50"] == 3.0 and st["mean"] == 22.0
    assert 4.0 < st["p99"] <= 100.0


def test_sample_rows_cover_tile_edges_of_every_head():
    S, BH = 8192, 3
    rows = bench.sample_rows(S, BH)
    assert rows.dtype == np.int64 and np.all(np.diff(rows) > 0)
    for bh in range(BH):
        mine = rows[(rows >= bh * S) & (rows < (bh + 1) * S)] - bh * S
        for e in (0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 511, 512, S // 2, S - 2, S - 1):
            assert e in mine
        assert len(mine) <= 15 + 64
    assert np.array_equal(rows, bench.sample_rows(S, BH))  # seeded


def test_algorithmic_bytes():
    p = inputs.make_problem(1, 2, 64, 32, inputs.BF16, seed=0)
    comp = kb.attention_bytes(1, 2, 64, 32, 2)
    assert comp == 2 * 64 * 32 * (3 * 2 + 4)
    assert bench.algorithmic_bytes(kb, p, "flash") == comp
    assert bench.algorithmic_bytes(kb, p, "fused") == comp
    assert bench.algorithmic_bytes(kb, p, "naive") == comp + 16 * 2 * 64 * 64


def test_host_cpu_reports_cores():
    info = bench.host_cpu()
    assert info["affinity_cpus"] >= 1
    if "lscpu_error" not in info:
        assert info["physical_cores"] is None or info["physical_cores"] >= 1
        assert info["smt_threads_per_core"] is None or info["smt_threads_per_core"] >= 1


def test_clock_probe_reads_the_probe_clock_around_a_call():
    """ClockProbe.around runs the call between two probe readings (a stand-in
    library object here; the real probe needs a GPU)."""
    calls = []

    class FakeKb:
        def kb_ceiling_work_size(self):
            return 16

        def kb_bench_ceiling(self, kind, iters, work, n, stream, warmup, reps):
            calls.append(kind)
            return [0.04], 1.0, 1700.0 + len(calls)

    class FakeTorch:
        uint8 = None

        @staticmethod
        def empty(n, dtype=None, device=None):
            class T:
                def data_ptr(self):
                    return 1

                def numel(self):
                    return n
            return T()

    probe = bench.ClockProbe(FakeKb(), FakeTorch(), 0)
    out, clk = probe.around(lambda: "ran")
    assert out == "ran" and calls == ["fma_f32", "fma_f32"]
    assert clk["shader_mhz_before"] == 1701.0 and clk["shader_mhz_after"] == 1702.0
