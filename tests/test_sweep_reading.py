"""Host logic of the sequence sweep's reading (no GPU): the relative
latencies at S = 2048, where naive reaches its DRAM ceiling, and where
flash's compulsory bandwidth peaks."""
from transformer_attention_micro_amd.sweep import reading


def _row(S, naive_gbs, flash_gbs, flash_tf, fused_x, flash_x):
    return {"S": S, "naive_hbm_gbs_algorithmic": naive_gbs, "flash_hbm_gbs_compulsory": flash_gbs,
            "flash_tflops": flash_tf, "fused_speedup_vs_naive": fused_x, "flash_speedup_vs_naive": flash_x}


def test_reading_names_the_crossovers():
    rows = [_row(1024, 2000, 190, 48.0, 0.34, 1.5), _row(2048, 5500, 200, 98.0, 0.28, 2.3),
            _row(4096, 5600, 150, 120.0, 0.2, 4.0)]
    text = reading(rows, 6000.0)
    assert "fused 0.28x, flash 2.30x" in text
    assert "90% of the triad from S=2048" in text
    assert "peaks at S=2048 (200 GB/s)" in text and "to 150 GB/s at S=4096" in text


def test_reading_when_nothing_crosses():
    rows = [_row(128, 100, 50, 1.0, 2.0, 1.5), _row(256, 300, 80, 3.0, 1.2, 1.4)]
    text = reading(rows, 6000.0)
    assert "stays below 90% of the triad" in text
    assert "still rises at the largest S (256)" in text
    assert "S=2048" not in text
