"""MI355X (gfx950) scaled dot-product attention forward: naive, fused and
flash HIP kernels behind the C ABI of libkb.so (include/kb_attention.h),
plus the HBM triad used to calibrate the bandwidth roofline.

The Python layer only marshals arguments; see _lib.py.
"""
from ._lib import (  # noqa: F401
    CEILINGS, EXPORTS, STREAM_BYTES, STREAMS, KB_BF16, KB_F32, KB_FLASH, KB_FUSED, KB_NAIVE, VARIANTS, KbError, attention,
    NOALLOC_SCRATCH_BYTES, attention_bytes, attention_flops, kb_attention, kb_attention_naive_noalloc,
    kb_attention_workspace_size, kb_bench_attention,
    kb_bench_ceiling, kb_bench_stream, kb_bench_triad, kb_ceiling_work_size, kb_device_info, kb_status_string, kb_triad,
    lib, make_cfg, triad, workspace_size,
)
