"""Host-side checks of the C ABI (CPU only; nothing is launched).

libkb.so must load here (no GPU), export every function include/kb_attention.h
declares, and reject bad arguments before touching the device.  With valid
arguments and no device the library must say so (KB_ERR_NO_DEVICE) instead of
launching anything.
"""
import ctypes
import re
from pathlib import Path

import pytest

import transformer_attention_micro_amd as kb
from transformer_attention_micro_amd import _lib

HEADER = Path(__file__).resolve().parents[1] / "include" / "kb_attention.h"
FAKE = 1 << 28  # aligned, non-NULL stand-in pointer; never dereferenced on these paths


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(kb_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert names == sorted(_lib.EXPORTS)
    lib = kb.lib()
    for n in names:
        assert isinstance(getattr(lib, n), ctypes._CFuncPtr), n


def test_ceiling_kinds_match_the_header():
    """The Python names of the ceiling probes map to the header's
    kb_ceiling_kind values, every one of them."""
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    kinds = {m.group(1).lower(): int(m.group(2)) for m in re.finditer(r"\bKB_CEIL_([A-Z0-9_]+)\s*=\s*(\d+)", text)}
    assert kinds == dict(_lib.CEILINGS)


def test_status_strings():
    for code in range(6):
        assert kb.kb_status_string(code) and kb.kb_status_string(code) != "unknown status"
    assert kb.kb_status_string(99) == "unknown status"


def cfg(**kw):
    base = dict(batch=2, heads=3, seq=100, dim=64, causal=False, dtype=kb.KB_BF16)
    base.update(kw)
    return kb.make_cfg(base["batch"], base["heads"], base["seq"], base["dim"], base["causal"], base["dtype"],
                       base.get("scale", 0.0), base.get("workspace", 0), base.get("workspace_bytes", 0))


def test_workspace_size():
    assert kb.kb_attention_workspace_size(cfg(), "naive") == 4 * 2 * 3 * 100 * 100
    assert kb.kb_attention_workspace_size(cfg(), "flash") == 0
    assert kb.kb_attention_workspace_size(cfg(), "fused") == 0
    with pytest.raises(kb.KbError):
        kb.kb_attention_workspace_size(cfg(seq=0), "naive")


def status_of(c, variant="flash", ptrs=(FAKE, FAKE * 2, FAKE * 3, FAKE * 4)):
    try:
        kb.kb_attention(c, *ptrs, variant)
    except kb.KbError as e:
        return e.status
    return 0


@pytest.mark.parametrize("bad", [dict(batch=0), dict(heads=-1), dict(seq=0), dict(dim=0),
                                 dict(causal=2), dict(dtype=7), dict(scale=-1.0),
                                 dict(scale=float("inf"))])
def test_invalid_arguments(bad):
    c = cfg(**{k: v for k, v in bad.items() if k != "causal"})
    if "causal" in bad:
        c.causal = bad["causal"]
    assert status_of(c) == 1


def test_null_pointers_and_bad_variant():
    assert kb.lib().kb_attention(None, FAKE, FAKE, FAKE, FAKE, 2, None) == 1
    assert status_of(cfg(), ptrs=(0, FAKE, FAKE, FAKE * 4)) == 1
    assert status_of(cfg(), ptrs=(FAKE, FAKE * 2, FAKE * 3, 0)) == 1
    assert status_of(cfg(), variant=3) == 1


def test_unsupported_dims_and_sizes():
    assert status_of(cfg(dim=48)) == 2
    assert status_of(cfg(dim=256)) == 2
    assert status_of(cfg(batch=1, heads=1, seq=1 << 24, dim=128)) == 2
    c = cfg()
    c.out_dtype = 5
    assert status_of(c) == 1


def test_dispatch_limits_of_the_row_per_workgroup_variants():
    """naive's softmax and fused launch one 256-thread workgroup per query
    row, so B*H*S must stay below 2^24 rows; naive's slice grid dimension
    holds at most 65535.  Both are refused before any launch (and before any
    device query), while flash takes the same shapes."""
    big_rows = cfg(batch=1, heads=16384, seq=1024, dim=32)  # 2^24 rows, 2^29 elements
    assert status_of(big_rows, variant="naive") == 2
    assert status_of(big_rows, variant="fused") == 2
    assert b"dispatch" in kb.lib().kb_last_error()
    many_slices = cfg(batch=1, heads=65536, seq=4, dim=32)
    assert status_of(many_slices, variant="naive") == 2
    with pytest.raises(kb.KbError):
        kb.kb_attention_workspace_size(big_rows, "naive")
    # just under the row limit: accepted by validation (the host has no
    # device, so a valid call stops at the device check, status 5)
    import torch
    if not torch.cuda.is_available():
        far = tuple(i << 34 for i in range(1, 5))  # 1 GiB tensors must not overlap
        ok = cfg(batch=1, heads=16383, seq=1024, dim=32)
        assert status_of(ok, variant="fused", ptrs=far) == 5
        assert status_of(big_rows, variant="flash", ptrs=far) == 5


def test_noalloc_entry_point_checks_before_touching_a_device():
    """kb_attention_naive_noalloc: bad arguments and problems whose scores
    exceed the static scratch are refused before any device query or launch;
    a valid call without a device reports KB_ERR_NO_DEVICE."""
    lib = kb.lib()
    ptrs = (FAKE, FAKE * 2, FAKE * 3, FAKE * 4)
    assert lib.kb_attention_naive_noalloc(None, *ptrs, None) == 1
    assert lib.kb_attention_naive_noalloc(ctypes.byref(cfg(dim=48)), *ptrs, None) == 2
    big = cfg(batch=1, heads=2, seq=4096, dim=32)  # 2 * 4096^2 * 4 B = 128 MiB > 64 MiB
    assert lib.kb_attention_naive_noalloc(ctypes.byref(big), *ptrs, None) == 3
    assert b"static scratch" in lib.kb_last_error()
    import torch
    if not torch.cuda.is_available():
        fits = cfg(batch=1, heads=1, seq=4096, dim=32)  # exactly 64 MiB
        assert lib.kb_attention_naive_noalloc(ctypes.byref(fits), *ptrs, None) == 5


def test_misaligned_or_overlapping_buffers():
    assert status_of(cfg(), ptrs=(FAKE + 2, FAKE * 2, FAKE * 3, FAKE * 4)) == 1
    # O overlapping Q
    assert status_of(cfg(), ptrs=(FAKE, FAKE * 2, FAKE * 3, FAKE + 64)) == 1


def test_naive_needs_workspace():
    assert status_of(cfg(), variant="naive") == 3
    c = cfg(workspace=FAKE * 8, workspace_bytes=4 * 2 * 3 * 100 * 100 - 1)
    assert status_of(c, variant="naive") == 3
    c = cfg(workspace=FAKE * 8 + 16, workspace_bytes=4 * 2 * 3 * 100 * 100)
    assert status_of(c, variant="naive") == 3


def test_naive_workspace_must_not_overlap_the_tensors():
    nb = 4 * 2 * 3 * 100 * 100
    # Q at FAKE (76,800 bytes of bf16), O at 4 FAKE (153,600 bytes of fp32)
    for ws in (FAKE, FAKE - nb + 256, FAKE * 4 + 1024, FAKE * 3 - 256 * 4):
        assert status_of(cfg(workspace=ws - ws % 256, workspace_bytes=nb), variant="naive") == 1, ws
    if not __import__("torch").cuda.is_available():
        # clear of every tensor: past the argument checks, to the device query
        assert status_of(cfg(workspace=FAKE * 8, workspace_bytes=nb), variant="naive") == 5


def test_valid_call_without_device_reports_no_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert status_of(cfg()) == 5
    c = cfg()
    c.out_dtype = kb.KB_BF16
    assert status_of(c) == 5
    assert "device" in kb.lib().kb_last_error().decode().lower() or kb.lib().kb_last_error()


def test_triad_argument_checks():
    lib = kb.lib()
    assert lib.kb_triad(None, FAKE, FAKE, 1.0, 16, 256, None) == 1
    assert lib.kb_triad(FAKE, FAKE * 2, FAKE * 3, 1.0, 0, 256, None) == 1
    assert lib.kb_triad(FAKE, FAKE * 2, FAKE * 3, 1.0, 16, 100, None) == 1
    assert lib.kb_triad(FAKE, FAKE * 2, FAKE * 3, 1.0, 16, 2048, None) == 1
    assert lib.kb_triad(FAKE, FAKE + 8, FAKE * 3, 1.0, 16, 256, None) == 1


def test_flop_and_byte_counts():
    assert kb.attention_flops(1, 1, 64, 32, False) == 524288
    assert kb.attention_flops(2, 32, 8192, 128, True) == 1099645845504
    assert kb.attention_flops(1, 16, 32768, 128, False) == 8796093022208
    assert kb.attention_bytes(1, 1, 64, 32, 4) == 32 * 1024


def test_ceiling_argument_checks():
    import ctypes as ct
    lib = kb.lib()
    per = (ct.c_float * 2)()
    ops = ct.c_double()
    clk = ct.c_float()
    # bad kind, iters, reps, warmup, NULL results: rejected before any device query
    bad = max(_lib.CEILINGS.values()) + 1
    assert lib.kb_bench_ceiling(bad, 10, FAKE, 1 << 20, None, 0, 2, per, ct.byref(ops), ct.byref(clk)) == 1
    assert lib.kb_bench_ceiling(-1, 10, FAKE, 1 << 20, None, 0, 2, per, ct.byref(ops), ct.byref(clk)) == 1
    assert lib.kb_bench_ceiling(0, 0, FAKE, 1 << 20, None, 0, 2, per, ct.byref(ops), ct.byref(clk)) == 1
    assert lib.kb_bench_ceiling(0, 10, FAKE, 1 << 20, None, 0, 0, per, ct.byref(ops), ct.byref(clk)) == 1
    assert lib.kb_bench_ceiling(0, 10, FAKE, 1 << 20, None, -1, 2, per, ct.byref(ops), ct.byref(clk)) == 1
    assert lib.kb_bench_ceiling(0, 10, FAKE, 1 << 20, None, 0, 2, None, ct.byref(ops), ct.byref(clk)) == 1
    assert lib.kb_bench_ceiling(0, 10, FAKE, 1 << 20, None, 0, 2, per, None, ct.byref(clk)) == 1


def test_ceiling_without_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    import ctypes as ct
    per = (ct.c_float * 2)()
    ops = ct.c_double()
    assert kb.kb_ceiling_work_size() == 0
    assert kb.lib().kb_bench_ceiling(0, 10, FAKE, 1 << 20, None, 0, 2, per, ct.byref(ops), None) == 5


def test_stream_argument_checks():
    import ctypes as ct
    lib = kb.lib()
    per = (ct.c_float * 2)()
    tot = ct.c_float()
    ok = (FAKE, FAKE * 2)
    assert lib.kb_bench_stream(0, *ok, 1.0, 1024, 256, None, 0, 2, per, ct.byref(tot)) == 1   # kind
    assert lib.kb_bench_stream(4, *ok, 1.0, 1024, 256, None, 0, 2, per, ct.byref(tot)) == 1
    assert lib.kb_bench_stream(1, *ok, 1.0, 1022, 256, None, 0, 2, per, ct.byref(tot)) == 1   # n % 4
    assert lib.kb_bench_stream(1, *ok, 1.0, 0, 256, None, 0, 2, per, ct.byref(tot)) == 1
    assert lib.kb_bench_stream(1, FAKE + 4, FAKE * 2, 1.0, 1024, 256, None, 0, 2, per, ct.byref(tot)) == 1
    assert lib.kb_bench_stream(1, FAKE, FAKE + 64, 1.0, 1024, 256, None, 0, 2, per, ct.byref(tot)) == 1
    assert lib.kb_bench_stream(1, *ok, 1.0, 1024, 100, None, 0, 2, per, ct.byref(tot)) == 1   # block
    assert lib.kb_bench_stream(1, None, FAKE, 1.0, 1024, 256, None, 0, 2, per, ct.byref(tot)) == 1


def test_last_error_is_per_thread():
    """The error text lives in thread-local storage: a failing call on one
    host thread leaves another thread's message alone."""
    import threading

    lib = kb.lib()
    assert lib.kb_attention(None, FAKE, FAKE, FAKE, FAKE, 2, None) == 1
    mine = lib.kb_last_error()
    assert b"cfg" in mine
    seen = {}

    def other():
        assert status_of(cfg(dim=48)) == 2  # unsupported head dimension
        seen["msg"] = lib.kb_last_error()

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["msg"] != mine and b"48" in seen["msg"]
    assert lib.kb_last_error() == mine
