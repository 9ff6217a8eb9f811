"""ctypes binding of libkb.so (declared in include/kb_attention.h).

Argument marshalling only: every step of the attention forward pass runs in
the library's HIP kernels.  torch is used for device memory and streams: the
tensor helpers below pass data_ptr() values and the current stream's handle
to the C entry points and raise KbError on any non-OK status.  There is no
fallback: if libkb.so is missing or cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import math
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libkb.so"

KB_F32, KB_BF16 = 0, 1
KB_NAIVE, KB_FUSED, KB_FLASH = 0, 1, 2
VARIANTS = {"naive": KB_NAIVE, "fused": KB_FUSED, "flash": KB_FLASH}
STATUS = {0: "KB_OK", 1: "KB_ERR_INVALID", 2: "KB_ERR_UNSUPPORTED", 3: "KB_ERR_WORKSPACE",
          4: "KB_ERR_HIP", 5: "KB_ERR_NO_DEVICE"}
SIZE_MAX = 2 ** (8 * ctypes.sizeof(ctypes.c_size_t)) - 1

# Every symbol the header declares (checked by the CPU tests).
EXPORTS = ("kb_attention", "kb_attention_naive_noalloc", "kb_attention_workspace_size", "kb_triad", "kb_bench_attention",
           "kb_bench_triad", "kb_bench_stream", "kb_ceiling_work_size", "kb_bench_ceiling", "kb_device_info",
           "kb_status_string", "kb_last_error")
CEILINGS = {"mfma_bf16": 0, "mfma_f32": 1, "fma_f32": 2, "exp_f32": 3, "lds_read": 4, "l1_read": 5, "l2_read": 6,
            "mfma_bf16_data": 7, "mfma_bf16_fma3": 8, "mfma_bf16_exp3": 9, "mfma_bf16_exp4": 10,
            "mfma_bf16_lds": 11}
STREAMS = {"copy": 1, "read": 2, "write": 3}
STREAM_BYTES = {"triad": 12, "copy": 8, "read": 4, "write": 4}  # per fp32 element


class KbAttnCfg(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq", ctypes.c_int32),
                ("dim", ctypes.c_int32), ("causal", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class KbDeviceProps(ctypes.Structure):
    _fields_ = [("arch", ctypes.c_char * 64), ("compute_units", ctypes.c_int32),
                ("max_lds_per_block", ctypes.c_int32), ("clock_mhz", ctypes.c_int32),
                ("memory_clock_mhz", ctypes.c_int32), ("global_mem_bytes", ctypes.c_int64)]


class KbError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")


_handle = None


def lib() -> ctypes.CDLL:
    """Load libkb.so once; raise if it has not been built."""
    global _handle
    if _handle is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m transformer_attention_micro_amd.build`")
        h = ctypes.CDLL(str(LIB_PATH))
        vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
        cfgp = ctypes.POINTER(KbAttnCfg)
        fp = ctypes.POINTER(ctypes.c_float)
        h.kb_attention.argtypes = [cfgp, vp, vp, vp, vp, i32, vp]
        h.kb_attention.restype = i32
        h.kb_attention_naive_noalloc.argtypes = [cfgp, vp, vp, vp, vp, vp]
        h.kb_attention_naive_noalloc.restype = i32
        h.kb_attention_workspace_size.argtypes = [cfgp, i32]
        h.kb_attention_workspace_size.restype = sz
        h.kb_triad.argtypes = [vp, vp, vp, f32, sz, i32, vp]
        h.kb_triad.restype = i32
        h.kb_bench_attention.argtypes = [cfgp, vp, vp, vp, vp, i32, vp, i32, i32, fp, fp]
        h.kb_bench_attention.restype = i32
        h.kb_bench_triad.argtypes = [vp, vp, vp, f32, sz, i32, vp, i32, i32, fp, fp]
        h.kb_bench_triad.restype = i32
        h.kb_bench_stream.argtypes = [i32, vp, vp, f32, sz, i32, vp, i32, i32, fp, fp]
        h.kb_bench_stream.restype = i32
        h.kb_ceiling_work_size.argtypes = []
        h.kb_ceiling_work_size.restype = sz
        h.kb_bench_ceiling.argtypes = [i32, i32, vp, sz, vp, i32, i32, fp, ctypes.POINTER(ctypes.c_double), fp]
        h.kb_bench_ceiling.restype = i32
        h.kb_device_info.argtypes = [ctypes.POINTER(KbDeviceProps)]
        h.kb_device_info.restype = i32
        h.kb_status_string.argtypes = [i32]
        h.kb_status_string.restype = ctypes.c_char_p
        h.kb_last_error.argtypes = []
        h.kb_last_error.restype = ctypes.c_char_p
        _handle = h
    return _handle


def _check(status: int, where: str) -> None:
    if status != 0:
        raise KbError(status, where, lib().kb_last_error().decode(errors="replace"))


def make_cfg(batch: int, heads: int, seq: int, dim: int, causal: bool, dtype: int,
             scale: float = 0.0, workspace: int = 0, workspace_bytes: int = 0,
             out_dtype: int = KB_F32) -> KbAttnCfg:
    return KbAttnCfg(batch, heads, seq, dim, int(bool(causal)), dtype, out_dtype, float(scale),
                     workspace or None, workspace_bytes)


def _variant(v) -> int:
    return VARIANTS[v] if isinstance(v, str) else int(v)


# ---------------------------------------------------------------- raw entry points

def kb_attention(cfg: KbAttnCfg, q: int, k: int, v: int, o: int, variant, stream: int = 0) -> None:
    _check(lib().kb_attention(ctypes.byref(cfg), q, k, v, o, _variant(variant), stream or None),
           "kb_attention")


def kb_attention_naive_noalloc(cfg: KbAttnCfg, q: int, k: int, v: int, o: int, stream: int = 0) -> None:
    _check(lib().kb_attention_naive_noalloc(ctypes.byref(cfg), q, k, v, o, stream or None),
           "kb_attention_naive_noalloc")


# Bytes of the library's static scratch behind kb_attention_naive_noalloc
# (KB_NOALLOC_SCRATCH_BYTES in the header).
NOALLOC_SCRATCH_BYTES = 64 << 20


def kb_attention_workspace_size(cfg: KbAttnCfg, variant) -> int:
    n = lib().kb_attention_workspace_size(ctypes.byref(cfg), _variant(variant))
    if n == SIZE_MAX:
        raise KbError(1, "kb_attention_workspace_size", lib().kb_last_error().decode(errors="replace"))
    return n


def kb_triad(a: int, b: int, c: int, s: float, n: int, block: int = 256, stream: int = 0) -> None:
    _check(lib().kb_triad(a, b, c, s, n, block, stream or None), "kb_triad")


def kb_bench_attention(cfg: KbAttnCfg, q: int, k: int, v: int, o: int, variant, stream: int,
                       warmup: int, iters: int, per_launch: bool = True):
    """(per-launch ms list, total ms).  per_launch=False records only the two
    outer events (no event between the launches): the list is then empty and
    total / iters is the batched mean."""
    per = (ctypes.c_float * iters)() if per_launch else None
    tot = ctypes.c_float()
    _check(lib().kb_bench_attention(ctypes.byref(cfg), q, k, v, o, _variant(variant), stream or None,
                                    warmup, iters, per, ctypes.byref(tot)), "kb_bench_attention")
    return (list(per) if per_launch else []), tot.value


def kb_bench_triad(a: int, b: int, c: int, s: float, n: int, block: int, stream: int, warmup: int,
                   iters: int):
    per = (ctypes.c_float * iters)()
    tot = ctypes.c_float()
    _check(lib().kb_bench_triad(a, b, c, s, n, block, stream or None, warmup, iters, per,
                                ctypes.byref(tot)), "kb_bench_triad")
    return list(per), tot.value


def kb_bench_stream(kind, a: int, b: int, s: float, n: int, block: int, stream: int, warmup: int,
                    iters: int):
    per = (ctypes.c_float * iters)()
    tot = ctypes.c_float()
    k = STREAMS[kind] if isinstance(kind, str) else int(kind)
    _check(lib().kb_bench_stream(k, a, b, s, n, block, stream or None, warmup, iters, per, ctypes.byref(tot)),
           "kb_bench_stream")
    return list(per), tot.value


def kb_ceiling_work_size() -> int:
    return lib().kb_ceiling_work_size()


def kb_bench_ceiling(kind, iters: int, work: int, work_bytes: int, stream: int, warmup: int, reps: int):
    """Returns (ms per timed launch, operations per launch, mean shader clock in MHz)."""
    per = (ctypes.c_float * reps)()
    ops = ctypes.c_double()
    clk = ctypes.c_float()
    k = CEILINGS[kind] if isinstance(kind, str) else int(kind)
    _check(lib().kb_bench_ceiling(k, iters, work or None, work_bytes, stream or None, warmup, reps, per,
                                  ctypes.byref(ops), ctypes.byref(clk)), "kb_bench_ceiling")
    return list(per), ops.value, clk.value


def kb_device_info() -> dict:
    p = KbDeviceProps()
    _check(lib().kb_device_info(ctypes.byref(p)), "kb_device_info")
    return {"arch": p.arch.decode(), "compute_units": p.compute_units,
            "max_lds_per_block": p.max_lds_per_block, "clock_mhz": p.clock_mhz,
            "memory_clock_mhz": p.memory_clock_mhz, "global_mem_bytes": p.global_mem_bytes}


def kb_status_string(status: int) -> str:
    return lib().kb_status_string(status).decode()


# ---------------------------------------------------------------- torch helpers

def _stream_handle(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return KB_F32
    if t.dtype == torch.bfloat16:
        return KB_BF16
    raise TypeError(f"Q/K/V must be float32 or bfloat16, got {t.dtype}")


def _shape(q, heads):
    if q.dim() == 4:
        return q.shape[0], q.shape[1], q.shape[2], q.shape[3]
    if q.dim() == 3:
        bh = q.shape[0]
        h = heads or 1
        if bh % h:
            raise ValueError("heads must divide the leading dimension")
        return bh // h, h, q.shape[1], q.shape[2]
    raise ValueError("Q must be [B, H, S, d] or [B*H, S, d]")


def attention(q, k, v, out=None, *, causal: bool = False, variant="flash", scale: float = 0.0,
              heads: int | None = None, workspace=None, stream=None):
    """O = softmax(scale * Q K^T [causal]) V through kb_attention.

    q, k, v: contiguous CUDA tensors of one shape, [B, H, S, d] or [B*H, S, d],
    float32 or bfloat16.  out: optional float32 or bfloat16 tensor of the same
    shape (bfloat16: the fp32 result rounded to nearest even); a float32 one
    is allocated when not given.  variant "naive" needs a uint8/float CUDA
    workspace of at least workspace_size(...) bytes; one is allocated (outside
    the kernels) when not given.  Returns the output tensor.
    """
    import torch
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("Q, K, V must be contiguous CUDA tensors")
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("Q, K, V must share shape and dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("Q, K, V must be on one device")
    B, H, S, d = _shape(q, heads)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    elif out.dtype not in (torch.float32, torch.bfloat16) or out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 or bfloat16 tensor shaped like Q")
    # The kernels write O (and naive's workspace) through raw device
    # pointers: a host tensor's address there would be a GPU memory fault.
    if not out.is_cuda or out.device != q.device:
        raise ValueError("out must be a CUDA tensor on Q's device")
    cfg = make_cfg(B, H, S, d, causal, _dtype_code(q), scale,
                   out_dtype=KB_BF16 if out.dtype == torch.bfloat16 else KB_F32)
    vcode = _variant(variant)
    if vcode == KB_NAIVE:
        need = kb_attention_workspace_size(cfg, vcode)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        elif not workspace.is_cuda or workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous CUDA tensor on Q's device")
        cfg.workspace = workspace.data_ptr()
        cfg.workspace_bytes = workspace.numel() * workspace.element_size()
    kb_attention(cfg, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), vcode,
                 _stream_handle(stream))
    return out


def workspace_size(B: int, H: int, S: int, d: int, *, causal=False, dtype="bf16", variant="naive") -> int:
    cfg = make_cfg(B, H, S, d, causal, KB_BF16 if dtype == "bf16" else KB_F32)
    return kb_attention_workspace_size(cfg, variant)


def triad(a, b, c, s: float, block: int = 256, stream=None) -> None:
    """a = b + s * c on fp32 CUDA tensors through kb_triad."""
    import torch
    for t in (a, b, c):
        if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("triad operands must be contiguous float32 CUDA tensors")
    if not (a.numel() == b.numel() == c.numel()):
        raise ValueError("triad operands must have one length")
    kb_triad(a.data_ptr(), b.data_ptr(), c.data_ptr(), s, a.numel(), block, _stream_handle(stream))


def attention_flops(B: int, H: int, S: int, d: int, causal: bool) -> int:
    """Algorithmic FLOPs of one forward pass: 4 d per visible (query, key)
    pair (2 for Q K^T, 2 for P V); exp / max / sum not counted."""
    pairs = S * (S + 1) // 2 if causal else S * S
    return 4 * d * pairs * B * H


def attention_bytes(B: int, H: int, S: int, d: int, in_bytes: int) -> int:
    """Compulsory HBM bytes: read Q, K, V once and write fp32 O once."""
    return B * H * S * d * (3 * in_bytes + 4)


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
