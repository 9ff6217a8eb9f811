"""Helpers shared by the GPU tests: device copies of seeded problems, the
oracle comparison and the tolerances.

Tolerances (max absolute error of the fp32 output against the fp64 oracle on
the same rounded inputs): 1e-4 for fp32 inputs, 2e-2 for bf16 inputs.
"""
import numpy as np
import pytest

import oracle
from transformer_attention_micro_amd import inputs

TOL = {inputs.F32: 1e-4, inputs.BF16: 2e-2}


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def to_device(p):
    """Q, K, V of problem p as CUDA tensors [B*H, S, d] (bf16 as bf16 bits)."""
    torch = torch_cuda()
    out = []
    for a in p.device_arrays():
        if a.dtype == np.uint16:
            t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(a))
        out.append(t.cuda())
    return out


def nan_output(p):
    torch = torch_cuda()
    return torch.full((p.BH, p.S, p.d), float("nan"), dtype=torch.float32, device="cuda")


def sample_rows(S: int, BH: int, seed: int, per_head: int = 64):
    """Flat row ids bh * S + i: tile-edge rows of every head plus seeded rows."""
    edges = {0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 511, 512, S // 2, S - 2, S - 1}
    rng = np.random.default_rng(seed)
    rows = []
    for bh in range(BH):
        r = {e for e in edges if 0 <= e < S}
        r |= set(rng.integers(0, S, size=per_head).tolist())
        rows.extend(bh * S + i for i in sorted(r))
    return np.array(rows, dtype=np.int64)


def compare(got, want, dtype, label=""):
    """Max-abs and relative L2 error; asserts finiteness and the tolerance."""
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    err = np.abs(got - want)
    max_abs = float(err.max()) if err.size else 0.0
    rel_l2 = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
    print(f"[parity] {label} max_abs={max_abs:.3e} rel_l2={rel_l2:.3e} tol={TOL[dtype]:.0e}", flush=True)
    assert max_abs <= TOL[dtype], f"{label}: max abs error {max_abs:.3e} > {TOL[dtype]:.0e}"
    return max_abs, rel_l2


def oracle_full(p):
    return oracle.sdpa(p.q, p.k, p.v, causal=p.causal)


def oracle_rows(p, rows):
    return oracle.sdpa(p.q, p.k, p.v, causal=p.causal, rows=rows)
