"""kb_attention_naive_noalloc: the naive variant on the library's static
scratch (no allocation) against kb_attention's naive variant on a
caller-provided workspace.  Both run the same kernels on the same inputs,
so the outputs must agree bit for bit; two calls in a row, the second on a
smaller problem (the scratch keeps the first call's scores), and a call past
the scratch limit is refused before any launch."""
import numpy as np
import pytest

import transformer_attention_micro_amd as kb
from transformer_attention_micro_amd import inputs
from tests.gpu_util import compare, nan_output, oracle_full, to_device, torch_cuda

pytestmark = pytest.mark.gpu


def _with_workspace(p):
    torch = torch_cuda()
    q, k, v = to_device(p)
    o = nan_output(p)
    kb.attention(q, k, v, o, causal=p.causal, variant="naive", heads=p.H)
    torch.cuda.synchronize()
    return o.cpu().numpy()


def _noalloc(p):
    torch = torch_cuda()
    q, k, v = to_device(p)
    o = nan_output(p)
    dt = kb.KB_BF16 if p.dtype == inputs.BF16 else kb.KB_F32
    cfg = kb.make_cfg(p.B, p.H, p.S, p.d, p.causal, dt)
    stream = int(torch.cuda.current_stream().cuda_stream)
    kb.kb_attention_naive_noalloc(cfg, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), stream)
    torch.cuda.synchronize()
    return o.cpu().numpy()


def test_noalloc_matches_the_workspace_entry_point_twice_in_a_row():
    # the first call fills most of the 64 MiB scratch (8 * 1024^2 * 4 B =
    # 32 MiB); the second, smaller one finds the first one's scores there
    big = inputs.make_problem(2, 4, 1024, 64, inputs.BF16, causal=True, seed=21)
    small = inputs.make_problem(1, 3, 333, 128, inputs.F32, causal=False, seed=22)
    for label, p in (("first B2H4S1024d64 bf16 causal", big), ("second B1H3S333d128 f32", small)):
        print(f"[noalloc] {label}", flush=True)
        want = _with_workspace(p)
        got = _noalloc(p)
        assert np.array_equal(got, want), label
        compare(got, oracle_full(p), p.dtype, f"noalloc/{label}")


def test_noalloc_refuses_problems_past_the_scratch():
    torch = torch_cuda()
    S = 1 << 12  # 4 * 1 * 1 * 4096^2 = 64 MiB: fits exactly; one more head does not
    q = torch.zeros((2, S, 32), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((2, S, 32), dtype=torch.float32, device="cuda")
    cfg = kb.make_cfg(1, 2, S, 32, False, kb.KB_BF16)
    with pytest.raises(kb.KbError) as ei:
        kb.kb_attention_naive_noalloc(cfg, q.data_ptr(), q.data_ptr(), q.data_ptr(), o.data_ptr(), 0)
    assert ei.value.status == 3 and "static scratch" in str(ei.value)
    assert 4 * S * S == kb.NOALLOC_SCRATCH_BYTES
