"""GPU parity: every variant of kb_attention against the fp64 oracle.

Inputs are the seeded N(0, 1) problems of transformer_attention_micro_amd.inputs
(bf16 problems rounded once on the host, so both sides see the same values).
Outputs are pre-filled with NaN so an element the kernels never write fails.
Every variant is compared on every element of the small and medium problems.
The flash kernel is also compared on every element of the large ones (B2 H32
S8192 d128 causal, its large-logit variant, and B1 H16 S32768 d128, the last
split by heads over several tests so each runs in well under a minute on the
oracle's host threads).  naive and fused, and the extra seeds of the large
flash problems, are compared on the tile-edge rows of every head plus 64
seeded rows per head, computed by the oracle one row at a time.
"""
import numpy as np
import pytest

import oracle
import transformer_attention_micro_amd as kb
from transformer_attention_micro_amd import inputs
from tests.flash_cases import diagonal_keys, first_tile_dominant, growing_keys, sum_overflow_problem
from tests.gpu_util import (TOL, compare, nan_output, oracle_full, oracle_rows, sample_rows, to_device,
                            torch_cuda)

pytestmark = pytest.mark.gpu

VARIANTS = ("naive", "fused", "flash")
_oracle_cache = {}
_problems = {}


def workload(name, seed=0):
    """Named workloads are drawn once per session (the large ones take seconds)."""
    if (name, seed) not in _problems:
        _problems[(name, seed)] = inputs.workload(name, seed=seed)
    return _problems[(name, seed)]


def run(p, variant, **kw):
    torch = torch_cuda()
    q, k, v = to_device(p)
    o = nan_output(p)
    kb.attention(q, k, v, o, causal=p.causal, variant=variant, heads=p.H, **kw)
    torch.cuda.synchronize()
    return o


def full_check(p, variant, label):
    key = (p.B, p.H, p.S, p.d, p.dtype, p.causal, p.seed, p.q_scale)
    if key not in _oracle_cache:
        _oracle_cache[key] = oracle_full(p)
    o = run(p, variant).cpu().numpy()
    return compare(o, _oracle_cache[key], p.dtype, label)


def sampled_check(p, variant, label, seed=0):
    rows = sample_rows(p.S, p.BH, seed)
    key = (p.B, p.H, p.S, p.d, p.dtype, p.causal, p.seed, p.q_scale, "rows", seed)
    if key not in _oracle_cache:
        _oracle_cache[key] = oracle_rows(p, rows)
    o = run(p, variant).cpu().numpy().reshape(p.BH * p.S, p.d)
    assert np.all(np.isfinite(o)), f"{label}: non-finite output somewhere"
    return compare(o[rows], _oracle_cache[key], p.dtype, label)


# ---------------------------------------------------------------- the workloads

@pytest.mark.parametrize("variant", VARIANTS)
def test_b1h1s64d32_f32(variant):
    for seed in (0, 1, 2):
        p = workload("b1h1s64d32_f32", seed=seed)
        full_check(p, variant, f"b1h1s64d32_f32/seed{seed}/{variant}")


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("causal", [False, True])
def test_b1h8s512d64_f32(variant, causal):
    name = "b1h8s512d64_f32" + ("_causal" if causal else "")
    for seed in (0, 1, 2):
        p = workload(name, seed=seed)
        full_check(p, variant, f"{name}/seed{seed}/{variant}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_b4h16s2048d64_bf16_causal(variant):
    for seed in (0, 1, 2):
        p = workload("b4h16s2048d64_bf16_causal", seed=seed)
        full_check(p, variant, f"b4h16s2048d64_bf16_causal/seed{seed}/{variant}")


@pytest.mark.parametrize("variant", ("naive", "fused"))
@pytest.mark.parametrize("name", ["b2h32s8192d128_bf16_causal", "b2h32s8192d128_bf16_causal_q8"])
def test_b2h32s8192d128(variant, name):
    p = workload(name)
    sampled_check(p, variant, f"{name}/{variant}")


@pytest.mark.parametrize("name", ["b2h32s8192d128_bf16_causal", "b2h32s8192d128_bf16_causal_q8"])
def test_b2h32s8192d128_flash_every_row(name):
    """The measured kernel and its large-logit variant, all 524,288 output
    rows against the oracle (on all host threads)."""
    p = workload(name)
    o = run(p, "flash").cpu().numpy()
    want = oracle.sdpa(p.q, p.k, p.v, causal=p.causal)
    compare(o, want, p.dtype, f"{name}/flash/every-row")


@pytest.mark.parametrize("seed", [1, 2])
@pytest.mark.parametrize("name", ["b2h32s8192d128_bf16_causal", "b2h32s8192d128_bf16_causal_q8"])
def test_b2h32s8192d128_flash_more_seeds(name, seed):
    """The measured kernel on two more input draws (not cached: 768 MiB each)."""
    p = inputs.workload(name, seed=seed)
    rows = sample_rows(p.S, p.BH, seed)
    want = oracle_rows(p, rows)
    o = run(p, "flash").cpu().numpy().reshape(p.BH * p.S, p.d)
    assert np.all(np.isfinite(o)), "non-finite output somewhere"
    compare(o[rows], want, p.dtype, f"{name}/seed{seed}/flash")


_C5_PARTS = 8
_flash_outputs = {}


@pytest.mark.parametrize("part", range(_C5_PARTS))
def test_b1h16s32768d128_flash_every_row(part):
    """The long non-causal workload, every output row: the flash output is
    computed once, and each part compares 2 of the 16 heads (65,536 rows)
    against the oracle."""
    name = "b1h16s32768d128_bf16"
    p = workload(name)
    if name not in _flash_outputs:
        _flash_outputs[name] = run(p, "flash").cpu().numpy()
    o = _flash_outputs[name]
    per = p.BH // _C5_PARTS
    h0, h1 = part * per, (part + 1) * per
    rows = np.arange(h0 * p.S, h1 * p.S, dtype=np.int64)
    want = oracle.sdpa(p.q, p.k, p.v, causal=p.causal, rows=rows)
    compare(o[h0:h1].reshape(-1, p.d), want, p.dtype, f"{name}/flash/heads{h0}-{h1 - 1}")
    if part == _C5_PARTS - 1:
        _flash_outputs.pop(name, None)


@pytest.mark.parametrize("seed", [1, 2])
def test_b1h16s32768d128_flash_more_seeds(seed):
    """The long non-causal workload on two more input draws: tile-edge rows
    and 64 seeded rows of every head, and a finite output everywhere."""
    p = inputs.workload("b1h16s32768d128_bf16", seed=seed)
    rows = sample_rows(p.S, p.BH, seed)
    want = oracle_rows(p, rows)
    o = run(p, "flash").cpu().numpy().reshape(p.BH * p.S, p.d)
    assert np.all(np.isfinite(o)), "non-finite output somewhere"
    compare(o[rows], want, p.dtype, f"b1h16s32768d128_bf16/seed{seed}/flash")


@pytest.mark.parametrize("variant", ("naive", "fused"))
def test_b1h16s32768d128_bf16(variant):
    p = workload("b1h16s32768d128_bf16")
    try:
        sampled_check(p, variant, f"b1h16s32768d128_bf16/{variant}")
    except kb.KbError as e:
        # fused needs 4*S bytes of LDS per row; the library reports when the
        # device cannot hold it (never silently).
        if variant == "fused" and e.status == 2:
            pytest.skip(str(e))
        raise


# ---------------------------------------------------------------- ragged and tiny shapes

TINY_S = (1, 2, 3, 17, 31, 33, 64, 65, 127, 129, 200)


@pytest.mark.parametrize("dtype", [inputs.F32, inputs.BF16])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("variant", VARIANTS)
def test_ragged_shapes(dtype, d, causal, variant):
    for S in TINY_S:
        p = inputs.make_problem(1, 3, S, d, dtype, causal=causal, seed=S)
        full_check(p, variant, f"S{S}/d{d}/{dtype}/{'c' if causal else 'nc'}/{variant}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_several_query_tiles_and_ragged_tail(variant):
    """Multi-tile shapes with a tail in both the query and key directions."""
    for dtype, d, S in ((inputs.BF16, 128, 1000), (inputs.F32, 64, 777), (inputs.BF16, 64, 1541)):
        for causal in (False, True):
            p = inputs.make_problem(2, 2, S, d, dtype, causal=causal, seed=S + d)
            full_check(p, variant, f"B2H2S{S}/d{d}/{dtype}/{'c' if causal else 'nc'}/{variant}")


@pytest.mark.parametrize("causal", [False, True])
def test_flash_work_split_over_xcds(causal):
    """Slice counts that do not divide over the 8 XCDs (some get two slices,
    some none) and odd query-tile counts (a causal unit with a single middle
    tile), through the flash kernel's persistent schedule."""
    for (B, H, S, d) in ((3, 3, 700, 128), (1, 17, 1300, 64), (1, 1, 2600, 128), (5, 2, 300, 32)):
        p = inputs.make_problem(B, H, S, d, inputs.BF16, causal=causal, seed=B * 100 + H + S)
        full_check(p, "flash", f"B{B}H{H}S{S}/d{d}/{'c' if causal else 'nc'}/flash")


@pytest.mark.parametrize("causal", [False, True])
def test_flash_several_units_per_workgroup(causal):
    """More work units than CUs, so each persistent workgroup runs units of
    several slices one after another (512 one-tile slices; 160 three-tile
    slices, whose causal units are a pair and a single middle tile), checked
    on every element."""
    for (B, H, S, d) in ((8, 64, 256, 64), (4, 40, 520, 64)):
        p = inputs.make_problem(B, H, S, d, inputs.BF16, causal=causal, seed=B * H + S)
        full_check(p, "flash", f"B{B}H{H}S{S}/d{d}/{'c' if causal else 'nc'}/flash")


@pytest.mark.parametrize("causal", [False, True])
def test_flash_f32_both_kernels(causal):
    """fp32 flash takes the 128-query tile kernel once its grid covers the
    CUs (B*H*ceil(S/128) >= 256 here) and the key-split kernel on 16-query
    blocks below that: shapes on both sides of the switch, every d, ragged
    tails, checked on every element."""
    for (B, H, S, d) in ((2, 16, 1100, 64), (4, 16, 520, 128), (8, 32, 200, 32),  # tile kernel
                         (1, 15, 1100, 64), (2, 3, 520, 128), (1, 1, 2000, 32)):  # key-split kernel
        p = inputs.make_problem(B, H, S, d, inputs.F32, causal=causal, seed=B * H + S + d)
        full_check(p, "flash", f"f32/B{B}H{H}S{S}/d{d}/{'c' if causal else 'nc'}/flash")


@pytest.mark.parametrize("causal", [False, True])
def test_flash_bf16_both_widths(causal):
    """bf16 flash runs 8-wave workgroups on 256-query items, or 4-wave ones
    on 128-query items when ceil(B*H/8) times the 256-query units per slice
    (ceil(S/256), halved up when causal) is below the 32 CUs of an XCD:
    shapes on both sides of that switch, every d, ragged tails, and d=64
    shapes with more 128-query units than CUs (two workgroups per CU),
    checked on every element."""
    shapes = ((1, 16, 2048, 64), (1, 8, 1100, 128), (2, 5, 700, 32),  # 4 waves
              (4, 30, 300, 64), (2, 60, 700, 64),                     # 4 waves, two per CU
              (2, 16, 4096, 64), (1, 64, 1800, 128), (4, 64, 260, 32))  # 8 waves
    for (B, H, S, d) in shapes:
        p = inputs.make_problem(B, H, S, d, inputs.BF16, causal=causal, seed=B * H + S + d)
        full_check(p, "flash", f"bf16/B{B}H{H}S{S}/d{d}/{'c' if causal else 'nc'}/flash")


@pytest.mark.parametrize("variant", VARIANTS)
def test_bf16_output(variant):
    """out_dtype bf16 is the fp32 result rounded to nearest even: bit-exact
    against rounding the fp32 output of the same call on the host, hence
    within the fp32 tolerance plus one bf16 ulp of the oracle."""
    torch = torch_cuda()
    for dtype, d, S, causal in ((inputs.BF16, 128, 700, True), (inputs.F32, 64, 333, False),
                                (inputs.BF16, 32, 129, False)):
        p = inputs.make_problem(2, 3, S, d, dtype, causal=causal, seed=S + d)
        q, k, v = to_device(p)
        o32 = kb.attention(q, k, v, causal=causal, variant=variant, heads=p.H)
        ob = torch.full(o32.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        kb.attention(q, k, v, ob, causal=causal, variant=variant, heads=p.H)
        torch.cuda.synchronize()
        want_bits = inputs.bf16_bits(o32.cpu().numpy())
        got_bits = ob.cpu().view(torch.int16).numpy().view(np.uint16)
        label = f"bf16-out/S{S}/d{d}/{dtype}/{variant}"
        assert np.array_equal(got_bits, want_bits), label
        got = inputs.bf16_bits_to_f32(got_bits).astype(np.float64)
        ref = oracle_full(p)
        _, e = np.frexp(np.abs(ref))
        ulp = np.ldexp(1.0, e - 8)
        assert np.all(np.abs(got - ref) <= TOL[dtype] + ulp), label


# ------------------------------------------- scores that grow along the key axis
# The bf16 flash kernel takes most tiles without a row maximum, against a
# reference that starts a margin above the first tile's exact maximum, and
# checks the tile's probability sums instead.  Keys scaled by powers of two
# (exact in bf16) make later tiles' scores outgrow the reference: by tens of
# log2 units (the sum check fails and the tile is corrected in place), or by
# hundreds (the exponentials overflow and the whole query tile is recomputed
# exactly).  tests/test_reference_model.py checks, on a CPU model of that
# tracking, which of the two each case below reaches.

@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("jump", [False, True])
@pytest.mark.parametrize("S", [1024, 1000])
def test_flash_scores_outgrowing_the_reference(d, causal, jump, S):
    """S = 1000 adds a ragged last tile and a last query tile with rows past
    the sequence end."""
    p = growing_keys(d, causal, jump, S)
    o = run(p, "flash").cpu().numpy()
    want = oracle_full(p)
    compare(o, want, p.dtype, f"growing-keys/S{S}/d{d}/{'c' if causal else 'nc'}/{'jump' if jump else 'steps'}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("jump", [False, True])
def test_flash_scores_outgrowing_the_reference_8_waves(d, causal, jump):
    """The same growing keys on enough heads (64, or 128 causal, at S=1024)
    that the kernel runs 8-wave workgroups on 256-query items: in-place
    corrections and exact redos there, and (causal, d=64) the early output
    stores of waves whose last tile comes before the item's last step."""
    p = growing_keys(d, causal, jump, 1024, H=128 if causal else 64)
    o = run(p, "flash").cpu().numpy()
    want = oracle_full(p)
    compare(o, want, p.dtype, f"growing-keys-8w/H{p.H}/d{d}/{'c' if causal else 'nc'}/{'jump' if jump else 'steps'}")


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("scale", [16.0, 256.0])
def test_flash_last_waves_diagonal_tile_outgrowing_the_reference(d, scale):
    """Keys from 448 on scaled by 16 (scores tens of log2 units above the
    reference, margin included: about a third of the waves at rows 448..511
    correct that tile in place, none overflows) or 256 (the exponentials
    overflow: the query tile is redone exactly).  Key tile 7 (keys 448..511)
    is the diagonal tile of waves 6 and 7 of the query tile at 256..511, the
    waves whose last tile is the item's last: they take that tile's P V in
    the same step, after its correction.  128 heads at S=1024 causal run
    8-wave workgroups."""
    p = diagonal_keys(d, scale)
    o = run(p, "flash").cpu().numpy()
    compare(o, oracle_full(p), p.dtype, f"last-waves-diagonal/d{d}/x{int(scale)}")


# A steady tile whose probabilities are each finite but whose sum is not:
# the scores of every key past the first tile sit 126.4-127.8 log2 units
# above the reference, so each probability is finite in fp32 and in bf16 and
# a lane's sum of 32 of them overflows fp32 (flash_cases.sum_overflow_problem).
# The correction has to take the sum again from the corrected probabilities;
# scaling the infinite sum would give l = inf and a zero output.

@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_flash_steady_tile_sum_overflowing_fp32(d, causal):
    p = sum_overflow_problem(d, causal)
    o = run(p, "flash").cpu().numpy()
    compare(o, oracle_full(p), p.dtype, f"sum-overflow/d{d}/{'c' if causal else 'nc'}")


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_flash_later_probabilities_underflowing_below_the_margin(d, causal):
    """The first tile's keys scaled by 64: with the reference a margin above
    its maximum, every later probability underflows (flash_cases), and the
    output must still match the oracle, finite, on every row."""
    p = first_tile_dominant(d, causal)
    o = run(p, "flash").cpu().numpy()
    compare(o, oracle_full(p), p.dtype, f"first-tile-dominant/d{d}/{'c' if causal else 'nc'}")


# ---------------------------------------------------------------- invariants through the GPU

@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("dtype", [inputs.F32, inputs.BF16])
def test_identical_value_rows_give_that_row(variant, dtype):
    torch = torch_cuda()
    p = inputs.make_problem(1, 2, 300, 64, dtype, causal=True, seed=3)
    p.v[:] = p.v[:, :1, :]
    o = run(p, variant).cpu().numpy()
    want = np.broadcast_to(p.v[:, :1, :].astype(np.float64), o.shape)
    # a convex combination of identical rows: only the P V rounding remains
    compare(o, want, dtype, f"identical-rows/{dtype}/{variant}")


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_prefix_mean(variant, causal):
    p = inputs.make_problem(1, 2, 257, 32, inputs.F32, causal=causal, seed=4)
    p.q[:] = 0
    o = run(p, variant).cpu().numpy()
    v = p.v.astype(np.float64)
    if causal:
        want = np.cumsum(v, axis=1) / np.arange(1, p.S + 1)[None, :, None]
    else:
        want = np.broadcast_to(v.mean(axis=1, keepdims=True), v.shape)
    compare(o, want, inputs.F32, f"zero-query/{'c' if causal else 'nc'}/{variant}")


def test_naive_probability_rows_sum_to_one():
    torch = torch_cuda()
    for causal in (False, True):
        p = inputs.make_problem(1, 2, 333, 64, inputs.BF16, causal=causal, seed=5)
        need = kb.workspace_size(p.B, p.H, p.S, p.d, dtype="bf16")
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
        run(p, "naive", workspace=ws)
        P = ws.view(torch.float32).view(p.BH, p.S, p.S).double().cpu().numpy()
        assert np.all(np.isfinite(P)) and np.all(P >= 0)
        np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-5)
        if causal:
            iu = np.triu_indices(p.S, 1)
            assert np.all(P[:, iu[0], iu[1]] == 0.0)


@pytest.mark.parametrize("variant", VARIANTS)
def test_repeat_runs_are_bit_identical(variant):
    p = inputs.make_problem(2, 4, 700, 128, inputs.BF16, causal=True, seed=6)
    a = run(p, variant).cpu().numpy()
    b = run(p, variant).cpu().numpy()
    assert np.array_equal(a, b)


def test_bench_batched_mean_without_per_launch_events():
    """kb_bench_attention with no per-launch array records only the two outer
    events (the batched mean); the launches still compute the right output,
    and a NULL total is rejected."""
    import ctypes
    torch = torch_cuda()
    p = inputs.make_problem(1, 4, 300, 64, inputs.BF16, causal=True, seed=5)
    q, k, v = to_device(p)
    o = nan_output(p)
    cfg = kb.make_cfg(p.B, p.H, p.S, p.d, True, kb.KB_BF16)
    stream = int(torch.cuda.current_stream().cuda_stream)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr())
    per, tot = kb.kb_bench_attention(cfg, *ptrs, "flash", stream, 1, 20)
    assert len(per) == 20 and all(x > 0 for x in per) and tot >= sum(per) * 0.99
    o.fill_(float("nan"))
    per2, tot2 = kb.kb_bench_attention(cfg, *ptrs, "flash", stream, 0, 20, per_launch=False)
    assert per2 == [] and tot2 > 0
    compare(o.cpu().numpy(), oracle_full(p), p.dtype, "bench-batched/flash")
    st = kb.lib().kb_bench_attention(ctypes.byref(cfg), *ptrs, kb.KB_FLASH, stream, 0, 5, None, None)
    assert st == 1  # KB_ERR_INVALID


def test_concurrent_host_threads_match_serial():
    """Four host threads, each on its own stream, run flash on the same
    inputs at once (the ctypes call releases the interpreter lock); every
    output equals the serial one bit for bit."""
    import threading

    torch = torch_cuda()
    p = inputs.make_problem(1, 4, 1024, 128, inputs.BF16, causal=True, seed=5)
    q, k, v = to_device(p)
    ref = nan_output(p)
    kb.attention(q, k, v, ref, causal=True, variant="flash", heads=p.H)
    torch.cuda.synchronize()
    outs = [nan_output(p) for _ in range(4)]
    streams = [torch.cuda.Stream() for _ in range(4)]
    errors = []

    def work(i):
        try:
            for _ in range(5):
                kb.attention(q, k, v, outs[i], causal=True, variant="flash", heads=p.H, stream=streams[i])
        except Exception as e:  # reported below, on the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for o in outs:
        assert torch.equal(o, ref)


def test_variants_agree_with_each_other():
    p = inputs.make_problem(1, 4, 1024, 64, inputs.F32, causal=True, seed=7)
    outs = {v: run(p, v).cpu().numpy() for v in VARIANTS}
    for v in ("naive", "fused"):
        assert np.max(np.abs(outs[v] - outs["flash"])) <= 2e-5


def test_explicit_scale_and_4d_layout():
    torch = torch_cuda()
    p = inputs.make_problem(2, 3, 150, 64, inputs.F32, causal=False, seed=8)
    q, k, v = (t.view(2, 3, 150, 64) for t in to_device(p))
    for variant in VARIANTS:
        o = kb.attention(q, k, v, causal=False, variant=variant, scale=0.3)
        torch.cuda.synchronize()
        want = oracle.sdpa(p.q, p.k, p.v, causal=False, scale=0.3)
        compare(o.view(p.BH, p.S, p.d).cpu().numpy(), want, inputs.F32, f"scale0.3/{variant}")


# ---------------------------------------------------------------- errors on the device

def test_fused_reports_lds_limit():
    torch = torch_cuda()
    info = kb.kb_device_info()
    S = info["max_lds_per_block"] // 4 + 64
    q = torch.zeros((1, S, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kb.KbError) as ei:
        kb.attention(q, q.clone(), q.clone(), variant="fused")
    assert ei.value.status == 2


def test_device_info_is_gfx950():
    torch_cuda()
    info = kb.kb_device_info()
    print(f"[device] {info}", flush=True)
    assert info["arch"].startswith("gfx950")
    assert info["compute_units"] > 0


def test_compute_ceiling_probes_run():
    """The ceiling probes run on the device and report sane rates and clocks."""
    torch = torch_cuda()
    work = torch.empty(kb.kb_ceiling_work_size(), dtype=torch.uint8, device="cuda")
    cus = kb.kb_device_info()["compute_units"]
    # per clock per CU (bytes for the memory probes: generous upper bounds)
    bound = {"mfma_bf16": 4096, "mfma_f32": 256, "fma_f32": 128, "exp_f32": 128, "lds_read": 512,
             "l1_read": 512, "l2_read": 512, "mfma_bf16_data": 4096, "mfma_bf16_fma3": 4096,
             "mfma_bf16_exp3": 4096, "mfma_bf16_exp4": 4096, "mfma_bf16_lds": 4096}
    for kind in kb.CEILINGS:
        per, ops, mhz = kb.kb_bench_ceiling(kind, 200, work.data_ptr(), work.numel(), 0, 1, 2)
        rate = ops / (min(per) * 1e-3)
        print(f"[ceiling] {kind}: {rate / 1e12:.1f} T/s at {mhz:.0f} MHz", flush=True)
        assert 300 < mhz < 3000
        assert 0 < rate <= bound[kind] * cus * 3.0e9
    with pytest.raises(kb.KbError) as ei:
        kb.kb_bench_ceiling("mfma_bf16", 10, work.data_ptr(), 16, 0, 0, 1)
    assert ei.value.status == 3


def test_bandwidth_kernels_move_the_right_bytes():
    """copy writes b into a, write fills a with s, read (with s = NaN) leaves a
    untouched; the triad matches b + s c."""
    torch = torch_cuda()
    n = (1 << 20) + 12
    b = torch.rand(n, device="cuda")
    c = torch.rand(n, device="cuda")
    for kind in ("copy", "read", "write"):
        a = torch.full((n,), -7.0, device="cuda")
        s = float("nan") if kind == "read" else 2.5
        kb.kb_bench_stream(kind, a.data_ptr(), b.data_ptr(), s, n, 256, 0, 1, 2)
        torch.cuda.synchronize()
        want = {"copy": b, "read": torch.full_like(a, -7.0), "write": torch.full_like(a, 2.5)}[kind]
        assert torch.equal(a, want), kind
    a = torch.empty(n, device="cuda")
    kb.triad(a, b, c, 1.5)
    torch.cuda.synchronize()
    assert torch.allclose(a, b + 1.5 * c, rtol=0, atol=1e-6)


def test_triad_values_at_the_calibration_size_and_on_tails():
    """The triad at the calibration's 2 GiB working set, and on lengths and
    offsets that take its scalar path: an aligned length with a 3-element
    tail (vector body plus scalar tail) and buffers one element off 16-byte
    alignment (scalar throughout).  s = 2 makes s * c exact, so the fused
    multiply-add equals b + 2 c bit for bit."""
    torch = torch_cuda()
    n = 2048 * 1024 * 1024 // 12
    n -= n % 4
    b = torch.rand(n, device="cuda")
    c = torch.rand(n, device="cuda")
    a = torch.full((n,), float("nan"), device="cuda")
    for block in (64, 1024):
        a.fill_(float("nan"))
        kb.triad(a, b, c, 2.0, block=block)
        torch.cuda.synchronize()
        assert torch.equal(a, b + 2.0 * c), f"2 GiB, block {block}"
    del a, b, c
    torch.cuda.empty_cache()
    m = (1 << 20) + 7
    b = torch.rand(m + 1, device="cuda")
    c = torch.rand(m + 1, device="cuda")
    for off, label in ((0, "vector body + 3-element tail"), (1, "misaligned, scalar")):
        a = torch.full((m + 1,), float("nan"), device="cuda")
        kb.triad(a[off:off + m], b[off:off + m], c[off:off + m], 2.0)
        torch.cuda.synchronize()
        want = b[off:off + m] + 2.0 * c[off:off + m]
        assert torch.equal(a[off:off + m], want), label
        untouched = a[m:] if off == 0 else a[:1]
        assert torch.isnan(untouched).all(), f"{label}: wrote outside the range"


def test_binding_rejects_host_output_and_workspace():
    """attention() refuses an output or workspace tensor that is not on Q's
    GPU before anything is launched (its address would be a host pointer in
    the kernels)."""
    torch = torch_cuda()
    p = inputs.make_problem(1, 2, 64, 32, inputs.F32, seed=3)
    q, k, v = to_device(p)
    with pytest.raises(ValueError):
        kb.attention(q, k, v, torch.empty(q.shape, dtype=torch.float32), variant="flash")
    with pytest.raises(ValueError):
        kb.attention(q, k, v, variant="naive", workspace=torch.empty(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError):
        kb.attention(q, k.cpu(), v, variant="flash")
