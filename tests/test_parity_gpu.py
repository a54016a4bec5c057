"""GPU path against the oracle, element by element, through the C ABI.

Tolerances: max-abs error on out of 1e-4 with binary32 storage and 2e-2
with bfloat16 storage (binary32 arithmetic); y from spectre_mix_y within
1e-4 * max(1, max|y|).  The workloads are the five seeded shapes; the edge
cases cover tiny and ragged lengths, every plan shape (single-level,
two-level, three-level, radix-3 in each position), widths that do and do
not fuse the LayerNorm, and the truncation extremes.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (DeviceInputs, empty_like_storage, oracle_out, oracle_threads, run_out,
                      run_y, to_host_f64, tol, torch, y_tol)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_full(w, keep=None, check_y=True):
    say("case", w.describe(), "keep", keep)
    inp = workloads.make_inputs(w)
    ref_out, ref_y = oracle_out(w, inp, keep, want_y=True)
    got = run_out(w, inp, keep)
    err = np.abs(got - ref_out).max()
    say("  out max-abs err %.3g (tol %.1g), max|ref| %.3f" % (err, tol(w), np.abs(ref_out).max()))
    assert np.all(np.isfinite(got))
    assert err <= tol(w)
    if check_y:
        gy = run_y(w, inp, keep)
        ey = np.abs(gy - ref_y).max()
        say("  y max-abs err %.3g (tol %.3g)" % (ey, y_tol(ref_y)))
        assert ey <= y_tol(ref_y)


@pytest.mark.parametrize("wid", [1, 2, 3, 4])
def test_workload_full(wid):
    check_full(workloads.WORKLOADS[wid])


def c1_row_tokens(w):
    """One token of every row the last inverse pass handles: that pass runs one
    workgroup per (b, m), m < M = L2 * L3, over the tokens n1 * M + m; token
    m + M * (m mod L1) takes each m once and every n1 in turn, plus the batch
    boundaries and the sample of workloads.sample_tokens."""
    import efficient_attention_fft_amd as sm
    st, (l1, l2, l3) = sm.spectre_mix_plan(w.L)
    assert st == 0
    M = l2 * l3
    m = np.arange(M, dtype=np.int64)
    rows = np.concatenate([b * w.L + m + M * (m % l1) for b in range(w.B)])
    return np.unique(np.concatenate([rows, workloads.sample_tokens(w, 48)]))


@pytest.mark.timeout(900)
def test_workload5_sampled_tokens():
    """786432 tokens (64 x 12 x 1024): the oracle transforms every column in
    full and keeps one token of each of the 12288 rows of the last inverse
    pass (every workgroup of it, each of its 64 token positions in turn); the
    GPU output and y are compared at those tokens."""
    w = workloads.WORKLOADS[5]
    say("case", w.describe(), "(one token per C1 row)")
    t = torch()
    inp = workloads.make_inputs(w)
    toks = c1_row_tokens(w)
    assert len(toks) >= 12288
    ref_out, ref_y = oracle.spectre_mix_tokens(inp["q"], inp["k"], inp["v"], inp["x"],
                                               inp["gate"], inp["gamma"], inp["beta"],
                                               w.keep_bins, toks, nthreads=oracle_threads())
    d = DeviceInputs(w, inp)
    _, out = empty_like_storage(w)
    import efficient_attention_fft_amd as sm
    sm.check(d.fwd(out))
    t.cuda.synchronize()
    sel = t.from_numpy(toks).cuda()
    got = to_host_f64(out.view(w.tokens, w.C)[sel], w.dtype).reshape(-1, w.H, w.D)
    err = np.abs(got - ref_out).max()
    say("  out max-abs err %.3g over %d tokens" % (err, len(toks)))
    assert err <= tol(w)
    del out
    y = t.empty((w.N,), dtype=t.float32, device="cuda")
    sm.check(d.y(y))
    t.cuda.synchronize()
    gy = y.view(w.tokens, w.C)[sel].cpu().numpy().astype(np.float64).reshape(-1, w.H, w.D)
    ey = np.abs(gy - ref_y).max()
    say("  y max-abs err %.3g (tol %.3g)" % (ey, y_tol(ref_y)))
    assert ey <= y_tol(ref_y)


EDGE = [
    # (B, L, H, D, dtype, keep)  keep None = no truncation
    (1, 2, 1, 2, 0, None),
    (2, 4, 1, 2, 0, None),
    (1, 6, 2, 1, 0, None),
    (3, 8, 1, 6, 0, 3),
    (1, 12, 2, 2, 1, None),
    (2, 24, 2, 4, 0, 5),
    (1, 96, 3, 2, 0, None),         # head size 2, odd head count
    (1, 256, 1, 32, 0, 0),          # keep 0: out = LayerNorm(x)
    (1, 256, 2, 16, 0, 1),          # only the DC bin
    (1, 1536, 4, 8, 1, 700),
    (2, 4096, 2, 8, 0, 2048),       # Nyquist dropped (one pass: 16 x 16 x 16 column kernel)
    (1, 3072, 2, 32, 0, None),      # one pass, 12 x 16 x 16
    (1, 2048, 2, 64, 0, 700),       # the longest single-level column
    (1, 6144, 2, 64, 0, None),      # two-level, radix 3 in the strided pass (l1 = 6)
    (2, 8192, 4, 32, 1, 1000),      # two-level, fused norm, bf16
    (1, 12288, 1, 6, 0, None),      # two-level, narrow: separate norm pass
    (1, 49152, 2, 64, 0, 20000),    # two-level, l1 = 48
    (1, 98304, 2, 64, 0, None),     # three-level, l2 = 3
    (1, 196608, 1, 128, 1, 50000),  # three-level, l2 = 6
    (1, 16384, 4, 256, 0, None),    # H*D = 1024: separate norm pass
    (1, 4096, 2, 5, 0, None),       # channel pairs straddle heads (odd D), ragged pair block
    (2, 65536, 4, 64, 0, None),     # LDS-copy B kernel, 4 work items per workgroup across batches
    (1, 65536, 4, 64, 1, 30000),    # LDS-copy B kernel, 2 work items per workgroup, bf16, truncated
    (1, 8192, 32, 6, 0, None),      # tiled input, 4-pair blocks spanning heads: gate from the table
]


@pytest.mark.parametrize("B,L,H,D,dt,keep", EDGE)
def test_edge_shapes(B, L, H, D, dt, keep):
    kb = L // 2 + 1 if keep is None else keep
    w = workloads.custom(200 + L % 97, B=B, L=L, H=H, D=D, dtype=dt, keep_bins=kb, affine=True)
    check_full(w)


# The single-pass column kernel (L = 3072, 4096): ragged last pair blocks
# (CP2 = 9, 1, 3, 5), heads that split pairs, bfloat16 storage, truncation
# down to keep 0 and 1, several batch elements.
COLUMN = [
    (3, 4096, 3, 6, 0, None),       # CP2 = 9: last block holds one live pair
    (1, 4096, 8, 64, 1, 1000),      # bf16, truncated
    (2, 3072, 4, 10, 0, 777),
    (1, 3072, 1, 2, 0, None),       # a single pair
    (2, 3072, 2, 6, 1, None),       # CP2 = 6, bf16
    (1, 4096, 1, 2, 0, 1),          # a single pair, the DC bin only
    (1, 4096, 3, 2, 0, 0),          # CP2 = 3, keep 0: out = LayerNorm(x)
    (2, 3072, 8, 64, 0, None),
    (5, 4096, 2, 64, 0, 2049),
]

# Past one round of the column kernel (B * CP2 / 4 > 256): the same lengths
# take the four-step plan.
PAST_ONE_ROUND = [
    (5, 4096, 8, 64, 0, 1500),
    (2, 3072, 16, 64, 1, None),
]


@pytest.mark.parametrize("B,L,H,D,dt,keep", PAST_ONE_ROUND)
def test_column_lengths_past_one_round(B, L, H, D, dt, keep):
    kb = L // 2 + 1 if keep is None else keep
    w = workloads.custom(510 + L % 83, B=B, L=L, H=H, D=D, dtype=dt, keep_bins=kb, affine=True)
    check_full(w)


@pytest.mark.parametrize("B,L,H,D,dt,keep", COLUMN)
def test_column_kernel_shapes(B, L, H, D, dt, keep):
    import efficient_attention_fft_amd as sm
    assert sm.spectre_mix_plan(L) == (sm.SPECTRE_OK, (1, 1, L))
    kb = L // 2 + 1 if keep is None else keep
    w = workloads.custom(500 + L % 83, B=B, L=L, H=H, D=D, dtype=dt, keep_bins=kb, affine=True)
    check_full(w)


def _column_sweep(n=10, seed=777):
    """Seeded random shapes for the column kernel: L = 3072 or 4096, any even
    H*D up to 512, B within one round (B * ceil(H*D/8) <= 256), both dtypes,
    any keep_bins."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        L = int(rng.choice([3072, 4096]))
        H, D = int(rng.integers(1, 9)), int(rng.integers(1, 65))
        if (H * D) % 2:
            continue
        B = int(rng.integers(1, 5))
        if B * ((H * D // 2 + 3) // 4) > 256:
            continue
        cases.append((B, L, H, D, int(rng.integers(0, 2)), int(rng.integers(0, L // 2 + 2))))
    return cases


@pytest.mark.parametrize("B,L,H,D,dt,keep", _column_sweep())
def test_column_kernel_sweep(B, L, H, D, dt, keep):
    import efficient_attention_fft_amd as sm
    assert sm.spectre_mix_plan(L) == (sm.SPECTRE_OK, (1, 1, L))
    w = workloads.custom(530 + L % 79, B=B, L=L, H=H, D=D, dtype=dt, keep_bins=keep, affine=True)
    check_full(w)


def test_both_plans_of_one_length_in_one_process():
    """L = 4096 in one round (column kernel), past it (four-step) and in one
    round again, in one process: each plan must get its own tables."""
    for i, (B, H) in enumerate([(1, 8), (5, 8), (2, 4)]):
        w = workloads.custom(520 + i, B=B, L=4096, H=H, D=64, keep_bins=1800, affine=True)
        check_full(w, check_y=False)


def _sweep_cases(n=20, seed=4242):
    """Seeded random supported shapes: L = 2^a 3^b (b <= 1), H * D even, any
    keep_bins, both dtypes, at most about 2^22 elements per tensor."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        L = int(2 ** rng.integers(1, 17) * (3 if rng.random() < 0.3 else 1))
        H, D, B = int(rng.integers(1, 9)), int(rng.integers(1, 65)), int(rng.integers(1, 4))
        if (H * D) % 2 or B * L * H * D > 2 ** 22 or L > 3 * 2 ** 20:
            continue
        cases.append((B, L, H, D, int(rng.integers(0, 2)), int(rng.integers(0, L // 2 + 2))))
    return cases


@pytest.mark.parametrize("B,L,H,D,dt,keep", _sweep_cases())
def test_sweep_shapes(B, L, H, D, dt, keep):
    w = workloads.custom(300 + L % 89, B=B, L=L, H=H, D=D, dtype=dt, keep_bins=keep, affine=True)
    check_full(w)


@pytest.mark.timeout(600)
def test_longest_supported_length():
    """L = 3 * 2^20, the longest length the library plans: 64 x 48 x 1024,
    whose 48-point second pass runs in place in row layout."""
    import efficient_attention_fft_amd as sm
    st, plan = sm.spectre_mix_plan(3 * 2 ** 20)
    assert st == sm.SPECTRE_OK and plan == (64, 48, 1024)
    w = workloads.custom(303, B=1, L=3 * 2 ** 20, H=1, D=32, keep_bins=3 * 2 ** 19 + 1)
    check_full(w)


def test_truncated_band_matches_zeroed_gate_on_gpu():
    w = workloads.custom(301, B=1, L=65536, H=2, D=64, keep_bins=8193)
    inp = workloads.make_inputs(w)
    a = run_y(w, inp)
    inp2 = dict(inp)
    g = inp["gate"].copy()
    g[:, 8193:] = 0
    inp2["gate"] = g
    b = run_y(w, inp2, keep=w.L // 2 + 1)
    assert np.abs(a - b).max() <= 1e-6 * max(1.0, np.abs(b).max())


def test_deterministic_and_inputs_untouched():
    w = workloads.WORKLOADS[3]
    t = torch()
    inp = workloads.make_inputs(w)
    d = DeviceInputs(w, inp)
    before = [x.clone() for x in (d.q, d.k, d.v, d.x, d.gate, d.gamma, d.beta)]
    guard = 4096
    whole1, o1 = empty_like_storage(w, guard)
    whole2, o2 = empty_like_storage(w, guard)
    import efficient_attention_fft_amd as sm
    sm.check(d.fwd(o1))
    sm.check(d.fwd(o2))
    t.cuda.synchronize()
    assert t.equal(o1, o2), "two calls differ bitwise"
    for a, b in zip(before, (d.q, d.k, d.v, d.x, d.gate, d.gamma, d.beta)):
        assert t.equal(a, b), "an input was modified"
    for whole in (whole1, whole2):
        assert t.isnan(whole[:guard]).all() and t.isnan(whole[-guard:]).all(), \
            "write outside out"


def test_side_stream_and_release():
    w = workloads.WORKLOADS[2]
    t = torch()
    inp = workloads.make_inputs(w)
    ref = oracle_out(w, inp)
    d = DeviceInputs(w, inp)
    import efficient_attention_fft_amd as sm
    s = t.cuda.Stream()
    _, out = empty_like_storage(w)
    with t.cuda.stream(s):
        sm.check(d.fwd(out, stream=s))
    s.synchronize()
    assert np.abs(to_host_f64(out, w.dtype).reshape(ref.shape) - ref).max() <= tol(w)
    assert sm.spectre_mix_release() == sm.SPECTRE_OK
    _, out2 = empty_like_storage(w)
    sm.check(d.fwd(out2))
    t.cuda.synchronize()
    assert t.equal(out, out2)


def test_forced_allocation_failure_leaves_out_untouched(monkeypatch):
    w = workloads.custom(302, B=1, L=8192, H=2, D=64)
    t = torch()
    inp = workloads.make_inputs(w)
    d = DeviceInputs(w, inp)
    import efficient_attention_fft_amd as sm
    assert sm.spectre_mix_release() == sm.SPECTRE_OK
    monkeypatch.setenv("SPECTRE_MIX_FAIL_ALLOC", "1")
    _, out = empty_like_storage(w)
    assert d.fwd(out) == sm.SPECTRE_ENOMEM
    t.cuda.synchronize()
    assert t.isnan(out).all()
    monkeypatch.delenv("SPECTRE_MIX_FAIL_ALLOC")
    sm.check(d.fwd(out))
    t.cuda.synchronize()
    assert not t.isnan(out).any()
