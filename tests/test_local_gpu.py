"""The local branch on the GPU against the oracle: the sliding-window
attention alone (spectre_mix_local_attention) and the mix with it
(spectre_mix_fwd_local, out = LN(x + y + y_loc)), the SPECTRE article's
use_local_branch (section 3.2) and its FFT-plus-window hybrid (section 4.3).

Tolerances: out max-abs 1e-4 (binary32 storage), 2e-2 (bfloat16 storage), as
for the plain mix; y_loc within 1e-4 * max(1, max|y_loc|).  The MFMA products
run on split bfloat16 operands (hi + lo), about 2^-16 relative per product,
well inside 1e-4.

Windows: 128 and 256 keys (the article's sizes), one-sided (wr = 0),
asymmetric, a window of one key (y_loc = v), one longer than the sequence
(full attention); lengths with a ragged last 32-query tile, L = 1, and every
head size the kernel takes (16, 32, 64, 128).
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import dev, empty_like_storage, oracle_threads, to_host_f64, tol, torch, y_tol

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_local(sm, inp, w, wl, wr):
    t = torch()
    q, k, v = (dev(inp[n]) for n in "qkv")
    y = t.full((w.N,), float("nan"), dtype=t.float32, device="cuda")
    sm.check(sm.spectre_mix_local_attention(q, k, v, y, w.B, w.H, w.L, w.D, wl, wr, w.dtype))
    t.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64).reshape(w.B, w.L, w.H, w.D)


ATTN_CASES = [
    # (B, L, H, D, dtype, win_left, win_right)
    (1, 256, 2, 16, 0, 64, 64),       # window 128 on the tiny shape
    (2, 300, 2, 64, 0, 20, 5),        # ragged last tile, asymmetric
    (1, 1000, 4, 32, 1, 127, 0),      # one-sided (causal-style) window, bfloat16
    (1, 97, 1, 128, 0, 500, 500),     # window longer than the sequence: full attention
    (1, 1, 1, 16, 0, 3, 3),           # one token
    (2, 4096, 8, 64, 0, 64, 64),      # 4096-token shape, window 128
    (1, 4096, 8, 64, 1, 128, 128),    # window 256, bfloat16
    (3, 33, 3, 32, 0, 0, 40),         # B * tiles * H not a multiple of 8, look-ahead only
    (1, 300, 2, 128, 1, 64, 64),      # head size 128 in bfloat16
    (2, 520, 4, 16, 1, 200, 31),      # head size 16 in bfloat16, ragged, asymmetric
]


@pytest.mark.parametrize("B,L,H,D,dt,wl,wr", ATTN_CASES)
def test_local_attention_against_oracle(B, L, H, D, dt, wl, wr):
    import efficient_attention_fft_amd as sm
    w = workloads.custom(600 + L % 97, B=B, L=L, H=H, D=D, dtype=dt, keep_bins=L // 2 + 1)
    say("case", w.describe(), "window", wl, wr)
    inp = workloads.make_inputs(w)
    ref = oracle.local_attention(inp["q"], inp["k"], inp["v"], wl, wr, dtype=dt)
    got = run_local(sm, inp, w, wl, wr)
    err = np.abs(got - ref).max()
    say("  y_loc max-abs err %.3g (tol %.3g)" % (err, y_tol(ref)))
    assert np.all(np.isfinite(got)) and err <= y_tol(ref)


def _sweep_cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        L = int(rng.integers(1, 700))
        cases.append((int(rng.integers(1, 3)), L, int(rng.integers(1, 5)),
                      int(rng.choice([16, 32, 64, 128])), int(rng.integers(0, 2)),
                      int(rng.integers(0, 300)), int(rng.integers(0, 300))))
    return cases


@pytest.mark.parametrize("B,L,H,D,dt,wl,wr", _sweep_cases())
def test_local_attention_sweep(B, L, H, D, dt, wl, wr):
    """Seeded random shapes and windows (lengths not multiples of the 32-
    or 128-token tiles, windows wider than the sequence, both dtypes, every
    head size), against the oracle."""
    import efficient_attention_fft_amd as sm
    w = workloads.custom(700 + L, B=B, L=L, H=H, D=D, dtype=dt, keep_bins=L // 2 + 1)
    inp = workloads.make_inputs(w)
    ref = oracle.local_attention(inp["q"], inp["k"], inp["v"], wl, wr, dtype=dt)
    got = run_local(sm, inp, w, wl, wr)
    err = np.abs(got - ref).max()
    assert np.all(np.isfinite(got)) and err <= y_tol(ref), (err, y_tol(ref))


def test_window_of_one_key_is_v():
    """win_left = win_right = 0: each query sees only itself, so y_loc = v, to
    the split-bfloat16 representation of v (hi + lo carries 16 significant
    bits; 2^-16 relative bounds it)."""
    import efficient_attention_fft_amd as sm
    w = workloads.custom(611, B=1, L=200, H=2, D=64, dtype=0, keep_bins=101)
    inp = workloads.make_inputs(w)
    got = run_local(sm, inp, w, 0, 0)
    v = inp["v"].astype(np.float64).reshape(got.shape)
    err = np.abs(got - v).max()
    say("  one-key window: max |y_loc - v| %.3g" % err)
    assert err <= 2.0 ** -16 * np.abs(v).max()


def tile_tokens(w, salt=0):
    """One query of every 32-query tile of the branch's kernel in every batch
    element (position (tile + salt) mod 32 within the tile), plus each
    sequence's first and last tokens."""
    picks = []
    for b in range(w.B):
        tiles = np.arange((w.L + 31) // 32, dtype=np.int64)
        t = np.minimum(32 * tiles + (tiles + salt + b) % 32, w.L - 1)
        picks.append(b * w.L + np.concatenate([t, [0, w.L - 1]]))
    return np.unique(np.concatenate(picks))


def test_local_attention_full_size_sampled():
    """The 65536-token shape (B=1, H=8, D=64, binary32), window 128: the
    oracle computes one query of every 32-query tile (2048 tokens) and the
    edges."""
    import efficient_attention_fft_amd as sm
    w = workloads.WORKLOADS[3]
    inp = workloads.make_inputs(w)
    wl = wr = 64
    got = run_local(sm, inp, w, wl, wr)
    toks = tile_tokens(w, salt=5)
    ref = oracle.local_attention_tokens(inp["q"], inp["k"], inp["v"], wl, wr, toks)
    worst = np.abs(got.reshape(w.B * w.L, w.H, w.D)[toks] - ref).max()
    say("  sampled y_loc max-abs err %.3g over %d tokens" % (worst, len(toks)))
    assert worst <= 1e-4


MIX_CASES = [
    # (B, L, H, D, dtype, keep_bins, win_left, win_right)
    (1, 256, 2, 16, 0, 129, 64, 64),       # single-level square kernel
    (1, 1536, 2, 32, 1, 700, 64, 64),      # single-level generic LDS kernel (radix 3), bf16
    (2, 4096, 8, 64, 0, 2049, 64, 64),     # single-pass column kernel, window 128
    (1, 16384, 2, 32, 0, 3000, 128, 128),  # two-level plan, window 256
    (1, 16384, 8, 64, 1, 4097, 64, 63),    # bfloat16, LDS-copy B kernel
    (1, 98304, 1, 32, 0, 49153, 100, 0),   # three-level plan (32 x 3 x 1024), one-sided
    (1, 49152, 8, 64, 1, 12289, 128, 0),   # 48 x 1024: the split fused inverse adds y_loc, bf16
]


@pytest.mark.parametrize("B,L,H,D,dt,keep,wl,wr", MIX_CASES)
def test_mix_with_local_branch_against_oracle(B, L, H, D, dt, keep, wl, wr):
    import efficient_attention_fft_amd as sm
    t = torch()
    w = workloads.custom(620 + L % 89, B=B, L=L, H=H, D=D, dtype=dt, keep_bins=keep, affine=True)
    say("case", w.describe(), "window", wl, wr)
    inp = workloads.make_inputs(w)
    ref = oracle.spectre_mix_local(inp["q"], inp["k"], inp["v"], inp["x"], inp["gate"],
                                   inp["gamma"], inp["beta"], keep, wl, wr, dtype=dt,
                                   nthreads=oracle_threads())
    q, k, v, x = (dev(inp[n]) for n in "qkvx")
    g, gam, bet = dev(inp["gate"]), dev(inp["gamma"]), dev(inp["beta"])
    _, out = empty_like_storage(w)
    sm.check(sm.spectre_mix_fwd_local(q, k, v, x, g, gam, bet, out, B, H, L, D, keep, wl, wr, dt))
    t.cuda.synchronize()
    got = to_host_f64(out, dt).reshape(ref.shape)
    err = np.abs(got - ref).max()
    say("  out max-abs err %.3g (tol %.1g)" % (err, tol(w)))
    assert np.all(np.isfinite(got)) and err <= tol(w)


VARIANT_CASES = [
    # (B, L, H, D, dtype, keep_bins, win_left, win_right, gate_kind, norm_order)
    (1, 16384, 8, 64, 0, 4097, 64, 64, 2, 1),    # 16 x 1024, fused inverse, complex gate, pre-norm
    (1, 65536, 4, 64, 0, 30000, 64, 64, 1, 1),   # 64 x 1024, split fused inverse, logit gate, pre
    (2, 4096, 4, 32, 1, 1000, 128, 0, 2, 0),     # column kernel, bf16, complex gate, post
    (1, 2048, 2, 16, 0, 900, 40, 40, 1, 1),      # single level, LayerNorm pass, logit gate, pre
    (1, 16384, 2, 32, 0, 3000, 64, 63, 0, 1),    # unfused inverse + LayerNorm pass, pre
]


@pytest.mark.parametrize("B,L,H,D,dt,keep,wl,wr,gk,no", VARIANT_CASES)
def test_mix_with_local_branch_variants(B, L, H, D, dt, keep, wl, wr, gk, no):
    """spectre_mix_fwd_local_ex: the local branch with the logit and complex
    gates and the pre-norm order, on each inverse / norm path."""
    import efficient_attention_fft_amd as sm
    t = torch()
    w = workloads.custom(640 + L % 83, B=B, L=L, H=H, D=D, dtype=dt, keep_bins=keep, affine=True)
    say("case", w.describe(), "window", wl, wr, "gate kind", gk, "norm order", no)
    inp = workloads.make_inputs(w)
    gate = workloads.make_gate(w, gk)
    ref = oracle.spectre_mix_local(inp["q"], inp["k"], inp["v"], inp["x"], gate, inp["gamma"],
                                   inp["beta"], keep, wl, wr, dtype=dt, nthreads=oracle_threads(),
                                   gate_kind=gk, norm_order=no)
    q, k, v, x = (dev(inp[n]) for n in "qkvx")
    g, gam, bet = dev(gate), dev(inp["gamma"]), dev(inp["beta"])
    _, out = empty_like_storage(w)
    sm.check(sm.spectre_mix_fwd_local_ex(q, k, v, x, g, gam, bet, out, B, H, L, D, keep, wl, wr,
                                         dt, gk, no))
    t.cuda.synchronize()
    got = to_host_f64(out, dt).reshape(ref.shape)
    err = np.abs(got - ref).max()
    say("  out max-abs err %.3g (tol %.1g)" % (err, tol(w)))
    assert np.all(np.isfinite(got)) and err <= tol(w)


GATED_CASES = [
    # (B, L, H, D, dtype, keep_bins, win_left, win_right, gate_kind, norm_order)
    (1, 16384, 8, 64, 0, 4097, 64, 64, 0, 0),    # 16 x 1024, fused inverse, LayerNorm
    (1, 65536, 4, 64, 0, 30000, 64, 64, 0, 3),   # 64 x 1024, split fused inverse, pre RMSNorm
    (1, 49152, 8, 64, 1, 12289, 128, 0, 1, 2),   # 48 x 1024, split, bf16, logit gate, RMSNorm
    (1, 2048, 2, 16, 0, 900, 40, 40, 2, 1),      # single level, LayerNorm pass, complex gate, pre
    (1, 16384, 2, 32, 0, 3000, 64, 63, 0, 2),    # unfused inverse + norm pass, RMSNorm
    (2, 4096, 8, 64, 0, 2049, 64, 64, 2, 3),     # single-pass column kernel, pre RMSNorm
]


@pytest.mark.parametrize("B,L,H,D,dt,keep,wl,wr,gk,no", GATED_CASES)
def test_mix_with_gated_local_branch(B, L, H, D, dt, keep, wl, wr, gk, no):
    """spectre_mix_fwd_local_gated: the two branches weighted per channel
    (g y + (1 - g) y_loc, channel 0 at g = 1 and channel 1 at g = 0), on
    each inverse / norm path, with LayerNorm and RMSNorm in both orders."""
    import efficient_attention_fft_amd as sm
    t = torch()
    w = workloads.custom(660 + L % 79, B=B, L=L, H=H, D=D, dtype=dt, keep_bins=keep, affine=True)
    say("case", w.describe(), "window", wl, wr, "gate kind", gk, "norm order", no, "gated")
    inp = workloads.make_inputs(w)
    gate = workloads.make_gate(w, gk)
    mix = workloads.make_branch_mix(w)
    ref = oracle.spectre_mix_local_gated(inp["q"], inp["k"], inp["v"], inp["x"], gate, mix,
                                         inp["gamma"], inp["beta"], keep, wl, wr, dtype=dt,
                                         nthreads=oracle_threads(), gate_kind=gk, norm_order=no)
    q, k, v, x = (dev(inp[n]) for n in "qkvx")
    g, m, gam, bet = dev(gate), dev(mix), dev(inp["gamma"]), dev(inp["beta"])
    _, out = empty_like_storage(w)
    sm.check(sm.spectre_mix_fwd_local_gated(q, k, v, x, g, m, gam, bet, out, B, H, L, D, keep,
                                            wl, wr, dt, gk, no))
    t.cuda.synchronize()
    got = to_host_f64(out, dt).reshape(ref.shape)
    err = np.abs(got - ref).max()
    say("  out max-abs err %.3g (tol %.1g)" % (err, tol(w)))
    assert np.all(np.isfinite(got)) and err <= tol(w)


def test_gate_of_one_keeps_the_fft_branch_alone():
    """Every branch weight 1: the gated mix is the FFT mix without the local
    branch (spectre_mix_fwd_ex, RMSNorm post-norm), to rounding."""
    import efficient_attention_fft_amd as sm
    t = torch()
    w = workloads.custom(671, B=1, L=16384, H=4, D=64, dtype=0, keep_bins=5000, affine=True)
    inp = workloads.make_inputs(w)
    q, k, v, x = (dev(inp[n]) for n in "qkvx")
    g, gam, bet = dev(inp["gate"]), dev(inp["gamma"]), dev(inp["beta"])
    ones = dev(np.ones(w.C, np.float32))
    _, a = empty_like_storage(w)
    _, b = empty_like_storage(w)
    sm.check(sm.spectre_mix_fwd_ex(q, k, v, x, g, gam, bet, a, w.B, w.H, w.L, w.D, 5000, 0, 0, 2))
    sm.check(sm.spectre_mix_fwd_local_gated(q, k, v, x, g, ones, gam, bet, b, w.B, w.H, w.L, w.D,
                                            5000, 64, 64, 0, 0, 2))
    t.cuda.synchronize()
    err = (a - b).abs().max().item()
    say("  gate 1 vs FFT branch alone: max-abs diff %.3g" % err)
    assert err <= 1e-5


def test_local_plain_entry_is_the_real_post_variant():
    """spectre_mix_fwd_local and spectre_mix_fwd_local_ex(REAL, POST) agree bit for bit."""
    import efficient_attention_fft_amd as sm
    t = torch()
    w = workloads.custom(655, B=1, L=16384, H=4, D=64, dtype=0, keep_bins=5000, affine=True)
    inp = workloads.make_inputs(w)
    q, k, v, x = (dev(inp[n]) for n in "qkvx")
    g, gam, bet = dev(inp["gate"]), dev(inp["gamma"]), dev(inp["beta"])
    _, a = empty_like_storage(w)
    _, b = empty_like_storage(w)
    sm.check(sm.spectre_mix_fwd_local(q, k, v, x, g, gam, bet, a, w.B, w.H, w.L, w.D, 5000, 64, 64, 0))
    sm.check(sm.spectre_mix_fwd_local_ex(q, k, v, x, g, gam, bet, b, w.B, w.H, w.L, w.D, 5000, 64,
                                         64, 0, 0, 0))
    t.cuda.synchronize()
    assert t.equal(a, b)


@pytest.mark.parametrize("wid,wl,wr", [(3, 64, 64), (4, 128, 128)])
def test_mix_with_local_branch_full_size_sampled(wid, wl, wr):
    """The 65536-token shapes (binary32, B = 1, window 128, the launch
    configuration the benchmark times; bfloat16, B = 2, truncated, window
    256): at one query of every 32-query tile of every batch element, the
    oracle's spectral y plus its windowed attention, through its residual
    LayerNorm."""
    import efficient_attention_fft_amd as sm
    t = torch()
    w = workloads.WORKLOADS[wid]
    inp = workloads.make_inputs(w)
    toks = tile_tokens(w, salt=7)
    _, ref_y = oracle.spectre_mix_tokens(inp["q"], inp["k"], inp["v"], inp["x"], inp["gate"],
                                         inp["gamma"], inp["beta"], w.keep_bins, toks,
                                         dtype=w.dtype, nthreads=oracle_threads())
    yl = oracle.local_attention_tokens(inp["q"], inp["k"], inp["v"], wl, wr, toks, dtype=w.dtype)
    xs = inp["x"].reshape(w.B * w.L, w.H, w.D)[toks]
    ref = oracle.layernorm_residual(ref_y + yl, xs, inp["gamma"], inp["beta"], dtype=w.dtype)
    q, k, v, x = (dev(inp[n]) for n in "qkvx")
    g, gam, bet = dev(inp["gate"]), dev(inp["gamma"]), dev(inp["beta"])
    _, out = empty_like_storage(w)
    sm.check(sm.spectre_mix_fwd_local(q, k, v, x, g, gam, bet, out, w.B, w.H, w.L, w.D,
                                      w.keep_bins, wl, wr, w.dtype))
    t.cuda.synchronize()
    got = to_host_f64(out.view(w.B * w.L, w.C)[t.from_numpy(toks).cuda()], w.dtype).reshape(ref.shape)
    err = np.abs(got - ref).max()
    say("  %s window %d/%d: out max-abs err %.3g over %d tokens" % (w.name, wl, wr, err, len(toks)))
    assert err <= tol(w)
