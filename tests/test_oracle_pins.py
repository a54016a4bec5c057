"""Pins for the CPU oracle: it is checked against things other than itself.

* its FFT against the DFT's definition, summed term by term;
* Hermitian symmetry and Parseval's identity at the workloads' lengths;
* the whole mix against the closed form the convolution theorem gives
  (SPECTRE article, section 2.1 and section 2.2): y = (1/L) g (*) (q * k) (*) v,
  with (q * k) the circular cross-correlation, (*) circular convolution and
  g the inverse real transform of the gate, brute-forced with plain loops;
* inputs with closed-form outputs (constants, alternating sign, one cosine,
  impulses) at the long lengths, with a different gate per head;
* shift covariance, trilinearity and truncation-as-zeroed-gate;
* LayerNorm on inputs whose mean and variance are known by construction.

None of these re-types the oracle's steps: each is an independent statement
that a mistake in it (a dropped term, a wrong sign, a swapped operand, a
wrong index or scale) would violate.
"""
import numpy as np
import pytest

import oracle
import workloads

RNG = np.random.default_rng(12345)


def naive_dft(x, sign=-1):
    """The DFT by its definition, one output at a time, exponents reduced mod n."""
    n = len(x)
    j = np.arange(n)
    out = np.empty(n, np.complex128)
    for f in range(n):
        e = (f * j) % n
        out[f] = np.sum(x * np.exp(sign * 2j * np.pi * e / n))
    return out


LENGTHS_SMALL = list(range(1, 65))


@pytest.mark.parametrize("n", LENGTHS_SMALL + [96, 192, 384, 768])
def test_fft_equals_dft_definition(n):
    x = RNG.standard_normal(n) + 1j * RNG.standard_normal(n)
    for sign in (-1, 1):
        ref = naive_dft(x, sign)
        got = oracle.fft(x, sign)
        scale = max(1.0, np.abs(ref).max())
        assert np.abs(got - ref).max() <= 1e-12 * scale * max(1, np.log2(n))


def test_fft_4096_spot_bins():
    n = 4096
    x = RNG.standard_normal(n)
    got = oracle.fft(x)
    j = np.arange(n)
    for f in (0, 1, 2, 3, 5, 1000, 2047, 2048, 2049, 4095):
        ref = np.sum(x * np.exp(-2j * np.pi * ((f * j) % n) / n))
        assert abs(got[f] - ref) <= 1e-11 * np.sqrt(n)


@pytest.mark.parametrize("n", [65536, 786432, 3 * 1024, 6])
def test_hermitian_symmetry_and_parseval(n):
    x = RNG.standard_normal(n)
    X = oracle.fft(x)
    norm = np.sqrt(np.sum(np.abs(X) ** 2))
    f = np.arange(1, n)
    assert np.abs(X[n - f] - np.conj(X[f])).max() <= 1e-12 * norm
    assert abs(X[0].imag) <= 1e-12 * norm
    if n % 2 == 0:
        assert abs(X[n // 2].imag) <= 1e-12 * norm
    lhs = np.sum(x * x)
    rhs = np.sum(np.abs(X) ** 2) / n
    assert abs(lhs - rhs) <= 1e-12 * lhs


def test_fft_linear_and_shift():
    n = 768
    a, b = RNG.standard_normal(n), RNG.standard_normal(n)
    A, Bf = oracle.fft(a), oracle.fft(b)
    assert np.allclose(oracle.fft(2 * a - 3 * b), 2 * A - 3 * Bf, atol=1e-10)
    s = 7
    f = np.arange(n)
    shifted = oracle.fft(np.roll(a, s))
    assert np.allclose(shifted, A * np.exp(-2j * np.pi * ((f * s) % n) / n), atol=1e-9)


# ---------------------------------------------------------------- closed form

def irfft_gate(G, keep, L):
    """g[t] = inverse real transform of the gate G[f] * [f < keep], f = 0..L//2,
    written as its cosine series (a real, even sequence)."""
    t = np.arange(L)
    g = np.zeros(L)
    for f in range(L // 2 + 1):
        if f >= keep:
            continue
        if f == 0:
            g += G[0]
        elif L % 2 == 0 and f == L // 2:
            g += G[f] * np.cos(np.pi * t)
        else:
            g += 2 * G[f] * np.cos(2 * np.pi * ((f * t) % L) / L)
    return g / L


def circ_xcorr(q, k):
    """r[m] = sum_n q[(n + m) mod L] k[n]."""
    L = len(q)
    return np.array([sum(q[(n + m) % L] * k[n] for n in range(L)) for m in range(L)])


def circ_conv(a, b):
    """(a (*) b)[t] = sum_s a[s] b[(t - s) mod L]."""
    L = len(a)
    return np.array([sum(a[s] * b[(t - s) % L] for s in range(L)) for t in range(L)])


def closed_form_y(q, k, v, gate, keep):
    """y[b, :, h, d] = (1/L) g_h (*) (q * k) (*) v for every column."""
    B, L, H, D = q.shape
    y = np.zeros((B, L, H, D))
    for h in range(H):
        g = irfft_gate(gate[h].astype(np.float64), keep, L)
        for b in range(B):
            for d in range(D):
                r = circ_xcorr(q[b, :, h, d], k[b, :, h, d])
                y[b, :, h, d] = circ_conv(g, circ_conv(r, v[b, :, h, d])) / L
    return y


@pytest.mark.parametrize("L,keep", [(1, 1), (2, 2), (3, 2), (4, 3), (5, 3), (6, 4), (8, 5),
                                    (8, 3), (12, 7), (16, 0), (17, 9), (17, 4), (48, 25),
                                    (48, 10), (64, 33), (64, 1)])
def test_mix_equals_closed_form(L, keep):
    B, H, D = 2, 2, 2
    q, k, v = (RNG.standard_normal((B, L, H, D)).astype(np.float32) for _ in range(3))
    gate = RNG.uniform(0, 1, (H, L // 2 + 1)).astype(np.float32)
    y = oracle.spectre_y(q, k, v, gate, keep)
    ref = closed_form_y(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                        gate, keep)
    assert np.abs(y - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


# ------------------------------------------------------------ special inputs

def _heads_gate(H, L, seed):
    return RNG.uniform(0.1, 1.0, (H, L // 2 + 1)).astype(np.float32)


@pytest.mark.parametrize("L", [65536, 786432])
def test_constant_inputs(L):
    # q = k = v = 1: only bin 0 is non-zero, Q = K = V = L there, so y = G[h, 0] L.
    H, D = 2, 1
    one = np.ones((1, L, H, D), np.float32)
    gate = _heads_gate(H, L, 1)
    y = oracle.spectre_y(one, one, one, gate, L // 2 + 1)
    for h in range(H):
        ref = float(gate[h, 0]) * L
        assert np.abs(y[0, :, h, 0] - ref).max() <= 1e-9 * ref


@pytest.mark.parametrize("L", [65536, 786432])
def test_alternating_inputs(L):
    # q = k = v = (-1)^n: only the Nyquist bin is non-zero, y = G[h, L/2] L (-1)^t,
    # and it vanishes once the Nyquist bin is truncated.
    H, D = 2, 1
    alt = np.tile(np.array([1, -1], np.float32), L // 2)
    a = np.ascontiguousarray(np.broadcast_to(alt[None, :, None, None], (1, L, H, D)))
    gate = _heads_gate(H, L, 2)
    y = oracle.spectre_y(a, a, a, gate, L // 2 + 1)
    for h in range(H):
        ref = float(gate[h, L // 2]) * L * alt.astype(np.float64)
        assert np.abs(y[0, :, h, 0] - ref).max() <= 1e-9 * float(gate[h, L // 2]) * L
    y0 = oracle.spectre_y(a, a, a, gate, L // 2)
    assert np.abs(y0).max() <= 1e-9 * L


@pytest.mark.parametrize("L,bin_", [(65536, 1), (65536, 12345), (786432, 98304),
                                    (786432, 7)])
def test_single_cosine(L, bin_):
    # q = k = v = cos(2 pi a n / L): Q[a] = L/2, so y = G[h, a] (L/4) cos(2 pi a t / L),
    # and y = 0 when bin a is truncated.
    H, D = 2, 1
    t = np.arange(L)
    c = np.cos(2 * np.pi * ((bin_ * t) % L) / L)
    a = np.ascontiguousarray(np.broadcast_to(c[None, :, None, None], (1, L, H, D)))
    a32 = a.astype(np.float32)
    gate = _heads_gate(H, L, 3)
    y = oracle.spectre_y(a32, a32, a32, gate, L // 2 + 1)
    # the float32 rounding of the input perturbs the spectrum slightly
    for h in range(H):
        ref = float(gate[h, bin_]) * (L / 4) * c
        assert np.abs(y[0, :, h, 0] - ref).max() <= 1e-5 * L / 4
    y0 = oracle.spectre_y(a32, a32, a32, gate, bin_)
    assert np.abs(y0).max() <= 1e-5 * L / 4


@pytest.mark.parametrize("L", [4096, 65536])
def test_impulses(L):
    # q = k = delta_0 makes Q = K = 1, so with G = 1 and no truncation y = v / L.
    B, H, D = 1, 2, 2
    d = np.zeros((B, L, H, D), np.float32)
    d[:, 0] = 1
    v = RNG.standard_normal((B, L, H, D)).astype(np.float32)
    gate = np.ones((H, L // 2 + 1), np.float32)
    y = oracle.spectre_y(d, d, v, gate, L // 2 + 1)
    assert np.abs(y - v / L).max() <= 1e-12 * L


# ----------------------------------------------------------------- invariants

@pytest.mark.parametrize("L", [96, 4096])
def test_shift_covariance(L):
    B, H, D = 1, 2, 2
    q, k, v = (RNG.standard_normal((B, L, H, D)).astype(np.float32) for _ in range(3))
    gate = RNG.uniform(0, 1, (H, L // 2 + 1)).astype(np.float32)
    keep = L // 3
    y = oracle.spectre_y(q, k, v, gate, keep)
    s = 5
    tol = 1e-10 * max(1.0, np.abs(y).max())
    assert np.abs(oracle.spectre_y(np.roll(q, s, 1), k, v, gate, keep)
                  - np.roll(y, s, 1)).max() <= tol
    assert np.abs(oracle.spectre_y(q, np.roll(k, s, 1), v, gate, keep)
                  - np.roll(y, -s, 1)).max() <= tol
    assert np.abs(oracle.spectre_y(q, k, np.roll(v, s, 1), gate, keep)
                  - np.roll(y, s, 1)).max() <= tol


def test_trilinearity():
    L, B, H, D = 384, 1, 2, 2
    q1, q2, k, v = (RNG.standard_normal((B, L, H, D)) for _ in range(4))
    gate = RNG.uniform(0, 1, (H, L // 2 + 1)).astype(np.float32)
    f32 = lambda a: a.astype(np.float32)
    a, b = 0.75, -1.5
    lhs = oracle.spectre_y(f32(a * q1 + b * q2), f32(k), f32(v), gate, L // 2 + 1)
    rhs = (a * oracle.spectre_y(f32(q1), f32(k), f32(v), gate, L // 2 + 1)
           + b * oracle.spectre_y(f32(q2), f32(k), f32(v), gate, L // 2 + 1))
    # lhs sees the float32 rounding of the combined input
    assert np.abs(lhs - rhs).max() <= 1e-5 * np.abs(rhs).max()
    two_k = oracle.spectre_y(f32(q1), f32(2 * k), f32(v), gate, L // 2 + 1)
    assert np.allclose(two_k, 2 * oracle.spectre_y(f32(q1), f32(k), f32(v), gate,
                                                   L // 2 + 1), atol=1e-10)


@pytest.mark.parametrize("L,keep", [(4096, 1025), (4096, 1), (4096, 2048), (65536, 8193),
                                    (98, 13)])
def test_truncation_equals_zeroed_gate(L, keep):
    B, H, D = 1, 2, 2
    q, k, v = (RNG.standard_normal((B, L, H, D)).astype(np.float32) for _ in range(3))
    gate = RNG.uniform(0, 1, (H, L // 2 + 1)).astype(np.float32)
    gz = gate.copy()
    gz[:, keep:] = 0
    a = oracle.spectre_y(q, k, v, gate, keep)
    b = oracle.spectre_y(q, k, v, gz, L // 2 + 1)
    assert np.abs(a - b).max() <= 1e-13 * max(1.0, np.abs(b).max())


def test_keep_zero_and_gate_zero_give_layernorm_of_x():
    L, B, H, D = 256, 2, 2, 4
    q, k, v, x = (RNG.standard_normal((B, L, H, D)).astype(np.float32) for _ in range(4))
    gate = RNG.uniform(0, 1, (H, L // 2 + 1)).astype(np.float32)
    gamma = np.ones(H * D, np.float32)
    beta = np.zeros(H * D, np.float32)
    out0, y0 = oracle.spectre_mix(q, k, v, x, gate, gamma, beta, 0, want_y=True)
    assert np.abs(y0).max() == 0.0
    out1 = oracle.spectre_mix(q, k, v, x, np.zeros_like(gate), gamma, beta, L // 2 + 1)
    assert np.array_equal(out0, out1)


# ------------------------------------------------------------------ LayerNorm

def test_layernorm_known_statistics():
    # Per token, x = mu + s * e with e = +1/-1 alternating over channels: the
    # biased variance is exactly s^2, so out_c = e_c s / sqrt(s^2 + 1e-5) gamma_c + beta_c.
    # s = 2^-10 makes eps visible (s^2 ~ 9.5e-7 against 1e-5); all values are exact
    # in binary32, so the construction survives the float32 storage unchanged.
    H, D = 2, 4
    C = H * D
    e = np.array([1.0 if c % 2 == 0 else -1.0 for c in range(C)])
    mus = [0.0, 3.0, -2.5]
    ss = [1.0, 2.0 ** -10, 7.0]
    x = np.array([[mu + s * e for mu, s in zip(mus, ss)]])  # [1, 3, C]
    x = x.reshape(1, 3, H, D).astype(np.float64)
    x32 = x.astype(np.float32)
    gamma = np.linspace(0.5, 2.0, C).astype(np.float32)
    beta = np.linspace(-1.0, 1.0, C).astype(np.float32)
    y = np.zeros_like(x)
    out = oracle.layernorm_residual(y, x32, gamma, beta).reshape(3, C)
    xs = x32.astype(np.float64).reshape(3, C)
    for i in range(3):
        mu = xs[i].mean()
        s2 = ((xs[i] - mu) ** 2).mean()   # the float32 inputs, exact in double
        ref = (xs[i] - mu) / np.sqrt(s2 + 1e-5) * gamma + beta
        assert np.abs(out[i] - ref).max() <= 1e-12
        assert s2 == ss[i] ** 2
        assert np.abs(out[i] - (e * ss[i] / np.sqrt(ss[i] ** 2 + 1e-5) * gamma + beta)).max() \
            <= 1e-12


def test_layernorm_invariants_on_mix():
    w = workloads.WORKLOADS[1]
    inp = workloads.make_inputs(w)
    gamma = np.linspace(0.5, 1.5, w.C).astype(np.float32)
    beta = np.linspace(-0.2, 0.3, w.C).astype(np.float32)
    out, y = oracle.spectre_mix(inp["q"], inp["k"], inp["v"], inp["x"], inp["gate"], gamma,
                                beta, w.keep_bins, want_y=True)
    z = (inp["x"].astype(np.float64) + y).reshape(w.tokens, w.C)
    n = ((out.reshape(w.tokens, w.C) - beta) / gamma)
    assert np.abs(n.mean(axis=1)).max() <= 1e-12
    var_z = z.var(axis=1)
    assert np.abs(n.var(axis=1) - var_z / (var_z + 1e-5)).max() <= 1e-12


# ------------------------------------------------------------ storage and API

def test_bf16_storage_equals_decoded_f32():
    w = workloads.custom(90, B=1, L=512, H=2, D=4, dtype=workloads.BF16, keep_bins=100)
    inp = workloads.make_inputs(w)
    dec = {n: workloads.from_bf16(inp[n]) for n in "qkvx"}
    a = oracle.spectre_mix(inp["q"], inp["k"], inp["v"], inp["x"], inp["gate"], inp["gamma"],
                           inp["beta"], w.keep_bins, dtype=1)
    b = oracle.spectre_mix(dec["q"], dec["k"], dec["v"], dec["x"], inp["gate"], inp["gamma"],
                           inp["beta"], w.keep_bins, dtype=0)
    assert np.array_equal(a, b)


def test_token_sample_matches_full():
    w = workloads.custom(91, B=3, L=96, H=2, D=4)
    inp = workloads.make_inputs(w)
    out, y = oracle.spectre_mix(inp["q"], inp["k"], inp["v"], inp["x"], inp["gate"],
                                inp["gamma"], inp["beta"], w.keep_bins, want_y=True)
    toks = workloads.sample_tokens(w, 20)
    o2, y2 = oracle.spectre_mix_tokens(inp["q"], inp["k"], inp["v"], inp["x"], inp["gate"],
                                       inp["gamma"], inp["beta"], w.keep_bins, toks)
    flat_o = out.reshape(w.tokens, w.H, w.D)
    flat_y = y.reshape(w.tokens, w.H, w.D)
    assert np.array_equal(o2, flat_o[toks])
    assert np.array_equal(y2, flat_y[toks])


def test_thread_count_does_not_change_result():
    w = workloads.custom(92, B=2, L=192, H=2, D=4)
    inp = workloads.make_inputs(w)
    args = (inp["q"], inp["k"], inp["v"], inp["x"], inp["gate"], inp["gamma"], inp["beta"],
            w.keep_bins)
    assert np.array_equal(oracle.spectre_mix(*args, nthreads=1),
                          oracle.spectre_mix(*args, nthreads=5))


def test_rejects_bad_arguments():
    q = np.zeros((1, 8, 1, 2), np.float32)
    gate = np.zeros((1, 5), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.spectre_y(q, q, q, gate, 6)   # keep_bins > L/2 + 1
    with pytest.raises(oracle.OracleError):
        oracle.spectre_y(q, q, q, gate, -1)


# ------------------------------------------------------------- gate variants
#
# Gate kind 2 (complex multiplier: SPECTRE article, section 2.4's rotation
# inside G(f)) and kind 1 (logit through a sigmoid: section 3.1), and the
# pre-norm order of section 3.3.

def irfft_gate_complex(G, keep, L):
    """g[t] = inverse real transform of the complex gate G[f] * [f < keep],
    f = 0..L//2, as a cosine/sine series: the Hermitian extension gives the
    bins above L/2 the conjugate, and only the real part of bins 0 and L/2
    enters, as an inverse real transform reads them."""
    t = np.arange(L)
    g = np.zeros(L)
    for f in range(L // 2 + 1):
        if f >= keep:
            continue
        a, b = G[f].real, G[f].imag
        if f == 0:
            g += a
        elif L % 2 == 0 and f == L // 2:
            g += a * np.cos(np.pi * t)
        else:
            ang = 2 * np.pi * ((f * t) % L) / L
            g += 2 * (a * np.cos(ang) - b * np.sin(ang))
    return g / L


def closed_form_y_g(q, k, v, gseq):
    """y[b, :, h, d] = (1/L) g_h (*) (q * k) (*) v with g_h = gseq[h]."""
    B, L, H, D = q.shape
    y = np.zeros((B, L, H, D))
    for h in range(H):
        for b in range(B):
            for d in range(D):
                r = circ_xcorr(q[b, :, h, d], k[b, :, h, d])
                y[b, :, h, d] = circ_conv(gseq[h], circ_conv(r, v[b, :, h, d])) / L
    return y


def complex_gate(H, L, rng):
    g = rng.uniform(-1, 1, (H, L // 2 + 1, 2)).astype(np.float32)
    return g, g[..., 0].astype(np.float64) + 1j * g[..., 1].astype(np.float64)


@pytest.mark.parametrize("L,keep", [(1, 1), (2, 2), (4, 3), (5, 3), (6, 4), (8, 5), (12, 7),
                                    (16, 9), (17, 9), (48, 25), (64, 33)])
def test_complex_gate_equals_closed_form(L, keep):
    B, H, D = 1, 2, 2
    q, k, v = (RNG.standard_normal((B, L, H, D)).astype(np.float32) for _ in range(3))
    g32, gc = complex_gate(H, L, RNG)
    y = oracle.spectre_y(q, k, v, g32, keep, gate_kind=2)
    ref = closed_form_y_g(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                          [irfft_gate_complex(gc[h], keep, L) for h in range(H)])
    assert np.abs(y - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("L,shift", [(96, 7), (96, -13), (4096, 5), (4096, 2047)])
def test_complex_gate_linear_phase_is_a_shift(L, shift):
    """A gate exp(-2 pi i f d / L) times a real gate delays the output by d
    tokens (the shift theorem)."""
    B, H, D = 2, 2, 3
    q, k, v = (RNG.standard_normal((B, L, H, D)).astype(np.float32) for _ in range(3))
    real = RNG.uniform(0, 1, (H, L // 2 + 1))
    f = np.arange(L // 2 + 1)
    rot = np.exp(-2j * np.pi * ((f * shift) % L) / L)
    g = real * rot
    g32 = np.stack([g.real, g.imag], -1).astype(np.float32)
    # the reference uses the float32-rounded magnitudes, so both see one gate
    real32 = np.abs(g32[..., 0].astype(np.float64) + 1j * g32[..., 1].astype(np.float64))
    y = oracle.spectre_y(q, k, v, g32, L // 2 + 1, gate_kind=2)
    yr = oracle.spectre_y(q, k, v, real32.astype(np.float32), L // 2 + 1)
    assert np.abs(y - np.roll(yr, shift, axis=1)).max() <= 2e-6 * np.abs(yr).max()


def test_complex_gate_with_zero_imaginary_part_is_the_real_gate():
    L, H = 4096, 2
    q, k, v = (RNG.standard_normal((1, L, H, 4)).astype(np.float32) for _ in range(3))
    g = RNG.uniform(0, 1, (H, L // 2 + 1)).astype(np.float32)
    gc = np.stack([g, np.zeros_like(g)], -1)
    a = oracle.spectre_y(q, k, v, gc, 1500, gate_kind=2)
    b = oracle.spectre_y(q, k, v, g, 1500)
    assert np.abs(a - b).max() <= 1e-13 * np.abs(b).max()


def test_logit_gate_known_values():
    """sigmoid(0) = 1/2, sigmoid(30) = 1 - 9.4e-14, sigmoid(+-ln 3) = 3/4, 1/4;
    y is linear in the gate."""
    L, H = 256, 2
    q, k, v = (RNG.standard_normal((2, L, H, 4)).astype(np.float32) for _ in range(3))
    nb = L // 2 + 1
    y1 = oracle.spectre_y(q, k, v, np.ones((H, nb), np.float32), nb)
    scale = np.abs(y1).max()
    for logit, factor, tol in ((0.0, 0.5, 1e-13), (30.0, 1.0, 1e-12), (np.log(3.0), 0.75, 1e-6),
                               (-np.log(3.0), 0.25, 1e-6)):
        y = oracle.spectre_y(q, k, v, np.full((H, nb), logit, np.float32), nb, gate_kind=1)
        assert np.abs(y - factor * y1).max() <= tol * scale, logit


def test_pre_norm_known_cases():
    """With y = 0 (keep 0) the pre-norm output is x + beta exactly (the
    LayerNorm of a zero row is beta); with x = 0 both orders agree; and in
    general out - x is the LayerNorm of y alone."""
    B, L, H, D = 2, 48, 2, 4
    rng = np.random.default_rng(5)
    q, k, v, x = (rng.standard_normal((B, L, H, D)).astype(np.float32) for _ in range(4))
    gate = rng.uniform(0, 1, (H, L // 2 + 1)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, H * D).astype(np.float32)
    beta = rng.standard_normal(H * D).astype(np.float32)
    out0 = oracle.spectre_mix(q, k, v, x, gate, gamma, beta, 0, norm_order=1)
    assert np.abs(out0 - (x.astype(np.float64) + beta.reshape(H, D))).max() == 0.0
    z = np.zeros_like(x)
    a = oracle.spectre_mix(q, k, v, z, gate, gamma, beta, 20, norm_order=1)
    b = oracle.spectre_mix(q, k, v, z, gate, gamma, beta, 20, norm_order=0)
    assert np.abs(a - b).max() == 0.0
    c, y = oracle.spectre_mix(q, k, v, x, gate, gamma, beta, 20, norm_order=1, want_y=True)
    # LayerNorm of y by its definition, per token
    yt = y.reshape(B * L, H * D)
    mu = yt.mean(1, keepdims=True)
    var = ((yt - mu) ** 2).mean(1, keepdims=True)
    ln = (yt - mu) / np.sqrt(var + 1e-5) * gamma + beta
    assert np.abs(c.reshape(B * L, H * D) - x.reshape(B * L, H * D) - ln).max() <= 1e-12


def test_variant_arguments_rejected():
    q = np.zeros((1, 8, 1, 2), np.float32)
    g = np.ones((1, 5), np.float32)
    with pytest.raises(AssertionError):
        oracle.spectre_y(q, q, q, g, 5, gate_kind=2)  # a complex gate needs [H, bins, 2]
    with pytest.raises(oracle.OracleError):
        oracle.spectre_y(q, q, q, g, 5, gate_kind=3)
    for bad in (-1, 4):  # 0..3: post / pre, LayerNorm / RMSNorm
        with pytest.raises(oracle.OracleError):
            oracle.spectre_mix(q, q, q, q, g, np.ones(2, np.float32), np.zeros(2, np.float32), 5,
                               norm_order=bad)


# ------------------------------------------------------------------ RMSNorm
#
# Section 3.3's "RMSNorm or LayerNorm": norm_order + 2 selects an RMSNorm,
# z / sqrt(mean(z^2) + eps) * gamma + beta, in either order.

def test_rmsnorm_constant_token():
    """A token whose channels all equal c normalises to c / sqrt(c^2 + eps)
    under RMSNorm (a LayerNorm would give 0): with y = 0 (keep_bins 0) the
    post-norm output is that times gamma plus beta, and the pre-norm output
    of y = c (x = 0) is the same."""
    H, D, L = 2, 3, 4
    C = H * D
    c = 0.75
    gamma = np.linspace(0.5, 2.0, C).astype(np.float32)
    beta = np.linspace(-0.2, 0.3, C).astype(np.float32)
    x = np.full((1, L, H, D), c, np.float32)
    z = np.zeros_like(x)
    g = np.ones((H, L // 2 + 1), np.float32)
    out = oracle.spectre_mix(z, z, z, x, g, gamma, beta, 0, norm_order=2)
    ref = c / np.sqrt(c * c + 1e-5) * gamma.astype(np.float64) + beta
    assert np.abs(out.reshape(L, C) - ref).max() <= 1e-12
    ln = oracle.spectre_mix(z, z, z, x, g, gamma, beta, 0, norm_order=0)
    assert np.abs(ln.reshape(L, C) - beta).max() <= 1e-12
    y = np.full((1, L, H, D), c)
    pre = oracle.layernorm_residual(y, np.zeros_like(x), gamma, beta, norm_order=3)
    assert np.abs(pre.reshape(L, C) - ref).max() <= 1e-12


def test_rmsnorm_statistics_and_zero_mean_tokens():
    """RMSNorm with gamma = 1, beta = 0 leaves each token with mean square
    m / (m + eps), m the token's mean square; on tokens of zero mean it equals
    the LayerNorm; pre-norm RMS minus x is the RMSNorm of y."""
    rng = np.random.default_rng(21)
    B, L, H, D = 1, 16, 2, 8
    C = H * D
    y = 3.0 * rng.standard_normal((B, L, H, D)) + 1.5
    x = rng.standard_normal((B, L, H, D)).astype(np.float32)
    ones, zeros = np.ones(C, np.float32), np.zeros(C, np.float32)
    out = oracle.layernorm_residual(y, np.zeros_like(x), ones, zeros, norm_order=2).reshape(L, C)
    m = (y.reshape(L, C) ** 2).mean(axis=1)
    assert np.abs((out ** 2).mean(axis=1) - m / (m + 1e-5)).max() <= 1e-12
    zm = y.reshape(L, C) - y.reshape(L, C).mean(axis=1, keepdims=True)
    zm = zm.reshape(B, L, H, D)
    a = oracle.layernorm_residual(zm, np.zeros_like(x), ones, zeros, norm_order=2)
    b = oracle.layernorm_residual(zm, np.zeros_like(x), ones, zeros, norm_order=0)
    assert np.abs(a - b).max() <= 1e-12
    pre = oracle.layernorm_residual(y, x, ones, zeros, norm_order=3)
    rms = oracle.layernorm_residual(y, np.zeros_like(x), ones, zeros, norm_order=2)
    assert np.abs(pre - x.astype(np.float64) - rms).max() <= 1e-12


# ------------------------------------------------------- gated branch sum
#
# Section 4.3's branches "summed or gated": a per-channel weight g mixes the
# FFT branch and the local branch, g * y + (1 - g) * y_loc.

def test_gated_branches_limits_and_linearity():
    """g = 1 is the FFT mix alone, g = 0 the residual norm of the local branch
    alone, and y is affine in g channel by channel (half of each)."""
    B, L, H, D = 1, 40, 2, 4
    C = H * D
    q, k, v, x = (RNG.standard_normal((B, L, H, D)).astype(np.float32) for _ in range(4))
    gate = RNG.uniform(0, 1, (H, L // 2 + 1)).astype(np.float32)
    gamma = (1 + 0.1 * RNG.standard_normal(C)).astype(np.float32)
    beta = (0.1 * RNG.standard_normal(C)).astype(np.float32)
    one, zero = np.ones(C, np.float32), np.zeros(C, np.float32)
    for norm_order in (0, 1, 2, 3):
        out1 = oracle.spectre_mix_local_gated(q, k, v, x, gate, one, gamma, beta, 15, 5, 3,
                                              norm_order=norm_order)
        ref1 = oracle.spectre_mix(q, k, v, x, gate, gamma, beta, 15, norm_order=norm_order)
        assert np.abs(out1 - ref1).max() <= 1e-12
        out0 = oracle.spectre_mix_local_gated(q, k, v, x, gate, zero, gamma, beta, 15, 5, 3,
                                              norm_order=norm_order)
        yl = _brute_window_attention(*(a.astype(np.float64) for a in (q, k, v)), 5, 3)
        ref0 = oracle.layernorm_residual(yl, x, gamma, beta, norm_order=norm_order)
        assert np.abs(out0 - ref0).max() <= 1e-9
    g = RNG.uniform(0, 1, C).astype(np.float32)
    _, yg = oracle.spectre_mix_local_gated(q, k, v, x, gate, g, gamma, beta, 15, 5, 3, want_y=True)
    _, y1 = oracle.spectre_mix_local_gated(q, k, v, x, gate, one, gamma, beta, 15, 5, 3, want_y=True)
    _, y0 = oracle.spectre_mix_local_gated(q, k, v, x, gate, zero, gamma, beta, 15, 5, 3, want_y=True)
    gc = g.astype(np.float64).reshape(H, D)
    assert np.abs(yg - (gc * y1 + (1 - gc) * y0)).max() <= 1e-12


# ---------------------------------------------------------------- chunked mix
#
# Section 3.2's fft_len below L: blocks mixed on their own, plus the block
# means mixed over the block axis and added back to every token of a block.

def _chunk_inputs(rng, B, L, H, D):
    q, k, v, x = (rng.standard_normal((B, L, H, D)).astype(np.float32) for _ in range(4))
    gamma = rng.uniform(0.5, 1.5, H * D).astype(np.float32)
    beta = (0.1 * rng.standard_normal(H * D)).astype(np.float32)
    return q, k, v, x, gamma, beta


def test_chunked_without_block_gate_mixes_blocks_alone():
    B, L, H, D, F = 2, 96, 2, 2, 24
    rng = np.random.default_rng(21)
    q, k, v, x, gamma, beta = _chunk_inputs(rng, B, L, H, D)
    g = rng.uniform(0, 1, (H, F // 2 + 1)).astype(np.float32)
    gb = np.zeros((H, L // F // 2 + 1), np.float32)
    _, y = oracle.spectre_mix_chunked(q, k, v, x, g, gb, gamma, beta, F, 9, 3, want_y=True)
    for j in range(L // F):
        sl = slice(j * F, (j + 1) * F)
        ref = oracle.spectre_y(q[:, sl], k[:, sl], v[:, sl], g, 9)
        assert np.abs(y[:, sl] - ref).max() <= 1e-13 * max(1.0, np.abs(ref).max())


def test_chunked_block_term_on_piecewise_constant_inputs():
    """With no in-block gate, y is the mix of the block values over the block
    axis, repeated over each block's tokens."""
    B, H, D, F, nb = 1, 2, 2, 16, 12
    L = F * nb
    rng = np.random.default_rng(22)
    cq, ck, cv = (rng.standard_normal((B, nb, H, D)).astype(np.float32) for _ in range(3))
    q, k, v = (np.repeat(c, F, axis=1) for c in (cq, ck, cv))
    x = rng.standard_normal((B, L, H, D)).astype(np.float32)
    g = np.zeros((H, F // 2 + 1), np.float32)
    gb = rng.uniform(0, 1, (H, nb // 2 + 1)).astype(np.float32)
    ones, zeros = np.ones(H * D, np.float32), np.zeros(H * D, np.float32)
    out, y = oracle.spectre_mix_chunked(q, k, v, x, g, gb, ones, zeros, F, F // 2 + 1, 5,
                                        want_y=True)
    ref = np.repeat(closed_form_y(cq.astype(np.float64), ck.astype(np.float64),
                                  cv.astype(np.float64), gb, 5), F, axis=1)
    assert np.abs(y - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())
    assert np.abs(out - oracle.layernorm_residual(ref, x, ones, zeros)).max() <= 1e-9


def test_chunked_single_block_adds_product_of_means():
    """fft_len = L: one block, the plain mix, plus the length-1 mix of the
    means, G_b[h][0] * mean(q) * mean(k) * mean(v) per column."""
    B, L, H, D = 2, 64, 2, 3
    rng = np.random.default_rng(23)
    q, k, v, x, gamma, beta = _chunk_inputs(rng, B, L, H, D)
    g = rng.uniform(0, 1, (H, L // 2 + 1)).astype(np.float32)
    gb = rng.uniform(0, 1, (H, 1)).astype(np.float32)
    _, y = oracle.spectre_mix_chunked(q, k, v, x, g, gb, gamma, beta, L, 20, 1, want_y=True)
    plain = oracle.spectre_y(q, k, v, g, 20)
    m = [t.astype(np.float64).mean(axis=1, keepdims=True) for t in (q, k, v)]
    term = gb[:, 0].astype(np.float64).reshape(1, 1, H, 1) * m[0] * m[1] * m[2]
    assert np.abs(y - (plain + term)).max() <= 1e-12 * max(1.0, np.abs(y).max())


def test_chunked_rejects_bad_block_sizes():
    q = np.zeros((1, 48, 1, 2), np.float32)
    ones, zeros = np.ones(2, np.float32), np.zeros(2, np.float32)
    with pytest.raises(oracle.OracleError):  # 48 is not a multiple of 10
        oracle.spectre_mix_chunked(q, q, q, q, np.ones((1, 6), np.float32),
                                   np.ones((1, 3), np.float32), ones, zeros, 10, 6, 3)
    with pytest.raises(oracle.OracleError):  # keep_blocks above nb/2 + 1
        oracle.spectre_mix_chunked(q, q, q, q, np.ones((1, 7), np.float32),
                                   np.ones((1, 3), np.float32), ones, zeros, 12, 7, 4)


# -------------------------------------------------------------- local branch
#
# Section 4.3's sliding-window attention beside the FFT branch.

def _brute_window_attention(q, k, v, wl, wr):
    """Softmax attention by its definition, one query at a time, every key in
    the window t - wl .. t + wr inside the sequence."""
    B, L, H, D = q.shape
    y = np.zeros((B, L, H, D))
    for b in range(B):
        for h in range(H):
            for t in range(L):
                js = [j for j in range(L) if t - wl <= j <= t + wr]
                s = np.array([np.dot(q[b, t, h], k[b, j, h]) for j in js]) / np.sqrt(D)
                w = np.exp(s - s.max())
                w /= w.sum()
                y[b, t, h] = sum(wj * v[b, j, h] for wj, j in zip(w, js))
    return y


@pytest.mark.parametrize("L,wl,wr", [(1, 0, 0), (7, 2, 3), (16, 15, 0), (16, 4, 4), (9, 20, 20)])
def test_local_attention_equals_definition(L, wl, wr):
    B, H, D = 2, 2, 4
    q, k, v = (RNG.standard_normal((B, L, H, D)).astype(np.float32) for _ in range(3))
    y = oracle.local_attention(q, k, v, wl, wr)
    ref = _brute_window_attention(*(a.astype(np.float64) for a in (q, k, v)), wl, wr)
    assert np.abs(y - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_local_attention_at_listed_tokens():
    """The token-list form of the branch (used where the full sequence is too
    long to compute whole) gives, row by row, the full form's outputs at
    those tokens, ragged batch boundaries included."""
    B, L, H, D = 2, 50, 3, 8
    q, k, v = (RNG.standard_normal((B, L, H, D)).astype(np.float32) for _ in range(3))
    full = oracle.local_attention(q, k, v, 6, 4)
    toks = np.array([0, 1, 7, 49, 50, 51, 77, 99], np.int64)
    got = oracle.local_attention_tokens(q, k, v, 6, 4, toks)
    assert np.array_equal(got, full.reshape(B * L, H, D)[toks])
    with pytest.raises(oracle.OracleError):
        oracle.local_attention_tokens(q, k, v, 6, 4, np.array([100], np.int64))


def test_local_attention_closed_forms():
    """A one-token window returns v; with k = 0 every score is 0, so y is
    the plain mean of v over the window; the first token of a causal window
    sees only itself."""
    B, L, H, D = 1, 40, 2, 8
    q, k, v = (RNG.standard_normal((B, L, H, D)).astype(np.float32) for _ in range(3))
    assert np.abs(oracle.local_attention(q, k, v, 0, 0) - v).max() == 0.0
    z = np.zeros_like(k)
    y = oracle.local_attention(q, z, v, 3, 5)
    v64 = v.astype(np.float64)
    for t in (0, 2, 20, 36, 39):
        lo, hi = max(0, t - 3), min(L - 1, t + 5)
        assert np.abs(y[0, t] - v64[0, lo:hi + 1].mean(axis=0)).max() <= 1e-14
    yc = oracle.local_attention(q, k, v, 255, 0)
    assert np.abs(yc[:, 0] - v64[:, 0]).max() == 0.0


def two_key_case(D):
    """q, k, v of a two-token sequence whose window (one key on each side)
    holds both tokens: every query is e_0, key 0 is e_0 * sqrt(D) ln 3 in
    head 0 and e_0 * sqrt(D) ln(1/3) in head 1, key 1 is 0, and v is e_1 at
    token 0, e_2 at token 1.  The scores q.k / sqrt(D) are ln 3 (or ln 1/3)
    and 0, so the softmax weights are exactly 3/4 and 1/4 (1/4 and 3/4 in
    head 1) up to the binary32 rounding of the key: y = (0, 3/4, 1/4, 0...)
    in head 0 and (0, 1/4, 3/4, 0...) in head 1, for both tokens."""
    B, L, H = 1, 2, 2
    q = np.zeros((B, L, H, D), np.float32)
    k = np.zeros((B, L, H, D), np.float32)
    v = np.zeros((B, L, H, D), np.float32)
    q[..., 0] = 1.0
    k[0, 0, 0, 0] = np.sqrt(D) * np.log(3.0)
    k[0, 0, 1, 0] = -np.sqrt(D) * np.log(3.0)
    v[0, 0, :, 1] = 1.0
    v[0, 1, :, 2] = 1.0
    y = np.zeros((B, L, H, D))
    y[0, :, 0, 1], y[0, :, 0, 2] = 0.75, 0.25
    y[0, :, 1, 1], y[0, :, 1, 2] = 0.25, 0.75
    return q, k, v, y


@pytest.mark.parametrize("D", [4, 16, 64, 128])
def test_local_attention_two_key_weights(D):
    """The score scale 1/sqrt(D) and the exponential weighting: two keys
    whose scores differ by ln 3 get the weights 3/4 and 1/4 (the binary32
    key moves them by at most a few 1e-8)."""
    q, k, v, ref = two_key_case(D)
    y = oracle.local_attention(q, k, v, 1, 1)
    assert np.abs(y - ref).max() <= 1e-7


def test_local_attention_invariants():
    """Shifting q, k, v along the sequence shifts y_loc away from the ends;
    permuting the heads permutes y_loc's heads; q * c with k / c leaves
    every score, so y_loc, unchanged."""
    B, L, H, D = 1, 96, 3, 8
    q, k, v = (RNG.standard_normal((B, L, H, D)).astype(np.float32) for _ in range(3))
    wl, wr, sh = 7, 5, 11
    y = oracle.local_attention(q, k, v, wl, wr)
    ys = oracle.local_attention(*(np.roll(a, sh, axis=1) for a in (q, k, v)), wl, wr)
    inner = slice(wl + sh, L - wr)
    assert np.abs(ys[:, inner] - np.roll(y, sh, axis=1)[:, inner]).max() <= 1e-12
    perm = [2, 0, 1]
    yp = oracle.local_attention(*(np.ascontiguousarray(a[:, :, perm]) for a in (q, k, v)), wl, wr)
    assert np.abs(yp - y[:, :, perm]).max() <= 1e-12
    yc = oracle.local_attention(q * 2.0, k * 0.5, v, wl, wr)
    assert np.abs(yc - y).max() <= 1e-12


@pytest.mark.parametrize("gate_kind,norm_order", [(1, 0), (2, 1), (0, 1)])
def test_mix_with_local_branch_variants_compose(gate_kind, norm_order):
    """The local mix with a logit or complex gate and either norm order is
    the variant's y plus the window attention, through that norm order."""
    B, L, H, D = 1, 48, 2, 4
    q, k, v, x = (RNG.standard_normal((B, L, H, D)).astype(np.float32) for _ in range(4))
    shape = (H, L // 2 + 1, 2) if gate_kind == 2 else (H, L // 2 + 1)
    gate = RNG.uniform(-1, 1, shape).astype(np.float32)
    gamma = (1 + 0.1 * RNG.standard_normal(H * D)).astype(np.float32)
    beta = (0.1 * RNG.standard_normal(H * D)).astype(np.float32)
    out = oracle.spectre_mix_local(q, k, v, x, gate, gamma, beta, 17, 6, 3,
                                   gate_kind=gate_kind, norm_order=norm_order)
    y = oracle.spectre_y(q, k, v, gate, 17, gate_kind=gate_kind)
    yl = _brute_window_attention(*(a.astype(np.float64) for a in (q, k, v)), 6, 3)
    ref = oracle.layernorm_residual(y + yl, x, gamma, beta, norm_order=norm_order)
    assert np.abs(out - ref).max() <= 1e-9


def test_mix_with_local_branch_adds_the_two_outputs():
    B, L, H, D = 1, 64, 2, 4
    q, k, v, x = (RNG.standard_normal((B, L, H, D)).astype(np.float32) for _ in range(4))
    gate = RNG.uniform(0, 1, (H, L // 2 + 1)).astype(np.float32)
    ones, zeros = np.ones(H * D, np.float32), np.zeros(H * D, np.float32)
    out, y = oracle.spectre_mix_local(q, k, v, x, gate, ones, zeros, 20, 16, 15, want_y=True)
    y_fft = oracle.spectre_y(q, k, v, gate, 20)
    y_loc = _brute_window_attention(*(a.astype(np.float64) for a in (q, k, v)), 16, 15)
    assert np.abs(y - (y_fft + y_loc)).max() <= 1e-12
    assert np.abs(out - oracle.layernorm_residual(y_fft + y_loc, x, ones, zeros)).max() <= 1e-9
