"""Planted mistakes: each mutant is a copy of the oracle source with one
plausible error (a dropped conjugate, a wrong sign, index, scale, norm or
truncation bound), built on the CPU.  The pins must reject every mutant, and
accept the unmodified source, so they are shown to be able to catch such
mistakes in the oracle itself."""
import os

import numpy as np
import pytest

import oracle
from test_oracle_pins import (closed_form_y, closed_form_y_g, complex_gate,
                              irfft_gate_complex, naive_dft, two_key_case)

SRC = os.path.join(os.path.dirname(oracle.__file__), "spectre_oracle.c")

MUTANTS = {
    "conj_dropped": ("cmul(cmul(bufq[f], cconj(bufk[f])), bufv[f])",
                     "cmul(cmul(bufq[f], bufk[f]), bufv[f])"),
    "conj_on_q": ("cmul(cmul(bufq[f], cconj(bufk[f])), bufv[f])",
                  "cmul(cmul(cconj(bufq[f]), bufk[f]), bufv[f])"),
    "gate_scale_dropped": ("bufv[f]), g), invL);", "bufv[f]), g), 1.0);"),
    "complex_gate_conj": ("g.im = (double)J->gate[2 * (h * nbins + f) + 1];",
                          "g.im = -(double)J->gate[2 * (h * nbins + f) + 1];"),
    "complex_gate_im_index": ("g.im = (double)J->gate[2 * (h * nbins + f) + 1];",
                              "g.im = (double)J->gate[2 * (h * nbins + f)];"),
    "logit_sign": ("1.0 / (1.0 + exp(-a))", "1.0 / (1.0 + exp(a))"),
    "logit_ignored": ("g.re = J->gate_kind == 1 ? 1.0 / (1.0 + exp(-a)) : a;", "g.re = a;"),
    "pre_norm_stats_with_x": ("o[c] = pre ? yr[c] : load_elem(x, dtype, xr * C + c) + yr[c];",
                              "o[c] = load_elem(x, dtype, xr * C + c) + yr[c];"),
    "pre_norm_residual_dropped": ("if (pre) o[c] += load_elem(x, dtype, xr * C + c);",
                                  "if (pre) o[c] += 0.0;"),
    "chunk_mean_scale": ("means[((a * B + b) * nb + j) * C + c] = acc / (double)F;",
                         "means[((a * B + b) * nb + j) * C + c] = acc;"),
    "chunk_block_index": ("y2[(b * nb + t / F) * C + c]", "y2[(b * nb + (t / F + 1) % nb) * C + c]"),
    "chunk_block_gate": ("J.gate = gate_blocks;", "J.gate = gate;"),
    "local_scale_dropped": ("const double scale = 1.0 / sqrt((double)D);", "const double scale = 1.0;"),
    "local_scale_over_d": ("const double scale = 1.0 / sqrt((double)D);",
                           "const double scale = 1.0 / (double)D;"),
    "local_exp2_weights": ("sc[j - j0] = exp(sc[j - j0] - mx);", "sc[j - j0] = exp2(sc[j - j0] - mx);"),
    "local_window_right": ("const int64_t j1 = t + win_right > L - 1 ? L - 1 : t + win_right;",
                           "const int64_t j1 = t + win_right + 1 > L - 1 ? L - 1 : t + win_right + 1;"),
    "local_not_normalised": ("yq[d] = acc / sum;", "yq[d] = acc;"),
    "local_wrong_head": ("const int64_t kb = (b * L + j) * C + h * D;",
                         "const int64_t kb = (b * L + j) * C + ((h + 1) % H) * D;"),
    "local_window_left": ("const int64_t j0 = t - win_left < 0 ? 0 : t - win_left;",
                          "const int64_t j0 = t - win_left + 1 < 0 ? 0 : t - win_left + 1;"),
    "inverse_scale_dropped": ("double re = bufq[t].re * invL, im = bufq[t].im * invL;",
                              "double re = bufq[t].re, im = bufq[t].im * invL;"),
    "truncation_inclusive": ("if (f < J->keep) {", "if (f <= J->keep) {"),
    "head_index": ("const int64_t h = c / J->D;", "const int64_t h = c % J->H;"),
    "hermitian_no_conj": ("tmp[f] = cconj(tmp[L - f]);", "tmp[f] = tmp[L - f];"),
    "radix4_rotation": ("cpx jb1 = sign > 0 ? (cpx){-b1.im, b1.re} : (cpx){b1.im, -b1.re};",
                        "cpx jb1 = sign > 0 ? (cpx){b1.im, -b1.re} : (cpx){-b1.im, b1.re};"),
    "radix3_sign": ("cpx rot = {-(double)sign * s3 * dif.im, (double)sign * s3 * dif.re};",
                    "cpx rot = {(double)sign * s3 * dif.im, -(double)sign * s3 * dif.re};"),
    "twiddle_sign": ("t->w[j].im = -sin(a);", "t->w[j].im = sin(a);"),
    "prime_dft_index": ("acc = cadd(acc, cmul(y[r], twiddle(t, p, r * s, sign)));",
                        "acc = cadd(acc, cmul(y[r], twiddle(t, p, r + s, sign)));"),
    "variance_unbiased": ("var /= (double)C;", "var /= (double)(C - 1);"),
    "rms_subtracts_mean": ("double mean = rms ? 0.0 : sum / (double)C;",
                           "double mean = sum / (double)C;"),
    "gated_weights_swapped": ("y[i] = g * y[i] + (1.0 - g) * yl[i];",
                              "y[i] = (1.0 - g) * y[i] + g * yl[i];"),
    "gated_channel_index": ("const double g = (double)mix[i % C];",
                            "const double g = (double)mix[(i / C) % C];"),
    "eps_outside_sqrt": ("double rstd = 1.0 / sqrt(var + eps);",
                         "double rstd = 1.0 / (sqrt(var) + eps);"),
    "gamma_beta_swapped": ("o[c] = (o[c] - mean) * rstd * (double)gamma[c] + (double)beta[c];",
                           "o[c] = (o[c] - mean) * rstd * (double)beta[c] + (double)gamma[c];"),
    "residual_dropped": ("pre ? yr[c] : load_elem(x, dtype, xr * C + c) + yr[c];",
                         "pre ? yr[c] : yr[c];"),
    "nyquist_dropped": ("if (f == 0 || (L % 2 == 0 && f == half)) o.im = 0.0;",
                        "if (f == 0 || (L % 2 == 0 && f == half)) { o.im = 0.0; "
                        "if (f == half) o.re = 0.0; }"),
    "bf16_decode_shift": ("uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;",
                          "uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 15;"),
}


def _pins_pass() -> bool:
    """A compact run of the pins; False as soon as one fails."""
    rng = np.random.default_rng(7)
    try:
        for n in (5, 7, 12, 16, 18, 30):
            x = rng.standard_normal(n) + 1j * rng.standard_normal(n)
            for sign in (-1, 1):
                ref = naive_dft(x, sign)
                if np.abs(oracle.fft(x, sign) - ref).max() > 1e-10 * np.abs(ref).max():
                    return False
        for L, keep in ((8, 5), (12, 7), (16, 9), (17, 4), (48, 10)):
            B, H, D = 1, 2, 2
            q, k, v = (rng.standard_normal((B, L, H, D)).astype(np.float32) for _ in range(3))
            gate = rng.uniform(0.1, 1, (H, L // 2 + 1)).astype(np.float32)
            ref = closed_form_y(*(a.astype(np.float64) for a in (q, k, v)), gate, keep)
            if np.abs(oracle.spectre_y(q, k, v, gate, keep) - ref).max() > 1e-10:
                return False
        # LayerNorm on a constructed token (mean 3, variance s^2 = 2^-20)
        H, D = 2, 2
        C = H * D
        e = np.array([1.0, -1.0, 1.0, -1.0])
        s = 2.0 ** -10
        x = (3.0 + s * e).reshape(1, 1, H, D).astype(np.float32)
        gamma = np.array([0.5, 1.0, 1.5, 2.0], np.float32)
        beta = np.array([-0.1, 0.0, 0.1, 0.2], np.float32)
        # through the full mix with a zero gate (y = 0), bf16 storage of exact values
        bits = (x.view(np.uint32) >> 16).astype(np.uint16)
        xb = (bits.astype(np.uint32) << 16).view(np.float32)
        ref = e * s / np.sqrt(s * s + 1e-5) * gamma + beta
        for st, dt in ((x, 0), (bits, 1)):
            if dt == 1 and not np.array_equal(xb, x):
                continue
            z = np.zeros((1, 1, H, D), st.dtype)
            out = oracle.spectre_mix(z, z, z, st, np.zeros((H, 1), np.float32), gamma, beta,
                                     0, dtype=dt)
            if np.abs(out.reshape(C) - ref).max() > 1e-9:
                return False
        # bf16 decoding: a bf16-stored mix equals the float32 mix of the decoded values
        L = 16
        vals = rng.standard_normal((1, L, 1, 2)).astype(np.float32)
        b16 = (vals.view(np.uint32) >> 16).astype(np.uint16)
        dec = (b16.astype(np.uint32) << 16).view(np.float32)
        g = np.ones((1, L // 2 + 1), np.float32)
        ones, zeros = np.ones(2, np.float32), np.zeros(2, np.float32)
        a = oracle.spectre_mix(b16, b16, b16, b16, g, ones, zeros, L // 2 + 1, dtype=1)
        ref_y = closed_form_y(*(dec.astype(np.float64),) * 3, g, L // 2 + 1)
        ref = oracle.layernorm_residual(ref_y, dec, ones, zeros)
        if np.abs(a - ref).max() > 1e-9:
            return False
        # gate variants: a complex gate against its closed form, logits at
        # known sigmoid values, and the pre-norm order with y = 0
        for L, keep in ((12, 7), (17, 9)):
            B, H, D = 1, 2, 2
            q, k, v = (rng.standard_normal((B, L, H, D)).astype(np.float32) for _ in range(3))
            g32, gc = complex_gate(H, L, rng)
            ref = closed_form_y_g(*(a.astype(np.float64) for a in (q, k, v)),
                                  [irfft_gate_complex(gc[h], keep, L) for h in range(H)])
            if np.abs(oracle.spectre_y(q, k, v, g32, keep, gate_kind=2) - ref).max() > 1e-10:
                return False
        L, H = 16, 2
        q, k, v = (rng.standard_normal((1, L, H, 2)).astype(np.float32) for _ in range(3))
        nb = L // 2 + 1
        y1 = oracle.spectre_y(q, k, v, np.ones((H, nb), np.float32), nb)
        for logit, factor in ((0.0, 0.5), (30.0, 1.0), (-30.0, 0.0)):
            y = oracle.spectre_y(q, k, v, np.full((H, nb), logit, np.float32), nb, gate_kind=1)
            if np.abs(y - factor * y1).max() > 1e-9 * np.abs(y1).max():
                return False
        x = rng.standard_normal((1, L, H, 2)).astype(np.float32)
        beta = rng.standard_normal(H * 2).astype(np.float32)
        out = oracle.spectre_mix(q, k, v, x, np.ones((H, nb), np.float32),
                                 np.ones(H * 2, np.float32), beta, 0, norm_order=1)
        if np.abs(out - (x.astype(np.float64) + beta.reshape(H, 2))).max() > 0.0:
            return False
        # chunked mix: piecewise-constant inputs, no in-block gate
        B, H, D, F, nb = 1, 2, 2, 16, 12
        cq, ck, cv = (rng.standard_normal((B, nb, H, D)).astype(np.float32) for _ in range(3))
        qq, kk, vv = (np.repeat(c, F, axis=1) for c in (cq, ck, cv))
        xx = rng.standard_normal((B, F * nb, H, D)).astype(np.float32)
        gb = rng.uniform(0.1, 1, (H, nb // 2 + 1)).astype(np.float32)
        ones, zeros = np.ones(H * D, np.float32), np.zeros(H * D, np.float32)
        _, y = oracle.spectre_mix_chunked(qq, kk, vv, xx, np.zeros((H, F // 2 + 1), np.float32),
                                          gb, ones, zeros, F, F // 2 + 1, 5, want_y=True)
        ref = np.repeat(closed_form_y(*(c.astype(np.float64) for c in (cq, ck, cv)), gb, 5), F,
                        axis=1)
        if np.abs(y - ref).max() > 1e-10:
            return False
        # local branch by closed forms only: two keys whose scores differ by
        # ln 3 (weights 3/4, 1/4), and k = 0 (the plain mean over the window)
        for D in (4, 64):
            q, k, v, ref = two_key_case(D)
            if np.abs(oracle.local_attention(q, k, v, 1, 1) - ref).max() > 1e-7:
                return False
        q, v = (rng.standard_normal((1, 12, 2, 4)).astype(np.float32) for _ in range(2))
        y = oracle.local_attention(q, np.zeros_like(q), v, 3, 2)
        for t in (0, 5, 11):
            lo, hi = max(0, t - 3), min(11, t + 2)
            if np.abs(y[0, t] - v[0, lo:hi + 1].astype(np.float64).mean(axis=0)).max() > 1e-14:
                return False
        # RMSNorm: a constant token keeps c / sqrt(c^2 + eps)
        H, D, Lr = 2, 2, 4
        cst = np.full((1, Lr, H, D), 0.75, np.float32)
        zr = np.zeros_like(cst)
        o = oracle.spectre_mix(zr, zr, zr, cst, np.ones((H, 3), np.float32),
                               np.ones(H * D, np.float32), np.zeros(H * D, np.float32), 0,
                               norm_order=2)
        if np.abs(o - 0.75 / np.sqrt(0.75 ** 2 + 1e-5)).max() > 1e-12:
            return False
        # gated branches: g = 1 is the FFT mix alone; a half-and-half token
        # mix is affine in g channel by channel
        B, L, H, D = 1, 24, 2, 2
        C = H * D
        q, k, v, x = (rng.standard_normal((B, L, H, D)).astype(np.float32) for _ in range(4))
        gt = rng.uniform(0, 1, (H, L // 2 + 1)).astype(np.float32)
        ones, zeros = np.ones(C, np.float32), np.zeros(C, np.float32)
        a = oracle.spectre_mix_local_gated(q, k, v, x, gt, ones, ones, zeros, 9, 2, 2)
        if np.abs(a - oracle.spectre_mix(q, k, v, x, gt, ones, zeros, 9)).max() > 1e-12:
            return False
        gw = np.array([0.1, 0.4, 0.7, 0.9], np.float32)
        _, yg = oracle.spectre_mix_local_gated(q, k, v, x, gt, gw, ones, zeros, 9, 2, 2, want_y=True)
        yf = oracle.spectre_y(q, k, v, gt, 9)
        yl = oracle.local_attention(q, k, v, 2, 2)
        gc = gw.astype(np.float64).reshape(H, D)
        if np.abs(yg - (gc * yf + (1 - gc) * yl)).max() > 1e-12:
            return False
    except oracle.OracleError:
        return False
    return True


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


def test_unmodified_source_passes(mutant_dir):
    path = oracle.compile_source(SRC, str(mutant_dir / "lib_clean.so"))
    with oracle.use_library(path):
        assert _pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_dir):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site not found: %s" % name
    path_c = mutant_dir / ("%s.c" % name)
    path_c.write_text(src.replace(old, new))
    lib = oracle.compile_source(str(path_c), str(mutant_dir / ("lib_%s.so" % name)))
    with oracle.use_library(lib):
        assert not _pins_pass(), "planted mistake %s went unnoticed" % name
