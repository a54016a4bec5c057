"""The seeded input generator: determinism, independence from thread count,
distribution moments, bfloat16 rounding and the smooth component's recipe."""
import os
import subprocess
import sys

import numpy as np
import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_deterministic_and_seed_dependent():
    a = workloads.normal(7, (1000,))
    b = workloads.normal(7, (1000,))
    c = workloads.normal(8, (1000,))
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)


def test_counter_based_prefix_property():
    # element i depends only on (seed, i): a longer draw extends a shorter one
    a = workloads.normal(3, (100,))
    b = workloads.normal(3, (1000,))
    assert np.array_equal(a, b[:100])


def test_independent_of_thread_count():
    code = ("import sys; sys.path.insert(0, %r); import workloads, numpy as np;"
            "a = workloads.normal(11, (200003,)); u = workloads.uniform(12, (50001,));"
            "w = workloads.walk_mix(1, 0.5, 2, 0.5, 2, 257, 6);"
            "print(float(a.astype(np.float64).sum()), float(u.sum()), float(w.sum()))" % ROOT)
    outs = []
    for nt in ("1", "3"):
        env = dict(os.environ, OMP_NUM_THREADS=nt)
        outs.append(subprocess.check_output([sys.executable, "-c", code], env=env).strip())
    assert outs[0] == outs[1]


def test_normal_moments():
    a = workloads.normal(21, (1 << 20,)).astype(np.float64)
    assert abs(a.mean()) < 5e-3
    assert abs(a.var() - 1.0) < 5e-3
    assert abs((a ** 3).mean()) < 1e-2          # symmetric
    assert abs((a ** 4).mean() - 3.0) < 3e-2    # normal kurtosis
    assert np.all(np.isfinite(a))


def test_uniform_range_and_moments():
    u = workloads.uniform(22, (1 << 20,)).astype(np.float64)
    assert u.min() >= 0.0 and u.max() < 1.0
    assert abs(u.mean() - 0.5) < 2e-3
    assert abs(u.var() - 1.0 / 12.0) < 2e-3


def test_bf16_round_to_nearest_even():
    # binary32 bit patterns around bf16 rounding points
    bits = np.array([0x3F800000,  # 1.0 exact
                     0x3F808000,  # halfway, lsb 0 -> down
                     0x3F818000,  # halfway, lsb 1 -> up
                     0x3F808001,  # above halfway -> up
                     0x3F807FFF,  # below halfway -> down
                     0xBF818000,  # negative halfway, lsb 1 -> up in magnitude
                     0x00000000, 0x80000000], dtype=np.uint32)
    expect = np.array([0x3F80, 0x3F80, 0x3F82, 0x3F81, 0x3F80, 0xBF82, 0x0000, 0x8000],
                      dtype=np.uint16)
    got = workloads.to_bf16(bits.view(np.float32))
    assert np.array_equal(got, expect)
    back = workloads.from_bf16(expect)
    assert np.array_equal(back.view(np.uint32), expect.astype(np.uint32) << 16)


def test_smooth_component_unit_variance_per_column():
    B, L, C = 2, 4096, 8
    walk = workloads.walk_mix(1, 0.0, 2, 1.0, B, L, C).astype(np.float64)
    m = walk.mean(axis=1)
    v = walk.var(axis=1)
    assert np.abs(m).max() < 1e-5
    assert np.abs(v - 1.0).max() < 1e-5
    # low frequencies dominate: lag-1 autocorrelation of a random walk is near 1
    r = (walk[:, 1:] * walk[:, :-1]).mean(axis=1)
    assert r.min() > 0.9


def test_workload_table_shapes():
    w = workloads.WORKLOADS
    assert (w[1].B, w[1].L, w[1].H, w[1].D, w[1].keep_bins) == (1, 256, 2, 16, 129)
    assert (w[2].B, w[2].L, w[2].H, w[2].D, w[2].keep_bins) == (4, 4096, 8, 64, 2049)
    assert (w[3].B, w[3].L, w[3].H, w[3].D, w[3].keep_bins) == (1, 65536, 8, 64, 32769)
    assert (w[4].B, w[4].L, w[4].dtype, w[4].keep_bins) == (2, 65536, workloads.BF16, 8193)
    assert (w[5].B, w[5].L, w[5].keep_bins) == (1, 786432, 393217)
    assert w[5].L == 3 * 2 ** 18


def test_make_inputs_recipe_small():
    w = workloads.custom(77, B=1, L=64, H=2, D=4, dtype=workloads.BF16, keep_bins=9,
                         smooth=True, gate_zero_above_keep=True, affine=True)
    r = workloads.make_inputs(w)
    assert r["q"].dtype == np.uint16 and r["q"].shape == (1, 64, 2, 4)
    assert r["gate"].shape == (2, 33)
    assert np.all(r["gate"][:, 9:] == 0) and np.all(r["gate"][:, :9] > 0)
    assert r["gamma"].shape == (8,) and not np.all(r["gamma"] == 1)
    again = workloads.make_inputs(w)
    for k in r:
        assert np.array_equal(r[k], again[k])


def test_sample_tokens_cover_edges():
    w = workloads.WORKLOADS[4]
    t = workloads.sample_tokens(w, 32)
    assert t[0] == 0 and t[-1] == w.tokens - 1
    assert w.L - 1 in t and w.L in t
    assert np.all(np.diff(t) > 0)
