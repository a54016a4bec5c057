"""The variant entry points on the GPU against the oracle: a logit gate
(sigmoid applied in the kernels), a complex gate (the SPECTRE article's
section 2.4 rotation inside G(f)), the pre-norm order out = x + LN(y) and
RMSNorm in place of LayerNorm in either order (section 3.3), through
spectre_mix_fwd_ex / spectre_mix_y_ex.

Tolerances as for the plain mix: max-abs on out 1e-4 (binary32 storage) and
2e-2 (bfloat16 storage); y within 1e-4 * max(1, max|y|).  The shapes cover
every kernel path: single-level square and generic LDS kernels, the single-pass
column kernel, two-level
generic, tiled with the LDS-copy B kernel, tiled blocks that span heads,
three-level, the fused norm with and without the split inverse, and the
separate LayerNorm pass.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (DeviceInputs, empty_like_storage, oracle_threads, to_host_f64, tol, torch,
                      y_tol)

pytestmark = pytest.mark.gpu

# (gate kind, norm order); norm order bit 0 = pre-norm, bit 1 = RMSNorm
VARIANTS = [(1, 0), (2, 0), (0, 1), (2, 1), (0, 2), (1, 3)]

SHAPES = [
    # (B, L, H, D, dtype, keep)  keep None = no truncation
    (1, 256, 2, 16, 0, None),      # single level, square LDS kernel (16 x 16)
    (1, 1536, 4, 8, 1, 700),       # single level, generic LDS kernel, bf16, separate norm pass
    (1, 3072, 2, 32, 0, None),     # single-pass column kernel, 12 x 16 x 16
    (4, 4096, 8, 64, 0, None),     # single-pass column kernel, x + y into the norm pass
    (1, 16384, 8, 64, 0, None),    # two-level tiled, LDS-copy B kernel, fused norm
    (1, 8192, 32, 6, 0, None),     # tiled blocks spanning heads: square kernel, gate table
    (1, 98304, 2, 64, 0, None),    # three-level 32 x 3 x 1024
    (2, 8192, 4, 32, 1, 1000),     # fused norm with the one-lane inverse, bf16, truncated
    (1, 16384, 4, 256, 0, None),   # H*D = 1024: separate LayerNorm pass
]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_variant(w, gate_kind, norm_order):
    say("case", w.describe(), "gate kind", gate_kind, "norm order", norm_order)
    t = torch()
    inp = workloads.make_inputs(w)
    inp["gate"] = workloads.make_gate(w, gate_kind)
    ref_out, ref_y = oracle.spectre_mix(inp["q"], inp["k"], inp["v"], inp["x"], inp["gate"],
                                        inp["gamma"], inp["beta"], w.keep_bins, dtype=w.dtype,
                                        nthreads=oracle_threads(), want_y=True,
                                        gate_kind=gate_kind, norm_order=norm_order)
    d = DeviceInputs(w, inp)
    import efficient_attention_fft_amd as sm
    _, out = empty_like_storage(w)
    sm.check(d.fwd_ex(out, gate_kind, norm_order))
    t.cuda.synchronize()
    got = to_host_f64(out, w.dtype).reshape(ref_out.shape)
    err = np.abs(got - ref_out).max()
    say("  out max-abs err %.3g (tol %.1g)" % (err, tol(w)))
    assert np.all(np.isfinite(got))
    assert err <= tol(w)
    y = t.full((w.N,), float("nan"), dtype=t.float32, device="cuda")
    sm.check(d.y_ex(y, gate_kind))
    t.cuda.synchronize()
    gy = y.cpu().numpy().astype(np.float64).reshape(ref_y.shape)
    ey = np.abs(gy - ref_y).max()
    say("  y max-abs err %.3g (tol %.3g)" % (ey, y_tol(ref_y)))
    assert ey <= y_tol(ref_y)


@pytest.mark.parametrize("gate_kind,norm_order", VARIANTS)
@pytest.mark.parametrize("B,L,H,D,dt,keep", SHAPES)
def test_variant_shapes(B, L, H, D, dt, keep, gate_kind, norm_order):
    kb = L // 2 + 1 if keep is None else keep
    w = workloads.custom(400 + L % 97, B=B, L=L, H=H, D=D, dtype=dt, keep_bins=kb, affine=True)
    check_variant(w, gate_kind, norm_order)


@pytest.mark.parametrize("gate_kind,norm_order", VARIANTS)
def test_variant_long_workload(gate_kind, norm_order):
    """L = 65536, H = 8, D = 64: several work items per workgroup in the
    LDS-copy B kernel and the split fused inverse."""
    check_variant(workloads.WORKLOADS[3], gate_kind, norm_order)


def test_real_variant_entry_matches_plain_entry():
    """spectre_mix_fwd_ex with a real gate and post-norm is spectre_mix_fwd, bit for bit."""
    w = workloads.WORKLOADS[2]
    t = torch()
    inp = workloads.make_inputs(w)
    d = DeviceInputs(w, inp)
    import efficient_attention_fft_amd as sm
    _, a = empty_like_storage(w)
    _, b = empty_like_storage(w)
    sm.check(d.fwd(a))
    sm.check(d.fwd_ex(b, 0, 0))
    t.cuda.synchronize()
    assert t.equal(a, b)
