"""The allocation-free entry point (spectre_mix_fwd_noalloc) against
spectre_mix_fwd on the same device inputs: two calls in a row, the second
with a smaller input (its tables and workspace then overwrite the first
call's in the shared device array), for binary32 and bfloat16 storage.  The
bar is the oracle parity bar of the two storage types."""
import numpy as np
import pytest

import efficient_attention_fft_amd as sm
import workloads
from gpu_util import DeviceInputs, empty_like_storage, to_host_f64, tol, torch

pytestmark = pytest.mark.gpu

# (B, L, H, D, keep), two calls in a row, the second smaller: a two-level
# plan (8 x 1024, tiled LDS pass), then the single-pass column kernel; the
# column kernel at 12 x 16 x 16, then the square single-level kernel; a
# two-level plan in row layout (6 x 1024, CP2 = 16), then the generic
# single-level kernel
CASES = [((1, 8192, 4, 32, 1500), (1, 4096, 4, 32, 1025)),
         ((2, 3072, 4, 16, 700), (1, 256, 2, 16, 129)),
         ((1, 6144, 2, 16, 900), (1, 1536, 2, 16, 700))]


def _pair(w, keep):
    t = torch()
    d = DeviceInputs(w, workloads.make_inputs(w))
    _, a = empty_like_storage(w)
    _, b = empty_like_storage(w)
    sm.check(d.fwd(a, keep))
    sm.check(sm.spectre_mix_fwd_noalloc(d.q, d.k, d.v, d.x, d.gate, d.gamma, d.beta, b, w.B, w.H,
                                        w.L, w.D, keep, w.dtype))
    t.cuda.synchronize()
    return to_host_f64(a, w.dtype), to_host_f64(b, w.dtype)


@pytest.mark.parametrize("dtype", [workloads.F32, workloads.BF16])
@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_fwd_twice(first, second, dtype):
    for i, (B, L, H, D, keep) in enumerate((first, second)):
        w = workloads.custom(40 + i, B=B, L=L, H=H, D=D, keep_bins=keep, dtype=dtype, affine=True)
        ref, got = _pair(w, keep)
        assert np.isfinite(got).all()
        assert np.abs(got - ref).max() <= tol(w), (B, L, H, D, keep, dtype)


def test_noalloc_rejects_large_workspace_untouched():
    """A workspace beyond the array is refused before anything is enqueued:
    the output keeps its contents."""
    t = torch()
    w = workloads.custom(42, B=1, L=65536, H=8, D=64, keep_bins=32769)
    z = t.zeros(w.N, dtype=t.float32, device="cuda")
    out = t.full((w.N,), 7.0, dtype=t.float32, device="cuda")
    g = t.zeros((w.H, w.L // 2 + 1), dtype=t.float32, device="cuda")
    c = t.zeros(w.C, dtype=t.float32, device="cuda")
    st = sm.spectre_mix_fwd_noalloc(z, z.clone(), z.clone(), z.clone(), g, c, c.clone(), out, w.B,
                                    w.H, w.L, w.D, w.keep_bins, 0)
    t.cuda.synchronize()
    assert st == sm.SPECTRE_EUNSUPPORTED
    assert bool((out == 7.0).all())
