"""Helpers for the GPU tests: device copies of the seeded inputs, calls
through the C ABI, and the comparisons with the oracle."""
import os

import numpy as np

import efficient_attention_fft_amd as sm
import oracle
import workloads

TOL_F32 = 1e-4   # max-abs on out, binary32 storage
TOL_BF16 = 2e-2  # max-abs on out, bfloat16 storage


def oracle_threads():
    """The CPU share of this process: OMP_NUM_THREADS when set, else every
    online CPU."""
    online = os.cpu_count() or 1
    try:
        share = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        share = 0
    return max(1, min(share, online) if share > 0 else online)


def torch():
    import torch as t
    return t


def dev(a: np.ndarray):
    t = torch()
    if a.dtype == np.uint16:
        return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    return t.from_numpy(np.ascontiguousarray(a)).cuda()


def empty_like_storage(w, guard: int = 0):
    """Output buffer in the storage dtype, optionally with `guard` NaN-filled
    elements before and after (returns (whole, view))."""
    t = torch()
    n = w.N
    if w.dtype == workloads.F32:
        whole = t.full((n + 2 * guard,), float("nan"), dtype=t.float32, device="cuda")
    else:
        whole = t.full((n + 2 * guard,), -1, dtype=t.int16, device="cuda")  # 0xFFFF: a NaN
    return whole, whole[guard:guard + n]


def to_host_f64(t, dtype):
    a = t.cpu().numpy()
    if dtype == workloads.BF16:
        return workloads.from_bf16(a.view(np.uint16)).astype(np.float64)
    return a.astype(np.float64)


class DeviceInputs:
    def __init__(self, w, inp):
        self.w = w
        self.q, self.k, self.v, self.x = (dev(inp[n]) for n in "qkvx")
        self.gate = dev(inp["gate"])
        self.gamma = dev(inp["gamma"])
        self.beta = dev(inp["beta"])

    def fwd(self, out, keep=None, stream=None):
        w = self.w
        keep = w.keep_bins if keep is None else keep
        return sm.spectre_mix_fwd(self.q, self.k, self.v, self.x, self.gate, self.gamma,
                                  self.beta, out, w.B, w.H, w.L, w.D, keep, w.dtype, stream)

    def y(self, y, keep=None, stream=None):
        w = self.w
        keep = w.keep_bins if keep is None else keep
        return sm.spectre_mix_y(self.q, self.k, self.v, self.gate, y, w.B, w.H, w.L, w.D, keep,
                                w.dtype, stream)

    def fwd_ex(self, out, gate_kind, norm_order, stream=None):
        w = self.w
        return sm.spectre_mix_fwd_ex(self.q, self.k, self.v, self.x, self.gate, self.gamma,
                                     self.beta, out, w.B, w.H, w.L, w.D, w.keep_bins, w.dtype,
                                     gate_kind, norm_order, stream)

    def y_ex(self, y, gate_kind, stream=None):
        w = self.w
        return sm.spectre_mix_y_ex(self.q, self.k, self.v, self.gate, y, w.B, w.H, w.L, w.D,
                                   w.keep_bins, w.dtype, gate_kind, stream)


def run_out(w, inp, keep=None):
    """out of the GPU path as float64 host array [B, L, H, D]."""
    t = torch()
    d = DeviceInputs(w, inp)
    _, out = empty_like_storage(w)
    sm.check(d.fwd(out, keep))
    t.cuda.synchronize()
    return to_host_f64(out, w.dtype).reshape(w.B, w.L, w.H, w.D)


def run_y(w, inp, keep=None):
    t = torch()
    d = DeviceInputs(w, inp)
    y = t.full((w.N,), float("nan"), dtype=t.float32, device="cuda")
    sm.check(d.y(y, keep))
    t.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64).reshape(w.B, w.L, w.H, w.D)


def oracle_out(w, inp, keep=None, want_y=False):
    keep = w.keep_bins if keep is None else keep
    return oracle.spectre_mix(inp["q"], inp["k"], inp["v"], inp["x"], inp["gate"], inp["gamma"],
                              inp["beta"], keep, dtype=w.dtype, nthreads=oracle_threads(),
                              want_y=want_y)


def tol(w):
    return TOL_F32 if w.dtype == workloads.F32 else TOL_BF16


def y_tol(ref_y):
    return 1e-4 * max(1.0, float(np.abs(ref_y).max()))
