"""Seeded synthetic workloads for the SPECTRE spectral mix.

The five workload shapes, their value recipes, and a deterministic
generator (``synth.c``: counter-based SplitMix64 + Box-Muller, see that
file's header).  Nothing here computes any part of the mix: this module
only draws the inputs that the GPU library and the CPU oracle both receive.

The article (SPECTRE FFT-attention article, section 2.3) uses the shape
L = 65536, H = 8, D = 64 for its complexity example and keeps 25-50% of the
bins at L = 8192; those shapes and ratios drive the workloads below.  The
pages name no dataset, so every tensor is synthetic.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

F32 = 0
BF16 = 1

# tensor ids inside a workload's seed: seed = 1000 * workload + id
_Q, _K, _V, _X, _GATE, _GAMMA, _BETA = 1, 2, 3, 4, 5, 6, 7
_Q_WALK, _K_WALK, _V_WALK = 11, 12, 13


def build(force: bool = True) -> str:
    """Compile synth.c into libsynth.so next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-o", tmp,
                               _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        i64, u64, dbl, vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
        lib.synth_normal_f32.argtypes = [u64, i64, vp]
        lib.synth_uniform_f32.argtypes = [u64, i64, dbl, dbl, vp]
        lib.synth_normal_mix_f32.argtypes = [u64, dbl, u64, dbl, i64, vp]
        lib.synth_walk_mix_f32.argtypes = [u64, dbl, u64, dbl, i64, i64, i64, vp]
        lib.synth_f32_to_bf16.argtypes = [vp, i64, vp]
        lib.synth_bf16_to_f32.argtypes = [vp, i64, vp]
        for f in (lib.synth_normal_f32, lib.synth_uniform_f32, lib.synth_normal_mix_f32,
                  lib.synth_walk_mix_f32, lib.synth_f32_to_bf16, lib.synth_bf16_to_f32):
            f.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def normal(seed: int, shape) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().synth_normal_f32(seed, out.size, _ptr(out))
    return out


def uniform(seed: int, shape, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().synth_uniform_f32(seed, out.size, lo, hi, _ptr(out))
    return out


def normal_mix(seed_a: int, a: float, seed_b: int, b: float, shape) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().synth_normal_mix_f32(seed_a, a, seed_b, b, out.size, _ptr(out))
    return out


def walk_mix(seed_white: int, a: float, seed_walk: int, b: float, B: int, L: int,
             C: int) -> np.ndarray:
    """a * N(0,1) + b * (per-column random walk along L, unit variance)."""
    out = np.empty((B, L, C), dtype=np.float32)
    _load().synth_walk_mix_f32(seed_white, a, seed_walk, b, B, L, C, _ptr(out))
    return out


def to_bf16(a: np.ndarray) -> np.ndarray:
    """binary32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().synth_f32_to_bf16(_ptr(a), a.size, _ptr(out))
    return out


def from_bf16(a: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> binary32 (exact)."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    out = np.empty(a.shape, dtype=np.float32)
    _load().synth_bf16_to_f32(_ptr(a), a.size, _ptr(out))
    return out


@dataclasses.dataclass(frozen=True)
class Workload:
    """One workload: shape [B, L, H, D], storage dtype and value recipe."""
    wid: int
    name: str
    B: int
    L: int
    H: int
    D: int
    dtype: int  # F32 or BF16
    keep_bins: int
    smooth: bool = False        # q, k, v = sqrt(1/2) white + sqrt(1/2) walk
    affine: bool = False        # gamma ~ 1 + 0.1 N, beta ~ 0.1 N (else 1, 0)
    gate_zero_above_keep: bool = False

    @property
    def C(self) -> int:
        return self.H * self.D

    @property
    def N(self) -> int:
        return self.B * self.L * self.H * self.D

    @property
    def nbins(self) -> int:
        return self.L // 2 + 1

    @property
    def tokens(self) -> int:
        return self.B * self.L

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    def seed(self, tensor_id: int) -> int:
        return 1000 * self.wid + tensor_id

    def describe(self) -> dict:
        return {"workload": self.name, "B": self.B, "L": self.L, "H": self.H, "D": self.D,
                "dtype": "f32" if self.dtype == F32 else "bf16", "keep_bins": self.keep_bins}


# The five workloads: tiny, mid-length, the article's long-context shape,
# band-truncated bf16, and very long mixed-radix.
WORKLOADS = {
    1: Workload(1, "tiny_L256_f32", B=1, L=256, H=2, D=16, dtype=F32, keep_bins=129),
    2: Workload(2, "mid_L4096_f32", B=4, L=4096, H=8, D=64, dtype=F32, keep_bins=2049,
                affine=True),
    3: Workload(3, "long_L65536_f32", B=1, L=65536, H=8, D=64, dtype=F32, keep_bins=32769),
    4: Workload(4, "trunc_L65536_bf16", B=2, L=65536, H=8, D=64, dtype=BF16, keep_bins=8193,
                smooth=True, gate_zero_above_keep=True),
    5: Workload(5, "vlong_L786432_f32", B=1, L=786432, H=8, D=64, dtype=F32,
                keep_bins=393217),
}


def custom(wid: int, B: int, L: int, H: int, D: int, dtype: int = F32,
           keep_bins: int | None = None, **kw) -> Workload:
    """A workload of any shape with the same recipes (for edge-case tests)."""
    if keep_bins is None:
        keep_bins = L // 2 + 1
    return Workload(wid, "custom_B%d_L%d_H%d_D%d" % (B, L, H, D), B=B, L=L, H=H, D=D,
                    dtype=dtype, keep_bins=keep_bins, **kw)


def make_inputs(w: Workload) -> dict:
    """Host arrays for one workload.

    q, k, v, x: [B, L, H, D] in the storage dtype (float32, or uint16 bf16 bits);
    gate: [H, L//2 + 1] float32 in [0, 1); gamma, beta: [H*D] float32.
    """
    shape = (w.B, w.L, w.H, w.D)
    r = {}
    for name, tid, wid in (("q", _Q, _Q_WALK), ("k", _K, _K_WALK), ("v", _V, _V_WALK)):
        if w.smooth:
            a = np.sqrt(0.5)
            t = walk_mix(w.seed(tid), a, w.seed(wid), a, w.B, w.L, w.C).reshape(shape)
        else:
            t = normal(w.seed(tid), shape)
        r[name] = to_bf16(t) if w.dtype == BF16 else t
    x = normal(w.seed(_X), shape)
    r["x"] = to_bf16(x) if w.dtype == BF16 else x
    gate = uniform(w.seed(_GATE), (w.H, w.nbins))
    if w.gate_zero_above_keep:
        gate[:, w.keep_bins:] = 0.0
    r["gate"] = gate
    if w.affine:
        r["gamma"] = (1.0 + 0.1 * normal(w.seed(_GAMMA), (w.C,))).astype(np.float32)
        r["beta"] = (0.1 * normal(w.seed(_BETA), (w.C,))).astype(np.float32)
    else:
        r["gamma"] = np.ones(w.C, dtype=np.float32)
        r["beta"] = np.zeros(w.C, dtype=np.float32)
    return r


# gate kinds of the variant entry points (the same numbers as the C ABI)
GATE_REAL, GATE_LOGIT, GATE_COMPLEX = 0, 1, 2
_GATE_LOGIT_SEED, _GATE_RE_SEED, _GATE_IM_SEED = 51, 52, 53


def make_gate(w: Workload, gate_kind: int) -> np.ndarray:
    """The gate array for a gate kind: the workload's own gate (real), logits
    ~ N(0, 2^2) (their sigmoids spread over (0, 1)), or a complex gate with
    real and imaginary parts ~ U(-1, 1), laid out [H, L//2 + 1, 2].  Bins at
    or above keep_bins are zeroed when the workload asks for that."""
    if gate_kind == GATE_REAL:
        return make_inputs(w)["gate"]
    if gate_kind == GATE_LOGIT:
        g = 2.0 * normal(w.seed(_GATE_LOGIT_SEED), (w.H, w.nbins))
        if w.gate_zero_above_keep:
            g[:, w.keep_bins:] = -30.0
        return g.astype(np.float32)
    re = uniform(w.seed(_GATE_RE_SEED), (w.H, w.nbins), -1.0, 1.0)
    im = uniform(w.seed(_GATE_IM_SEED), (w.H, w.nbins), -1.0, 1.0)
    g = np.stack([re, im], -1)
    if w.gate_zero_above_keep:
        g[:, w.keep_bins:] = 0.0
    return np.ascontiguousarray(g, dtype=np.float32)


_GATE_BLOCK_SEED, _GATE_BLOCKS_SEED = 54, 55
_BRANCH_MIX_SEED = 56


def make_branch_mix(w: Workload) -> np.ndarray:
    """Per-channel weights of the gated branch sum, [H*D] float32 ~ U[0, 1),
    with channel 0 at 1 and channel 1 at 0 (each branch alone)."""
    g = uniform(w.seed(_BRANCH_MIX_SEED), (w.C,)).astype(np.float32)
    g[0], g[1] = 1.0, 0.0
    return g


def make_chunk_gates(w: Workload, fft_len: int):
    """Gates of the chunked mix: the in-block gate [H, fft_len//2 + 1] and the
    block-axis gate [H, nb//2 + 1] (nb = L // fft_len), both ~ U[0, 1)."""
    nb = w.L // fft_len
    return (uniform(w.seed(_GATE_BLOCK_SEED), (w.H, fft_len // 2 + 1)),
            uniform(w.seed(_GATE_BLOCKS_SEED), (w.H, nb // 2 + 1)))


def sample_tokens(w: Workload, count: int, seed: int = 99) -> np.ndarray:
    """Flat token ids b*L + t to check at full size: the first and last token,
    the tokens on either side of each batch boundary, and a seeded spread."""
    fixed = [0, w.tokens - 1]
    for b in range(1, w.B):
        fixed += [b * w.L - 1, b * w.L]
    rnd = (uniform(seed, (max(count - len(fixed), 0),)).astype(np.float64)
           * w.tokens).astype(np.int64)
    ids = np.unique(np.clip(np.concatenate([np.array(fixed, np.int64), rnd]), 0,
                            w.tokens - 1))
    return ids.astype(np.int64)
