"""Python access to the double-precision CPU oracle (``spectre_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use this to compute expected values.  The GPU library and
its binding never import it.

Every function takes host numpy arrays: q, k, v, x as [B, L, H, D] float32
(dtype 0) or uint16 bfloat16 bit patterns (dtype 1); gate as [H, L//2 + 1]
float32 (gate_kind 0: the multiplier, 1: its logit), or [H, L//2 + 1, 2]
float32 (gate_kind 2: real and imaginary parts); gamma, beta as [H*D]
float32.  norm_order 0 is out = LN(x + y), 1 is out = x + LN(y); adding 2
uses an RMSNorm (no mean subtracted) in place of the LayerNorm.  Results are
float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spectre_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, EINVAL, ENOMEM, EIMAG = 0, -1, -3, -5


def compile_source(src: str, out: str) -> str:
    """gcc -O2 (IEEE math, no fast-math) of an oracle source file into a shared library."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle into liboracle.so next to its source."""
    if force or not os.path.exists(_LIB):
        compile_source(_SRC, _LIB)
    return _LIB


_lib = None


def _bind(lib):
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.oracle_fft.argtypes = [i64, vp, vp, vp, vp, ci]
    lib.oracle_spectre_y.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, ci, vp, ci]
    lib.oracle_layernorm_residual.argtypes = [vp, vp, vp, vp, i64, i64, ci, vp]
    lib.oracle_spectre_mix.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                       ci, vp, vp, ci]
    lib.oracle_spectre_mix_tokens.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64,
                                              i64, i64, ci, vp, i64, vp, vp, ci]
    lib.oracle_threads.argtypes = [ci]
    lib.oracle_spectre_y_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, ci, ci, vp, ci]
    lib.oracle_layernorm_residual_ex.argtypes = [vp, vp, vp, vp, i64, i64, ci, ci, vp]
    lib.oracle_spectre_mix_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                          ci, ci, ci, vp, vp, ci]
    lib.oracle_spectre_mix_tokens_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64,
                                                 i64, i64, ci, ci, ci, vp, i64, vp, vp, ci]
    lib.oracle_spectre_mix_chunked.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64,
                                               i64, i64, i64, i64, ci, vp, vp, ci]
    lib.oracle_spectre_mix_chunked.restype = ci
    lib.oracle_local_attention.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, vp]
    lib.oracle_local_attention.restype = ci
    lib.oracle_local_attention_tokens.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, ci,
                                                  vp, i64, vp]
    lib.oracle_local_attention_tokens.restype = ci
    lib.oracle_spectre_mix_local.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                             i64, i64, ci, vp, vp, ci]
    lib.oracle_spectre_mix_local.restype = ci
    lib.oracle_spectre_mix_local_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                                i64, i64, i64, ci, ci, ci, vp, vp, ci]
    lib.oracle_spectre_mix_local_ex.restype = ci
    lib.oracle_spectre_mix_local_gated.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64,
                                                   i64, i64, i64, i64, ci, ci, ci, vp, vp, ci]
    lib.oracle_spectre_mix_local_gated.restype = ci
    for f in (lib.oracle_fft, lib.oracle_spectre_y, lib.oracle_layernorm_residual,
              lib.oracle_spectre_mix, lib.oracle_spectre_mix_tokens, lib.oracle_threads,
              lib.oracle_spectre_y_ex, lib.oracle_layernorm_residual_ex,
              lib.oracle_spectre_mix_ex, lib.oracle_spectre_mix_tokens_ex):
        f.restype = ci
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


class use_library:
    """Context manager: route this module's calls to another build of the
    oracle source (the mutation tests plant mistakes in a copy of it)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _load()
        _lib = _bind(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


class OracleError(RuntimeError):
    pass


def _check(status: int):
    if status != OK:
        raise OracleError("oracle returned status %d" % status)


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _storage(a: np.ndarray, dtype: int) -> np.ndarray:
    return _c(a, np.float32 if dtype == 0 else np.uint16)


def threads(nthreads: int = 0) -> int:
    """Threads a call with ``nthreads`` uses (0 = every online CPU)."""
    return _load().oracle_threads(nthreads)


def fft(x: np.ndarray, sign: int = -1) -> np.ndarray:
    """Unnormalised complex DFT of a 1-D array: sum_j x[j] exp(sign 2 pi i f j / n)."""
    x = np.asarray(x)
    re = _c(x.real, np.float64)
    im = _c(x.imag if np.iscomplexobj(x) else np.zeros_like(re), np.float64)
    n = re.size
    ore = np.empty(n, np.float64)
    oim = np.empty(n, np.float64)
    _check(_load().oracle_fft(n, re.ctypes.data, im.ctypes.data, ore.ctypes.data,
                              oim.ctypes.data, sign))
    return ore + 1j * oim


def _gate(gate, H: int, L: int, gate_kind: int) -> np.ndarray:
    gate = _c(gate, np.float32)
    shape = (H, L // 2 + 1, 2) if gate_kind == 2 else (H, L // 2 + 1)
    assert gate.shape == shape, (gate.shape, shape)
    return gate


def spectre_y(q, k, v, gate, keep_bins: int, dtype: int = 0, nthreads: int = 0,
              gate_kind: int = 0) -> np.ndarray:
    """y = irfft(G Q conj(K) V / L) per column, [B, L, H, D] float64."""
    B, L, H, D = q.shape
    q, k, v = (_storage(t, dtype) for t in (q, k, v))
    gate = _gate(gate, H, L, gate_kind)
    y = np.empty((B, L, H, D), np.float64)
    _check(_load().oracle_spectre_y_ex(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                       gate.ctypes.data, B, H, L, D, keep_bins, dtype,
                                       gate_kind, y.ctypes.data, nthreads))
    return y


def layernorm_residual(y, x, gamma, beta, dtype: int = 0, norm_order: int = 0) -> np.ndarray:
    """LayerNorm over the last two axes' H*D channels of (x + y) (norm_order
    0), or x + the LayerNorm of y (norm_order 1); eps 1e-5."""
    shape = y.shape
    C = shape[-1] * shape[-2]
    ntok = int(np.prod(shape[:-2]))
    y = _c(y, np.float64)
    x = _storage(x, dtype)
    gamma, beta = _c(gamma, np.float32), _c(beta, np.float32)
    out = np.empty(shape, np.float64)
    _check(_load().oracle_layernorm_residual_ex(y.ctypes.data, x.ctypes.data, gamma.ctypes.data,
                                                beta.ctypes.data, ntok, C, dtype, norm_order,
                                                out.ctypes.data))
    return out


def spectre_mix(q, k, v, x, gate, gamma, beta, keep_bins: int, dtype: int = 0,
                nthreads: int = 0, want_y: bool = False, gate_kind: int = 0,
                norm_order: int = 0):
    """The whole mix; returns out [B, L, H, D] float64 (and y if want_y)."""
    B, L, H, D = q.shape
    q, k, v, x = (_storage(t, dtype) for t in (q, k, v, x))
    gate = _gate(gate, H, L, gate_kind)
    gamma, beta = (_c(t, np.float32) for t in (gamma, beta))
    assert gamma.size == H * D and beta.size == H * D
    out = np.empty((B, L, H, D), np.float64)
    y = np.empty((B, L, H, D), np.float64) if want_y else None
    _check(_load().oracle_spectre_mix_ex(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                         x.ctypes.data, gate.ctypes.data, gamma.ctypes.data,
                                         beta.ctypes.data, B, H, L, D, keep_bins, dtype,
                                         gate_kind, norm_order, out.ctypes.data,
                                         y.ctypes.data if want_y else None, nthreads))
    return (out, y) if want_y else out


def spectre_mix_tokens(q, k, v, x, gate, gamma, beta, keep_bins: int, tokens,
                       dtype: int = 0, nthreads: int = 0, gate_kind: int = 0,
                       norm_order: int = 0):
    """The mix at sampled flat token ids b*L + t; returns (out, y), each [ntok, H, D]."""
    B, L, H, D = q.shape
    q, k, v, x = (_storage(t, dtype) for t in (q, k, v, x))
    gate = _gate(gate, H, L, gate_kind)
    gamma, beta = (_c(t, np.float32) for t in (gamma, beta))
    tokens = _c(tokens, np.int64)
    n = tokens.size
    out = np.empty((n, H, D), np.float64)
    y = np.empty((n, H, D), np.float64)
    _check(_load().oracle_spectre_mix_tokens_ex(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                                x.ctypes.data, gate.ctypes.data,
                                                gamma.ctypes.data, beta.ctypes.data, B, H, L,
                                                D, keep_bins, dtype, gate_kind, norm_order,
                                                tokens.ctypes.data, n, out.ctypes.data,
                                                y.ctypes.data, nthreads))
    return out, y


def spectre_mix_chunked(q, k, v, x, gate, gate_blocks, gamma, beta, fft_len: int,
                        keep_bins: int, keep_blocks: int, dtype: int = 0, nthreads: int = 0,
                        want_y: bool = False):
    """The chunked mix: blocks of fft_len tokens mixed on their own (gate
    [H, fft_len//2 + 1]), plus the mix of the block means over the block axis
    (gate_blocks [H, nb//2 + 1], nb = L // fft_len) added to every token of
    its block, then LN(x + y).  Returns out (and y if want_y), float64."""
    B, L, H, D = q.shape
    q, k, v, x = (_storage(t, dtype) for t in (q, k, v, x))
    nb = L // fft_len
    gate = _c(gate, np.float32)
    gate_blocks = _c(gate_blocks, np.float32)
    assert gate.shape == (H, fft_len // 2 + 1) and gate_blocks.shape == (H, nb // 2 + 1)
    gamma, beta = (_c(t, np.float32) for t in (gamma, beta))
    out = np.empty((B, L, H, D), np.float64)
    y = np.empty((B, L, H, D), np.float64) if want_y else None
    _check(_load().oracle_spectre_mix_chunked(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                              x.ctypes.data, gate.ctypes.data,
                                              gate_blocks.ctypes.data, gamma.ctypes.data,
                                              beta.ctypes.data, B, H, L, D, fft_len, keep_bins,
                                              keep_blocks, dtype, out.ctypes.data,
                                              y.ctypes.data if want_y else None, nthreads))
    return (out, y) if want_y else out


def local_attention(q, k, v, win_left: int, win_right: int, dtype: int = 0) -> np.ndarray:
    """The sliding-window branch: per head, softmax((q . k) / sqrt(D)) over keys
    t - win_left .. t + win_right inside the sequence, times v; [B, L, H, D] float64."""
    B, L, H, D = q.shape
    q, k, v = (_storage(t, dtype) for t in (q, k, v))
    y = np.empty((B, L, H, D), np.float64)
    _check(_load().oracle_local_attention(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, L, D,
                                          win_left, win_right, dtype, y.ctypes.data))
    return y


def local_attention_tokens(q, k, v, win_left: int, win_right: int, tokens,
                           dtype: int = 0) -> np.ndarray:
    """The sliding-window branch at listed flat tokens b * L + t only:
    [len(tokens), H, D] float64, each row as local_attention computes it."""
    B, L, H, D = q.shape
    q, k, v = (_storage(t, dtype) for t in (q, k, v))
    toks = np.ascontiguousarray(tokens, np.int64)
    y = np.empty((len(toks), H, D), np.float64)
    _check(_load().oracle_local_attention_tokens(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H,
                                                 L, D, win_left, win_right, dtype,
                                                 toks.ctypes.data, len(toks), y.ctypes.data))
    return y


def spectre_mix_local_gated(q, k, v, x, gate, mix, gamma, beta, keep_bins: int, win_left: int,
                            win_right: int, dtype: int = 0, nthreads: int = 0,
                            want_y: bool = False, gate_kind: int = 0, norm_order: int = 0):
    """The mix with the local branch weighted per channel: the branch sum is
    mix[c] * y + (1 - mix[c]) * y_loc (mix: [H*D] float32 in [0, 1]), then
    the residual and the norm of norm_order; y (if want_y) is that sum."""
    B, L, H, D = q.shape
    q, k, v, x = (_storage(t, dtype) for t in (q, k, v, x))
    gate = _gate(gate, H, L, gate_kind)
    mix, gamma, beta = (_c(t, np.float32) for t in (mix, gamma, beta))
    out = np.empty((B, L, H, D), np.float64)
    y = np.empty((B, L, H, D), np.float64) if want_y else None
    _check(_load().oracle_spectre_mix_local_gated(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                                  x.ctypes.data, gate.ctypes.data, mix.ctypes.data,
                                                  gamma.ctypes.data, beta.ctypes.data, B, H, L, D,
                                                  keep_bins, win_left, win_right, dtype, gate_kind,
                                                  norm_order, out.ctypes.data,
                                                  y.ctypes.data if want_y else None, nthreads))
    return (out, y) if want_y else out


def spectre_mix_local(q, k, v, x, gate, gamma, beta, keep_bins: int, win_left: int,
                      win_right: int, dtype: int = 0, nthreads: int = 0, want_y: bool = False,
                      gate_kind: int = 0, norm_order: int = 0):
    """The mix with the local branch: out = LN(x + y + y_loc) (norm_order 0)
    or x + LN(y + y_loc) (norm_order 1); y (if want_y) is y + y_loc."""
    B, L, H, D = q.shape
    q, k, v, x = (_storage(t, dtype) for t in (q, k, v, x))
    gate = _gate(gate, H, L, gate_kind)
    gamma, beta = (_c(t, np.float32) for t in (gamma, beta))
    out = np.empty((B, L, H, D), np.float64)
    y = np.empty((B, L, H, D), np.float64) if want_y else None
    _check(_load().oracle_spectre_mix_local_ex(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                               x.ctypes.data, gate.ctypes.data, gamma.ctypes.data,
                                               beta.ctypes.data, B, H, L, D, keep_bins, win_left,
                                               win_right, dtype, gate_kind, norm_order,
                                               out.ctypes.data, y.ctypes.data if want_y else None,
                                               nthreads))
    return (out, y) if want_y else out
