"""Python binding of the gfx950 SPECTRE spectral-mix library (libspectre_mix.so).

Argument marshalling only: every function has the name and the argument order
of the C ABI in include/spectre_mix.h, accepts device tensors (any object with
``data_ptr()``) or raw integer device addresses, passes them through ctypes
and returns the library's integer status.  All arithmetic runs in the HIP
kernels; there is no other code path.  ``check`` turns a status into an
exception.  Importing this module fails loudly if the library is not built.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspectre_mix.so")

SPECTRE_F32 = 0
SPECTRE_BF16 = 1
SPECTRE_OK = 0
SPECTRE_EINVAL = -1
SPECTRE_EUNSUPPORTED = -2
SPECTRE_ENOMEM = -3
SPECTRE_EHIP = -4
SPECTRE_GATE_REAL = 0
SPECTRE_GATE_LOGIT = 1
SPECTRE_GATE_COMPLEX = 2
SPECTRE_NORM_POST = 0
SPECTRE_NORM_PRE = 1
SPECTRE_NORM_POST_RMS = 2
SPECTRE_NORM_PRE_RMS = 3

EXPORTS = ("spectre_mix_fwd", "spectre_mix_y", "spectre_mix_workspace_bytes", "spectre_mix_plan",
           "spectre_mix_release", "spectre_mix_trace_start", "spectre_mix_trace_stop",
           "spectre_mix_strerror", "spectre_mix_fwd_ex", "spectre_mix_y_ex",
           "spectre_mix_workspace_bytes_ex", "spectre_mix_fwd_chunked", "spectre_mix_y_chunked",
           "spectre_mix_fwd_local", "spectre_mix_local_attention", "spectre_mix_fwd_local_ex",
           "spectre_mix_fwd_noalloc", "spectre_mix_fwd_local_gated")


class SpectreError(RuntimeError):
    def __init__(self, status: int):
        super().__init__("spectre_mix status %d: %s" % (status, spectre_mix_strerror(status)))
        self.status = status


def _hip_runtimes():
    """Distinct libamdhip64 files mapped into this process."""
    found = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                path = line.split()[-1] if len(line.split()) >= 6 else ""
                if "libamdhip64" in os.path.basename(path):
                    found.add(os.path.realpath(path))
    except OSError:
        pass
    return found


def _load():
    # One HIP runtime per process: when PyTorch supplies device memory and
    # streams, its bundled runtime must be the one this library binds to.
    # Loading torch first maps that runtime (soname libamdhip64.so.7), and the
    # library's dependency on libamdhip64.so.7 then resolves to it.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError("libspectre_mix.so is not built: run "
                          "python efficient_attention_fft_amd/csrc/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.spectre_mix_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ci, vp]
    lib.spectre_mix_fwd.restype = ci
    lib.spectre_mix_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                            ci, vp]
    lib.spectre_mix_fwd_noalloc.restype = ci
    lib.spectre_mix_y.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ci, vp]
    lib.spectre_mix_y.restype = ci
    lib.spectre_mix_workspace_bytes.argtypes = [i64, i64, i64, i64, ci]
    lib.spectre_mix_workspace_bytes.restype = ctypes.c_size_t
    lib.spectre_mix_fwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                       ci, ci, ci, vp]
    lib.spectre_mix_fwd_ex.restype = ci
    lib.spectre_mix_y_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ci, ci, vp]
    lib.spectre_mix_y_ex.restype = ci
    lib.spectre_mix_workspace_bytes_ex.argtypes = [i64, i64, i64, i64, ci, ci]
    lib.spectre_mix_workspace_bytes_ex.restype = ctypes.c_size_t
    lib.spectre_mix_fwd_chunked.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64,
                                            i64, i64, i64, i64, ci, vp]
    lib.spectre_mix_fwd_chunked.restype = ci
    lib.spectre_mix_y_chunked.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                          i64, ci, vp]
    lib.spectre_mix_y_chunked.restype = ci
    lib.spectre_mix_fwd_local.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                          i64, i64, ci, vp]
    lib.spectre_mix_fwd_local.restype = ci
    lib.spectre_mix_fwd_local_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                             i64, i64, i64, ci, ci, ci, vp]
    lib.spectre_mix_fwd_local_ex.restype = ci
    lib.spectre_mix_fwd_local_gated.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64,
                                                i64, i64, i64, i64, ci, ci, ci, vp]
    lib.spectre_mix_fwd_local_gated.restype = ci
    lib.spectre_mix_local_attention.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci,
                                                vp]
    lib.spectre_mix_local_attention.restype = ci
    lib.spectre_mix_plan.argtypes = [i64, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                     ctypes.POINTER(i64)]
    lib.spectre_mix_plan.restype = ci
    lib.spectre_mix_release.argtypes = []
    lib.spectre_mix_release.restype = ci
    lib.spectre_mix_trace_start.argtypes = [ci]
    lib.spectre_mix_trace_start.restype = ci
    lib.spectre_mix_trace_stop.argtypes = [ci, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ci),
                                           ctypes.POINTER(ci), ctypes.c_char_p, ci]
    lib.spectre_mix_trace_stop.restype = ci
    lib.spectre_mix_strerror.argtypes = [ci]
    lib.spectre_mix_strerror.restype = ctypes.c_char_p
    runtimes = _hip_runtimes()
    if len(runtimes) > 1:
        raise ImportError("two HIP runtimes are loaded (%s); import torch before any other "
                          "HIP library" % ", ".join(sorted(runtimes)))
    return lib


_lib = _load()


def lib():
    """The ctypes handle of libspectre_mix.so."""
    return _lib


def _addr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def spectre_mix_fwd(q, k, v, x, gate, gamma, beta, out, B, H, L, D, keep_bins, dtype,
                    stream=None) -> int:
    return _lib.spectre_mix_fwd(_addr(q), _addr(k), _addr(v), _addr(x), _addr(gate), _addr(gamma),
                                _addr(beta), _addr(out), B, H, L, D, keep_bins, dtype,
                                _stream(stream))


def spectre_mix_fwd_noalloc(q, k, v, x, gate, gamma, beta, out, B, H, L, D, keep_bins, dtype,
                            stream=None) -> int:
    return _lib.spectre_mix_fwd_noalloc(_addr(q), _addr(k), _addr(v), _addr(x), _addr(gate),
                                        _addr(gamma), _addr(beta), _addr(out), B, H, L, D,
                                        keep_bins, dtype, _stream(stream))


def spectre_mix_y(q, k, v, gate, y, B, H, L, D, keep_bins, dtype, stream=None) -> int:
    return _lib.spectre_mix_y(_addr(q), _addr(k), _addr(v), _addr(gate), _addr(y), B, H, L, D,
                              keep_bins, dtype, _stream(stream))


def spectre_mix_fwd_ex(q, k, v, x, gate, gamma, beta, out, B, H, L, D, keep_bins, dtype,
                       gate_kind, norm_order, stream=None) -> int:
    return _lib.spectre_mix_fwd_ex(_addr(q), _addr(k), _addr(v), _addr(x), _addr(gate),
                                   _addr(gamma), _addr(beta), _addr(out), B, H, L, D, keep_bins,
                                   dtype, gate_kind, norm_order, _stream(stream))


def spectre_mix_y_ex(q, k, v, gate, y, B, H, L, D, keep_bins, dtype, gate_kind,
                     stream=None) -> int:
    return _lib.spectre_mix_y_ex(_addr(q), _addr(k), _addr(v), _addr(gate), _addr(y), B, H, L, D,
                                 keep_bins, dtype, gate_kind, _stream(stream))


def spectre_mix_fwd_chunked(q, k, v, x, gate, gate_blocks, gamma, beta, out, B, H, L, D,
                            fft_len, keep_bins, keep_blocks, dtype, stream=None) -> int:
    return _lib.spectre_mix_fwd_chunked(_addr(q), _addr(k), _addr(v), _addr(x), _addr(gate),
                                        _addr(gate_blocks), _addr(gamma), _addr(beta), _addr(out),
                                        B, H, L, D, fft_len, keep_bins, keep_blocks, dtype,
                                        _stream(stream))


def spectre_mix_y_chunked(q, k, v, gate, gate_blocks, y, B, H, L, D, fft_len, keep_bins,
                          keep_blocks, dtype, stream=None) -> int:
    return _lib.spectre_mix_y_chunked(_addr(q), _addr(k), _addr(v), _addr(gate),
                                      _addr(gate_blocks), _addr(y), B, H, L, D, fft_len,
                                      keep_bins, keep_blocks, dtype, _stream(stream))


def spectre_mix_fwd_local(q, k, v, x, gate, gamma, beta, out, B, H, L, D, keep_bins, win_left,
                          win_right, dtype, stream=None) -> int:
    return _lib.spectre_mix_fwd_local(_addr(q), _addr(k), _addr(v), _addr(x), _addr(gate),
                                      _addr(gamma), _addr(beta), _addr(out), B, H, L, D, keep_bins,
                                      win_left, win_right, dtype, _stream(stream))


def spectre_mix_fwd_local_ex(q, k, v, x, gate, gamma, beta, out, B, H, L, D, keep_bins,
                             win_left, win_right, dtype, gate_kind, norm_order,
                             stream=None) -> int:
    return _lib.spectre_mix_fwd_local_ex(_addr(q), _addr(k), _addr(v), _addr(x), _addr(gate),
                                         _addr(gamma), _addr(beta), _addr(out), B, H, L, D,
                                         keep_bins, win_left, win_right, dtype, gate_kind,
                                         norm_order, _stream(stream))


def spectre_mix_fwd_local_gated(q, k, v, x, gate, mix, gamma, beta, out, B, H, L, D, keep_bins,
                                win_left, win_right, dtype, gate_kind, norm_order,
                                stream=None) -> int:
    return _lib.spectre_mix_fwd_local_gated(_addr(q), _addr(k), _addr(v), _addr(x), _addr(gate),
                                            _addr(mix), _addr(gamma), _addr(beta), _addr(out), B,
                                            H, L, D, keep_bins, win_left, win_right, dtype,
                                            gate_kind, norm_order, _stream(stream))


def spectre_mix_local_attention(q, k, v, y, B, H, L, D, win_left, win_right, dtype,
                                stream=None) -> int:
    return _lib.spectre_mix_local_attention(_addr(q), _addr(k), _addr(v), _addr(y), B, H, L, D,
                                            win_left, win_right, dtype, _stream(stream))


def spectre_mix_workspace_bytes(B, H, L, D, dtype) -> int:
    return _lib.spectre_mix_workspace_bytes(B, H, L, D, dtype)


def spectre_mix_workspace_bytes_ex(B, H, L, D, dtype, gate_kind) -> int:
    return _lib.spectre_mix_workspace_bytes_ex(B, H, L, D, dtype, gate_kind)


def spectre_mix_plan(L):
    """(status, (l1, l2, l3))."""
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    st = _lib.spectre_mix_plan(L, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
    return st, (a.value, b.value, c.value)


def spectre_mix_release() -> int:
    return _lib.spectre_mix_release()


def spectre_mix_trace_start(max_calls: int) -> int:
    return _lib.spectre_mix_trace_start(max_calls)


def spectre_mix_trace_stop(max_kernels: int = 40):
    """(status, [(kernel name, total ms over the traced calls)], calls traced)."""
    total = (ctypes.c_float * max_kernels)()
    nk, nc = ctypes.c_int(), ctypes.c_int()
    name_len = 32
    names = ctypes.create_string_buffer(max_kernels * name_len)
    st = _lib.spectre_mix_trace_stop(max_kernels, total, ctypes.byref(nk), ctypes.byref(nc),
                                     names, name_len)
    if st != SPECTRE_OK:
        return st, [], 0
    raw = names.raw
    out = []
    for k in range(nk.value):
        nm = raw[k * name_len:(k + 1) * name_len].split(b"\0", 1)[0].decode()
        out.append((nm, float(total[k])))
    return st, out, nc.value


def spectre_mix_strerror(status: int) -> str:
    return _lib.spectre_mix_strerror(status).decode()


def check(status: int) -> None:
    if status != SPECTRE_OK:
        raise SpectreError(status)
