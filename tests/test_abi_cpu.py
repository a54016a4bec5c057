"""The C-ABI library on a host without a GPU: it loads, exports every symbol
the header declares, and rejects bad arguments before touching the device.
No call here reaches a kernel."""
import ctypes
import os
import re

import pytest

import efficient_attention_fft_amd as sm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spectre_mix.h")

GOOD = 1 << 20          # a 16-byte-aligned fake address; never dereferenced here
SHAPE = (1, 8, 65536, 64)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spectre_mix_\w+)\s*\(", text)))


def test_header_declares_the_exports():
    assert declared_functions() == sorted(sm.EXPORTS)


@pytest.mark.parametrize("name", sm.EXPORTS)
def test_library_exports_symbol(name):
    lib = ctypes.CDLL(sm.LIB_PATH)
    assert hasattr(lib, name)


def test_strerror_names_every_status():
    for st in (0, -1, -2, -3, -4):
        assert sm.spectre_mix_strerror(st) not in ("", "unknown status")
    assert sm.spectre_mix_strerror(7) == "unknown status"


def fwd(**kw):
    a = dict(q=GOOD, k=GOOD + 0x1000000, v=GOOD + 0x2000000, x=GOOD + 0x3000000,
             gate=GOOD + 0x4000000, gamma=GOOD + 0x5000000, beta=GOOD + 0x6000000,
             out=GOOD + 0x70000000, B=1, H=8, L=65536, D=64, keep_bins=32769, dtype=0)
    a.update(kw)
    return sm.spectre_mix_fwd(a["q"], a["k"], a["v"], a["x"], a["gate"], a["gamma"], a["beta"],
                              a["out"], a["B"], a["H"], a["L"], a["D"], a["keep_bins"],
                              a["dtype"], 0)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), sm.SPECTRE_EINVAL),
    (dict(out=0), sm.SPECTRE_EINVAL),
    (dict(gate=0), sm.SPECTRE_EINVAL),
    (dict(B=0), sm.SPECTRE_EINVAL),
    (dict(H=0), sm.SPECTRE_EINVAL),
    (dict(D=-1), sm.SPECTRE_EINVAL),
    (dict(L=0), sm.SPECTRE_EINVAL),
    (dict(L=65535, keep_bins=1), sm.SPECTRE_EINVAL),  # odd
    (dict(L=5 * 4096, keep_bins=1), sm.SPECTRE_EUNSUPPORTED),    # prime factor 5
    (dict(L=9 * 4096, keep_bins=1), sm.SPECTRE_EUNSUPPORTED),    # 3^2
    (dict(L=6 * 2 ** 20), sm.SPECTRE_EUNSUPPORTED),  # above 3 * 2^20
    (dict(keep_bins=-1), sm.SPECTRE_EINVAL),
    (dict(keep_bins=32770), sm.SPECTRE_EINVAL),
    (dict(dtype=2), sm.SPECTRE_EINVAL),
    (dict(q=GOOD + 8), sm.SPECTRE_EINVAL),          # misaligned
    (dict(gamma=GOOD + 0x5000004), sm.SPECTRE_EINVAL),
    (dict(H=3, D=1), sm.SPECTRE_EUNSUPPORTED),      # odd H*D
    (dict(H=64, D=128), sm.SPECTRE_EUNSUPPORTED),   # H*D above 4096
    (dict(out=GOOD + 0x1000000 + 4096), sm.SPECTRE_EINVAL),  # out overlaps k
    (dict(out=GOOD + 0x3000000), sm.SPECTRE_EINVAL),         # out == x
])
def test_fwd_rejects_before_device(kw, expect):
    assert fwd(**kw) == expect


def fwd_ex(gate_kind, norm_order, **kw):
    a = dict(q=GOOD, k=GOOD + 0x1000000, v=GOOD + 0x2000000, x=GOOD + 0x3000000,
             gate=GOOD + 0x4000000, gamma=GOOD + 0x5000000, beta=GOOD + 0x6000000,
             out=GOOD + 0x70000000, B=1, H=8, L=65536, D=64, keep_bins=32769, dtype=0)
    a.update(kw)
    return sm.spectre_mix_fwd_ex(a["q"], a["k"], a["v"], a["x"], a["gate"], a["gamma"], a["beta"],
                                 a["out"], a["B"], a["H"], a["L"], a["D"], a["keep_bins"],
                                 a["dtype"], gate_kind, norm_order, 0)


@pytest.mark.parametrize("gate_kind,norm_order", [(3, 0), (-1, 0), (0, 4), (2, -1)])
def test_fwd_ex_rejects_unknown_variant(gate_kind, norm_order):
    assert fwd_ex(gate_kind, norm_order) == sm.SPECTRE_EINVAL
    assert sm.spectre_mix_y_ex(GOOD, GOOD + 0x1000000, GOOD + 0x2000000, GOOD + 0x4000000,
                               GOOD + 0x70000000, 1, 8, 65536, 64, 32769, 0, 3, 0) == \
        sm.SPECTRE_EINVAL


def test_fwd_ex_checks_shapes_like_fwd():
    assert fwd_ex(2, 1, L=65535, keep_bins=1) == sm.SPECTRE_EINVAL
    assert fwd_ex(1, 0, L=5 * 4096, keep_bins=1) == sm.SPECTRE_EUNSUPPORTED
    assert fwd_ex(2, 1, q=GOOD + 8) == sm.SPECTRE_EINVAL


def test_chunked_rejects_before_device():
    args = dict(B=1, H=8, L=65536, D=64, F=4096, keep=2049, keepb=9)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return sm.spectre_mix_fwd_chunked(GOOD, GOOD + 0x1000000, GOOD + 0x2000000,
                                          GOOD + 0x3000000, GOOD + 0x4000000, GOOD + 0x4100000,
                                          GOOD + 0x5000000, GOOD + 0x6000000, GOOD + 0x70000000,
                                          a["B"], a["H"], a["L"], a["D"], a["F"], a["keep"],
                                          a["keepb"], 0, 0)
    assert call(F=3000) == sm.SPECTRE_EINVAL            # L not a multiple of fft_len
    assert call(L=3 * 4096) == sm.SPECTRE_EINVAL        # odd block count
    assert call(keepb=10) == sm.SPECTRE_EINVAL          # keep_blocks above nb/2 + 1
    assert call(keep=2050) == sm.SPECTRE_EINVAL         # keep_bins above fft_len/2 + 1
    assert call(F=2, L=16384, keep=2, keepb=1) == sm.SPECTRE_EUNSUPPORTED  # nb = 8192: too long
    assert call(F=5 * 1024, L=10 * 1024, keepb=1) == sm.SPECTRE_EUNSUPPORTED  # fft_len: factor 5


def test_local_rejects_before_device():
    def mix(**kw):
        a = dict(B=1, H=8, L=65536, D=64, keep=32769, wl=64, wr=64, dt=0, out=GOOD + 0x70000000)
        a.update(kw)
        return sm.spectre_mix_fwd_local(GOOD, GOOD + 0x1000000, GOOD + 0x2000000,
                                        GOOD + 0x3000000, GOOD + 0x4000000, GOOD + 0x5000000,
                                        GOOD + 0x6000000, a["out"], a["B"], a["H"], a["L"],
                                        a["D"], a["keep"], a["wl"], a["wr"], a["dt"], 0)
    assert mix(wl=-1) == sm.SPECTRE_EINVAL
    assert mix(wr=-5) == sm.SPECTRE_EINVAL
    assert mix(D=48, H=8) == sm.SPECTRE_EUNSUPPORTED     # head size the kernel lacks
    assert mix(L=65535, keep=1) == sm.SPECTRE_EINVAL      # checked like spectre_mix_fwd
    assert mix(out=GOOD + 0x3000000) == sm.SPECTRE_EINVAL  # out == x
    for gk, no in ((3, 0), (0, 4), (-1, 0)):  # unknown gate kind or norm order
        assert sm.spectre_mix_fwd_local_ex(GOOD, GOOD + 0x1000000, GOOD + 0x2000000,
                                           GOOD + 0x3000000, GOOD + 0x4000000, GOOD + 0x5000000,
                                           GOOD + 0x6000000, GOOD + 0x70000000, 1, 8, 65536, 64,
                                           32769, 64, 64, 0, gk, no, 0) == sm.SPECTRE_EINVAL

    def attn(**kw):
        a = dict(B=1, H=2, L=100, D=64, wl=3, wr=3, dt=0, y=GOOD + 0x1000000, q=GOOD)
        a.update(kw)
        return sm.spectre_mix_local_attention(a["q"], GOOD + 0x400000, GOOD + 0x800000, a["y"],
                                              a["B"], a["H"], a["L"], a["D"], a["wl"], a["wr"],
                                              a["dt"], 0)

    def gated(mix=GOOD + 0x6800000, no=0, **kw):
        a = dict(B=1, H=8, L=65536, D=64, keep=32769, wl=64, wr=64, dt=0)
        a.update(kw)
        return sm.spectre_mix_fwd_local_gated(GOOD, GOOD + 0x1000000, GOOD + 0x2000000,
                                              GOOD + 0x3000000, GOOD + 0x4000000, mix,
                                              GOOD + 0x5000000, GOOD + 0x6000000, GOOD + 0x70000000,
                                              a["B"], a["H"], a["L"], a["D"], a["keep"], a["wl"],
                                              a["wr"], a["dt"], 0, no, 0)
    assert gated(mix=0) == sm.SPECTRE_EINVAL               # the branch weights are required
    assert gated(mix=GOOD + 0x6800004) == sm.SPECTRE_EINVAL  # misaligned
    assert gated(no=4) == sm.SPECTRE_EINVAL
    assert gated(wl=-1) == sm.SPECTRE_EINVAL
    assert gated(D=48) == sm.SPECTRE_EUNSUPPORTED

    assert attn(L=0) == sm.SPECTRE_EINVAL
    assert attn(wl=-1) == sm.SPECTRE_EINVAL
    assert attn(dt=2) == sm.SPECTRE_EINVAL
    assert attn(D=24) == sm.SPECTRE_EUNSUPPORTED
    assert attn(q=GOOD + 4) == sm.SPECTRE_EINVAL          # misaligned
    assert attn(y=GOOD + 0x400000 + 64) == sm.SPECTRE_EINVAL  # y overlaps k
    assert attn(q=0) == sm.SPECTRE_EINVAL


def test_y_rejects_before_device():
    assert sm.spectre_mix_y(0, GOOD, GOOD, GOOD, GOOD, 1, 8, 4096, 64, 2049, 0, 0) == \
        sm.SPECTRE_EINVAL
    assert sm.spectre_mix_y(GOOD, GOOD, GOOD, GOOD, GOOD + 0x40000000, 1, 8, 4096, 64, 2050, 0,
                            0) == sm.SPECTRE_EINVAL
    # y overlapping q
    assert sm.spectre_mix_y(GOOD, GOOD, GOOD, GOOD, GOOD + 16, 1, 8, 4096, 64, 2049, 0, 0) == \
        sm.SPECTRE_EINVAL


def test_plan_factorisation():
    # 3072 and 4096: one pass, the whole column in one workgroup
    cases = {256: (1, 1, 256), 2048: (1, 1, 2048), 4096: (1, 1, 4096), 3072: (1, 1, 3072),
             6144: (6, 1, 1024), 8192: (8, 1, 1024), 12288: (12, 1, 1024), 16384: (16, 1, 1024),
             65536: (64, 1, 1024), 98304: (32, 3, 1024),
             786432: (64, 12, 1024), 3 * 2 ** 20: (64, 48, 1024), 2: (1, 1, 2), 6: (1, 1, 6)}
    for L, want in cases.items():
        st, got = sm.spectre_mix_plan(L)
        assert st == sm.SPECTRE_OK and got == want, (L, got)
        assert got[0] * got[1] * got[2] == L


def test_every_supported_length_plans():
    ok = 0
    for a in range(1, 22):
        for b in range(0, 2):
            L = 2 ** a * 3 ** b
            st, (l1, l2, l3) = sm.spectre_mix_plan(L)
            if L > 3 * 2 ** 20:
                assert st == sm.SPECTRE_EUNSUPPORTED
                continue
            assert st == sm.SPECTRE_OK, L
            assert l1 * l2 * l3 == L and l1 <= 64 and l2 <= 64 and l3 <= 4096
            ok += 1
    assert ok == 41  # 2^1..2^21 and 3*2^1..3*2^20


def test_workspace_bytes():
    """Three binary32 complex spectra (12 bytes per real element) for
    multi-level plans, a fourth for B's output when the first pass writes the
    tiled layout (two-level, 48- or 64-point first pass), six when a
    three-level plan's second pass writes it out of place, y (4 bytes per
    element) for single-level ones (y is binary32 whatever the storage),
    plus the H * L binary32 gate table when a multi-level plan's column
    length is 256 or 1024."""
    N = 1 * 65536 * 512
    gate_tab = 4 * 8 * 65536
    assert sm.spectre_mix_workspace_bytes(1, 8, 65536, 64, 0) == 16 * N + gate_tab
    assert sm.spectre_mix_workspace_bytes(2, 8, 65536, 64, 1) == 16 * 2 * N + gate_tab
    # L = 16384 = 16 x 1024: tiled with CP2 = 256; row layout (three spectra) with CP2 = 8
    assert sm.spectre_mix_workspace_bytes(1, 8, 16384, 64, 0) == 16 * 16384 * 512 + 4 * 8 * 16384
    assert sm.spectre_mix_workspace_bytes(1, 2, 16384, 8, 0) == 12 * 16384 * 16 + 4 * 2 * 16384
    # L = 786432 = 64 x 12 x 1024: second pass out of place, six spectra
    N5 = 786432 * 512
    assert sm.spectre_mix_workspace_bytes(1, 8, 786432, 64, 0) == 24 * N5 + 4 * 8 * 786432
    # L = 4096 and 3072: one pass (column kernel), y only, no gate table, while
    # B * CP2 / 4 <= 256; beyond that the four-step plan (4 x 1024, tiled)
    assert sm.spectre_mix_workspace_bytes(4, 8, 4096, 64, 0) == 4 * 4 * 4096 * 512
    assert sm.spectre_mix_workspace_bytes(2, 8, 3072, 64, 1) == 4 * 2 * 3072 * 512
    assert sm.spectre_mix_workspace_bytes(5, 8, 4096, 64, 0) == 16 * 5 * 4096 * 512 + 4 * 8 * 4096
    # the boundary: 4 x 64 = 256 items (one round) against 4 x 65 = 260 (H*D = 520: the
    # four-step plan, row layout since CP2 = 260 is not a multiple of 32)
    assert sm.spectre_mix_workspace_bytes(4, 8, 4096, 64, 0) == 4 * 4 * 4096 * 512
    assert sm.spectre_mix_workspace_bytes(4, 8, 4096, 65, 0) == 12 * 4 * 4096 * 520 + 4 * 8 * 4096
    # L = 2048: single level, generic LDS kernel, y only, no gate table
    assert sm.spectre_mix_workspace_bytes(4, 8, 2048, 64, 0) == 4 * 4 * 2048 * 512
    # L = 256: single level, square kernel reading the gate itself (no table)
    assert sm.spectre_mix_workspace_bytes(1, 2, 256, 16, 0) == 4 * 256 * 32
    assert sm.spectre_mix_workspace_bytes(1, 8, 65535, 64, 0) == 0
    # a complex gate doubles the gate table of multi-level plans; the others keep it
    assert sm.spectre_mix_workspace_bytes_ex(1, 8, 65536, 64, 0, 2) == \
        sm.spectre_mix_workspace_bytes(1, 8, 65536, 64, 0) + 4 * 8 * 65536
    assert sm.spectre_mix_workspace_bytes_ex(1, 8, 65536, 64, 0, 1) == \
        sm.spectre_mix_workspace_bytes(1, 8, 65536, 64, 0)
    assert sm.spectre_mix_workspace_bytes_ex(1, 2, 256, 16, 0, 2) == 4 * 256 * 32
    assert sm.spectre_mix_workspace_bytes_ex(1, 8, 65536, 64, 0, 5) == 0


def test_release_without_device_is_clean():
    assert sm.spectre_mix_release() == sm.SPECTRE_OK


def test_noalloc_rejects_before_device():
    """The allocation-free entry point validates like spectre_mix_fwd and
    refuses, before any device call, the plans it does not serve: three
    levels (L = 98304 = 64 x 1.5 x 1024 plans as 64 x 3 x 512) and workspaces
    beyond its 64 MiB array."""
    def call(**kw):
        a = dict(q=GOOD, k=GOOD + 0x1000000, v=GOOD + 0x2000000, x=GOOD + 0x3000000,
                 gate=GOOD + 0x4000000, gamma=GOOD + 0x5000000, beta=GOOD + 0x6000000,
                 out=GOOD + 0x70000000, B=1, H=8, L=4096, D=64, keep_bins=2049, dtype=0)
        a.update(kw)
        return sm.spectre_mix_fwd_noalloc(a["q"], a["k"], a["v"], a["x"], a["gate"], a["gamma"],
                                          a["beta"], a["out"], a["B"], a["H"], a["L"], a["D"],
                                          a["keep_bins"], a["dtype"], 0)
    assert call(q=0) == sm.SPECTRE_EINVAL
    assert call(L=4095) == sm.SPECTRE_EINVAL
    assert call(q=GOOD + 8) == sm.SPECTRE_EINVAL
    assert call(out=GOOD + 0x3000000) == sm.SPECTRE_EINVAL
    assert call(L=98304, keep_bins=1) == sm.SPECTRE_EUNSUPPORTED   # three-level plan
    assert call(L=65536, keep_bins=1) == sm.SPECTRE_EUNSUPPORTED   # 537 MB of workspace
    assert call(B=8, L=4096, keep_bins=1) == sm.SPECTRE_EUNSUPPORTED  # y: 4 N bytes = 64 MiB, + tables
