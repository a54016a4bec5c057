"""The chunked (blockwise) mix on the GPU against the oracle, through
spectre_mix_fwd_chunked / spectre_mix_y_chunked: blocks of fft_len tokens
mixed on their own plus the block means mixed over the block axis (the
SPECTRE article's section 3.2 fft_len below L; the inter-block step is this
library's reading, pinned in the oracle tests).

Tolerances as for the plain mix: max-abs on out 1e-4 (binary32 storage),
2e-2 (bfloat16 storage); y within 1e-4 * max(1, max|y|).  The block sizes
cover the single-level square and generic LDS kernels, the two-level
LDS-copy kernel with the one-lane and the split fused inverse, and the
three-level plan.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import dev, empty_like_storage, oracle_threads, to_host_f64, tol, torch, y_tol

pytestmark = pytest.mark.gpu

CASES = [
    # (B, L, H, D, dtype, fft_len, keep_bins, keep_blocks)
    (1, 65536, 8, 64, 0, 4096, 2049, 9),     # the article's 4096-token blocks; 4 x 1024 plan
    (1, 16384, 4, 64, 0, 4096, 2049, 3),     # 4096-token blocks in one round of the column kernel
    (2, 12288, 2, 32, 1, 3072, 1000, 2),     # 3072-token blocks, column kernel, bf16
    (1, 8192, 2, 8, 0, 2, 2, 700),           # a block axis of 4096 blocks through the column kernel
    (2, 16384, 4, 32, 0, 2048, 700, 5),      # single-level generic LDS kernel, nb = 8
    (1, 49152, 2, 64, 0, 8192, 4097, 2),     # 8 x 1024 blocks, nb = 6, truncated block axis
    (1, 16384, 8, 64, 1, 256, 100, 20),      # single-level square kernel, bf16, nb = 64
    (1, 131072, 2, 64, 0, 65536, 32769, 2),  # 64 x 1024 blocks: split fused inverse, nb = 2
    (1, 196608, 1, 32, 0, 98304, 49153, 2),  # three-level blocks (32 x 3 x 1024)
]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("B,L,H,D,dt,F,keep,keepb", CASES)
def test_chunked_against_oracle(B, L, H, D, dt, F, keep, keepb):
    import efficient_attention_fft_amd as sm
    t = torch()
    w = workloads.custom(500 + L % 89, B=B, L=L, H=H, D=D, dtype=dt, keep_bins=keep, affine=True)
    say("case", w.describe(), "fft_len", F, "keep_blocks", keepb)
    inp = workloads.make_inputs(w)
    g, gb = workloads.make_chunk_gates(w, F)
    ref_out, ref_y = oracle.spectre_mix_chunked(inp["q"], inp["k"], inp["v"], inp["x"], g, gb,
                                                inp["gamma"], inp["beta"], F, keep, keepb,
                                                dtype=dt, nthreads=oracle_threads(), want_y=True)
    q, k, v, x = (dev(inp[n]) for n in "qkvx")
    gd, gbd, gam, bet = dev(g), dev(gb), dev(inp["gamma"]), dev(inp["beta"])
    _, out = empty_like_storage(w)
    sm.check(sm.spectre_mix_fwd_chunked(q, k, v, x, gd, gbd, gam, bet, out, B, H, L, D, F, keep,
                                        keepb, dt))
    t.cuda.synchronize()
    got = to_host_f64(out, dt).reshape(ref_out.shape)
    err = np.abs(got - ref_out).max()
    say("  out max-abs err %.3g (tol %.1g)" % (err, tol(w)))
    assert np.all(np.isfinite(got)) and err <= tol(w)
    y = t.full((w.N,), float("nan"), dtype=t.float32, device="cuda")
    sm.check(sm.spectre_mix_y_chunked(q, k, v, gd, gbd, y, B, H, L, D, F, keep, keepb, dt))
    t.cuda.synchronize()
    gy = y.cpu().numpy().astype(np.float64).reshape(ref_y.shape)
    ey = np.abs(gy - ref_y).max()
    say("  y max-abs err %.3g (tol %.3g)" % (ey, y_tol(ref_y)))
    assert ey <= y_tol(ref_y)


def test_chunked_rejects_bad_block_sizes():
    import efficient_attention_fft_amd as sm
    t = torch()
    a = t.zeros(1 << 16, device="cuda")
    p = a.data_ptr()
    # L not a multiple of fft_len; an odd block count; keep_blocks above nb/2 + 1
    for L, F, kb in ((4096, 1536, 1), (3 * 4096, 4096, 1), (8192, 1024, 6)):
        assert sm.spectre_mix_fwd_chunked(p, p, p, p, p, p, p, p, p + 4096, 1, 1, L, 2, F, 2, kb,
                                          0) == sm.SPECTRE_EINVAL
