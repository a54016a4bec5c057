"""The kernels' register DFTs (efficient_attention_fft_amd/csrc/dft.hpp),
compiled for the host, against the DFT definition.

Every pass of the GPU path transforms its columns with dft<R, SIGN> for
compile-time R: radix-2, -3 and -4 butterflies, the multiply-add radix-2
form for powers of two from 8 up, and the mixed split for 6, 12, 24 and 48.
Here each size a pass uses runs on the CPU (hipcc's host compiler, the
device qualifiers widened to host + device) on seeded inputs and is compared
with X[f] = sum_n x[n] exp(SIGN 2 pi i f n / R) evaluated in double; the
bound, 4e-7 of max |X|, is a few units of binary32 rounding for these sizes.
No GPU is involved.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DFT_HPP = os.path.join(ROOT, "efficient_attention_fft_amd", "csrc", "dft.hpp")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SIZES = (2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64)

PROGRAM = r"""
#include "dft_host.hpp"
#include <cstdio>
#include <cstdlib>
template <int R, int SIGN> void run(const float* in) {
  float2 a[R];
  for (int i = 0; i < R; ++i) a[i] = make_float2(in[2 * i], in[2 * i + 1]);
  spectre::dft<R, SIGN>(a);
  printf("%d %d", R, SIGN);
  for (int i = 0; i < R; ++i) printf(" %.9e %.9e", a[i].x, a[i].y);
  printf("\n");
}
int main(int argc, char** argv) {
  static float in[128];
  for (int i = 0; i < 128; ++i) in[i] = (float)atof(argv[1 + i]);
#define BOTH(R) run<R, -1>(in); run<R, 1>(in);
  BOTH(2) BOTH(3) BOTH(4) BOTH(6) BOTH(8) BOTH(12) BOTH(16) BOTH(24) BOTH(32) BOTH(48) BOTH(64)
  return 0;
}
"""


@pytest.fixture(scope="module")
def host_dfts(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("dft_host")
    with open(DFT_HPP) as f:
        src = f.read().replace("__device__ __forceinline__", "__host__ __device__ __forceinline__")
    (d / "dft_host.hpp").write_text(src)
    (d / "main.cpp").write_text(PROGRAM)
    exe = d / "dft_host"
    subprocess.run([HIPCC, "-x", "hip", "--offload-host-only", "-O2", "-std=c++17",
                    str(d / "main.cpp"), "-o", str(exe)], check=True, capture_output=True)
    rng = np.random.default_rng(2024)
    x = rng.standard_normal(128).astype(np.float32)
    out = subprocess.run([str(exe)] + ["%.9e" % v for v in x], check=True, capture_output=True,
                         text=True).stdout.split("\n")
    res = {}
    for line in out:
        if not line.strip():
            continue
        f = line.split()
        R, sign = int(f[0]), int(f[1])
        v = np.array(f[2:], dtype=np.float64)
        res[(R, sign)] = v[0::2] + 1j * v[1::2]
    return x.astype(np.float64), res


@pytest.mark.parametrize("sign", (-1, 1))
@pytest.mark.parametrize("R", SIZES)
def test_register_dft_matches_definition(host_dfts, R, sign):
    x, res = host_dfts
    z = x[0:2 * R:2] + 1j * x[1:2 * R:2]
    n = np.arange(R)
    want = np.array([np.sum(z * np.exp(sign * 2j * np.pi * ((f * n) % R) / R)) for f in range(R)])
    got = res[(R, sign)]
    assert got.shape == (R,)
    err = np.max(np.abs(got - want))
    assert err <= 4e-7 * np.max(np.abs(want)), (R, sign, err)
