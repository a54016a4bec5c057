"""bench.py's host side on a machine without a GPU: the byte models its
roofline divides by, and the argument checks that end a run before any
device work."""
import os
import subprocess
import sys

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_window_must_be_even_and_unchunked():
    assert run_bench("--window", "127").returncode == 2
    assert run_bench("--window", "128", "--fft-len", "4096").returncode == 2


def test_byte_models_of_the_long_workload():
    """Workload 3 (B=1, L=65536, H=8, D=64, binary32; N = 2^25 elements):
    A1 reads q, k, v (12N bytes) and writes three spectra (12N) plus the
    gate table it builds (4 H L) from the kept gate bins (4 H (L/2+1));
    B reads the three spectra, writes U (4N) and reads the table; C1 reads U
    and x, writes out (12N) plus gamma and beta; the local branch reads q,
    k, v and writes y_loc (16N)."""
    w = workloads.WORKLOADS[3]
    N = 2 ** 25
    gate = 4 * 8 * 32769
    table = 4 * 8 * 65536
    assert bench.kernel_bytes("A1_fwd_strided", w) == 24 * N + gate + table
    assert bench.kernel_bytes("B_mid_lds", w) == 16 * N + table
    assert bench.kernel_bytes("C1_inv_norm", w) == 12 * N + 8 * 512
    assert bench.kernel_bytes("C1_inv_norm", w, local=True) == 16 * N + 8 * 512
    assert bench.kernel_bytes("L_local", w) == 16 * N
    # the frozen whole-call model: 5 N s + 4 H K + 8 H D, plus 32 N of exchanges
    assert bench.model_bytes(w) == 20 * N + gate + 8 * 512 + 32 * N


def test_complex_gate_doubles_gate_bytes():
    w = workloads.WORKLOADS[3]
    assert bench.kernel_bytes("B_mid_lds", w, gate_kind=2) - bench.kernel_bytes("B_mid_lds", w) == \
        4 * 8 * 65536


def test_short_names_of_library_kernels():
    assert bench._short("void spectre::k_mid_dma<false, 17>(spectre::MidParams)") == "B_mid_lds"
    assert bench._short("void spectre::k_local_attn<0, 64>(spectre::LocalParams)") == "L_local"
    assert bench._short("void spectre::k_layernorm<0, false>(spectre::NormParams)") == "LN_norm"
    assert bench._short("void spectre::k_layernorm2<0, false, 2>(spectre::NormParams)") == "LN_norm"
    assert bench._short("void spectre::k_col<16, 16, 16, 4, 0>(spectre::ColParams)") == "B_col"
    assert bench._short("__amd_rocclr_copyBuffer") == "copy (calibration)"
