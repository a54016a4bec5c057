"""Compile the gfx950 HIP library into the package directory (libspectre_mix.so).

Run as a script (python efficient_attention_fft_amd/csrc/build.py): the package
itself cannot be imported before the library exists.

hipcc cross-compiles for gfx950 without a GPU.  Packed-FP32 instruction
selection is turned off for all device code.
"""
from __future__ import annotations

import os
import subprocess

CSRC = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(CSRC)
SRC = os.path.join(CSRC, "spectre_mix.hip")
LIB = os.path.join(PKG, "libspectre_mix.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = [HIPCC] + FLAGS + ["-o", tmp, SRC]
        proc = subprocess.run(cmd, capture_output=True, text=True)
        if proc.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + proc.stderr[-8000:])
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
