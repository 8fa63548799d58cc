"""Builds libfpi8.so (the HIP library, gfx950) in this package directory."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libfpi8.so")
SOURCES = ["csrc/fpi8_host.cpp", "csrc/fpi8_engine.cpp", "csrc/fpi8_tokenizer.cpp",
           "csrc/fpi8_pages.cpp", "csrc/fpi8_charges.cpp", "csrc/fpi8_kernels.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17", "-Wall",
         # no packed-FP32 instructions in any kernel
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build() -> str:
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *FLAGS, *SOURCES, "-o", tmp]
    r = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
