"""Builds libfpi8.so (the HIP library, gfx950) in this package directory.

Each source compiles to its own object in _build/ (in parallel), then one
link step writes the library.
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libfpi8.so")
OBJ_DIR = os.path.join(os.path.dirname(HERE), "_build", "fpi8")
SOURCES = ["csrc/fpi8_host.cpp", "csrc/fpi8_engine.cpp", "csrc/fpi8_tokenizer.cpp",
           "csrc/fpi8_pages.cpp", "csrc/fpi8_charges.cpp", "csrc/fpi8_planner.cpp",
           "csrc/fpi8_kernels.hip",
           "csrc/fpi8_rows_stream.hip", "csrc/fpi8_noalloc.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
         # No packed-FP32 instructions in device code.  Only the device pass
         # knows this feature; the host pass warns that it does not, which is
         # harmless.
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = ["hipcc", *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + r.stdout + r.stderr)
    return obj


def build() -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    # -z defs: a symbol the library uses but nothing defines fails the link, not the first load
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp]
    r = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
