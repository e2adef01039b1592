"""Builds the HIP/C++ library in-tree: ``liblora_sgmv.so`` next to this file.

hipcc cross-compiles for gfx950 without a GPU.  Packed-fp32 instructions are
disabled for the device code (``-packed-fp32-ops``); the host pass warns that it
does not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "liblora_sgmv.so")
SOURCES = [os.path.join(HERE, "csrc", "host.cpp"), os.path.join(HERE, "csrc", "kernels.hip"),
           os.path.join(HERE, "csrc", "base_gemm.hip"), os.path.join(HERE, "csrc", "residency.hip"),
           os.path.join(HERE, "csrc", "probe.hip")]
HEADERS = [os.path.join(ROOT, "include", "lora_sgmv.h"),
           os.path.join(HERE, "csrc", "lora_internal.h")]
ARCH = os.environ.get("LORA_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def command(out: str = LIB, extra=()) -> list:
    return [HIPCC, "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function",
            "-I", os.path.join(ROOT, "include"), *extra, *SOURCES, "-o", out]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


def up_to_date() -> bool:
    if not os.path.exists(LIB):
        return False
    t = os.path.getmtime(LIB)
    return all(os.path.getmtime(s) <= t for s in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
