"""Builds the HIP/C++ library in-tree: ``liblora_sgmv.so`` next to this file,
and ``liblora_sgmv_debug.so``, the same sources with ``-DLORA_DEBUG=1`` (kernels
record bad ids, pages, ranks, tokens and plan items in an error word that
``lora_debug_flags`` reads back).

hipcc cross-compiles for gfx950 without a GPU.  The sources are compiled to
objects in parallel processes, then linked.  Packed-fp32 instructions are
disabled for the device code (``-packed-fp32-ops``); the host pass warns that it
does not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "liblora_sgmv.so")
DEBUG_LIB = os.path.join(HERE, "liblora_sgmv_debug.so")
SOURCES = [os.path.join(HERE, "csrc", "host.cpp"), os.path.join(HERE, "csrc", "kernels.hip"),
           os.path.join(HERE, "csrc", "base_gemm.hip"), os.path.join(HERE, "csrc", "residency.hip"),
           os.path.join(HERE, "csrc", "probe.hip")]
HEADERS = [os.path.join(ROOT, "include", "lora_sgmv.h"), os.path.join(ROOT, "include", "lora_probe.h"),
           os.path.join(HERE, "csrc", "lora_internal.h")]
ARCH = os.environ.get("LORA_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]
NOISE = "is not a recognized feature for this target"


def command(out: str = LIB, extra=()) -> list:
    """One hipcc command that compiles and links every source into `out`."""
    return [HIPCC, *FLAGS, "-shared", *extra, *SOURCES, "-o", out]


def _clean(stderr: str) -> str:
    return "\n".join(l for l in stderr.splitlines() if NOISE not in l)


def build(verbose: bool = False) -> str:
    """Compiles every source for both libraries (release and debug) in
    parallel, then links each; replaces the libraries only when all succeed."""
    with tempfile.TemporaryDirectory(prefix="lora_build_") as tmp:
        jobs = []
        for tag, extra in (("rel", []), ("dbg", ["-DLORA_DEBUG=1"])):
            for src in SOURCES:
                obj = os.path.join(tmp, f"{tag}_{os.path.basename(src)}.o")
                cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
                if verbose:
                    print(" ".join(cmd), flush=True)
                jobs.append((tag, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                        stderr=subprocess.PIPE, text=True)))
        objs = {"rel": [], "dbg": []}
        errors = []
        for tag, obj, p in jobs:
            _, err = p.communicate()
            err = _clean(err)
            if p.returncode != 0:
                errors.append(err)
            elif verbose and err.strip():
                print(err, file=sys.stderr)
            objs[tag].append(obj)
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
        for tag, out in (("rel", LIB), ("dbg", DEBUG_LIB)):
            cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", *objs[tag], "-o", out + ".tmp"]
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError(f"link failed ({res.returncode}):\n{_clean(res.stderr)}")
        os.replace(LIB + ".tmp", LIB)
        os.replace(DEBUG_LIB + ".tmp", DEBUG_LIB)
    return LIB


def up_to_date() -> bool:
    if not (os.path.exists(LIB) and os.path.exists(DEBUG_LIB)):
        return False
    t = min(os.path.getmtime(LIB), os.path.getmtime(DEBUG_LIB))
    return all(os.path.getmtime(s) <= t for s in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
