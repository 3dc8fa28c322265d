"""Build libmla_decode.so in-tree with hipcc for gfx950.

    python -m mla_token_decode_amd.build

Compiles the host plan, the C ABI and the HIP kernels into one shared library
next to this file, and the cold read-stream probe (stream_read.hip) into
libmla_stream.so, which only the benchmark loads.  Packed-fp32 instruction
selection is disabled on purpose (`-target-feature -packed-fp32-ops`): the
kernels never rely on it.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmla_decode.so")
STREAM_LIB = os.path.join(HERE, "libmla_stream.so")
STREAM_SOURCE = "stream_read.hip"
SOURCES = ["api.cpp", "plan.cpp", "kernels.hip", "kernels_paged.hip", "fp8_decode.hip",
           "fp8_decode_paged.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def compile_flags():
    return ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I" + INCLUDE, "-I" + CSRC]


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel (the two kernel files are
    the long ones), then link the shared library."""
    import tempfile
    with tempfile.TemporaryDirectory(prefix="mla_build_") as tmpdir:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmpdir, src + ".o")
            cmd = [HIPCC, *compile_flags(), "-c", "-o", obj, os.path.join(CSRC, src)]
            if verbose:
                print(" ".join(cmd), flush=True)
            objs.append(obj)
            procs.append((cmd, subprocess.Popen(cmd)))
        stmp = STREAM_LIB + f".tmp{os.getpid()}"
        cmd = [HIPCC, *compile_flags(), "-shared", "-o", stmp, os.path.join(CSRC, STREAM_SOURCE)]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd)))
        for cmd, p in procs:
            if p.wait() != 0:
                raise subprocess.CalledProcessError(p.returncode, cmd)
        tmp = LIB + f".tmp{os.getpid()}"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    os.replace(stmp, STREAM_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
