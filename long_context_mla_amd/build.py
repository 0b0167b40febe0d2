"""Build the gfx950 HIP library in-tree: long_context_mla_amd/libmla_decode.so.

``python long_context_mla_amd/build.py`` compiles every source under ``csrc/``
with hipcc for gfx950 only.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla_decode.so")
SOURCES = ["api.hip", "kv_append.hip", "mla_decode.hip", "mla_decode_fp8.hip", "mla_combine.hip", "kv_check.hip"]
# measured-peak microbenchmarks (bench.py --peaks): a library of their own
PEAKS_LIB = os.path.join(HERE, "libmla_peaks.so")
PEAKS_SOURCES = ["peaks.hip"]
ARCH = "gfx950"

FLAGS = [
    "-O3",
    "-std=c++17",
    f"--offload-arch={ARCH}",
    "-fPIC",
    "-shared",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


def build(extra_flags=(), verbose: bool = False, out: str = LIB, sources=None) -> str:
    srcs = [os.path.join(CSRC, s) for s in (SOURCES if sources is None else sources)]
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, *extra_flags, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    if verbose and (r.stdout or r.stderr):
        print(r.stdout + r.stderr, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False) -> list:
    return [build(verbose=verbose), build(verbose=verbose, out=PEAKS_LIB, sources=PEAKS_SOURCES)]


if __name__ == "__main__":
    print(build_all(verbose=True))
