"""Build libpa.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

``python -m paged_kv_cache_91_amd.build`` or :func:`build`.  The library is
written next to this file; tests, ``smoke()`` and ``bench.py`` load it from
there and never build it themselves.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libpa.so")
SOURCES = [os.path.join(PKG, "csrc", f) for f in ("pa_kernels.hip", "pa_decode_fast.hip", "pa_api.cpp")]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    # keep packed-fp32 instructions out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: left to its heuristics the compiler
    # adds accumulation registers on top of ~200 VGPRs, which halves how many
    # decode waves a SIMD holds
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # the first scalar kernel arguments arrive preloaded in SGPRs rather than
    # through a load of the argument block at the start of every wave
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I" + os.path.join(ROOT, "include"),
    "-I" + os.path.join(PKG, "csrc"),
]


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    """Compile every source into ``libpa.so``; returns its path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    noise = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
