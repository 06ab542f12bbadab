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
# (source, extra defines) per object; the head-dim-128 decode file is built
# once per (q, cache) dtype pair so the pairs compile in parallel
UNITS = [("pa_kernels.hip", []), ("pa_api.cpp", []), ("pa_noalloc.hip", []), ("pa_prefill.hip", [])] + [
    ("pa_decode_fast.hip", [f"-DPA_FAST_COMBO={i}"]) for i in range(4)]
SOURCES = sorted({os.path.join(PKG, "csrc", f) for f, _ in UNITS})
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
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


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def _finish(proc, verbose):
    out, err = proc.communicate()
    if proc.returncode != 0:
        sys.stderr.write(out + err)
        raise RuntimeError(f"hipcc failed with status {proc.returncode}")
    noise = [l for l in err.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel, one object each) and link
    ``libpa.so``; returns its path."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs, procs = [], []
    for name, defs in UNITS:
        obj = os.path.join(objdir, name + "".join(d.replace("-D", ".").replace("=", "") for d in defs) + ".o")
        objs.append(obj)
        procs.append(_run([hipcc(), *FLAGS, *defs, "-c", os.path.join(PKG, "csrc", name), "-o", obj], verbose))
    for p in procs:
        _finish(p, verbose)
    tmp = LIB + ".tmp"
    _finish(_run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose), verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
