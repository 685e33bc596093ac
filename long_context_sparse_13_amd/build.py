"""Compile the HIP kernels and the C ABI into long_context_sparse_13_amd/libsa.so (gfx950),
and the memory read probe that bench.py times into libsa_probe.so.

Run ``python -m long_context_sparse_13_amd.build`` (or ``__graft_entry__.build()``).
Objects go to ``_build/`` at the repository root; the shared library is written
in-tree next to this file so that it travels with the source tree.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libsa.so")
# the memory-hierarchy read probe that bench.py times (measurement only, not libsa)
PROBE = os.path.join(PKG, "probe")
PROBE_OUT = os.path.join(PKG, "libsa_probe.so")
BUILD = os.path.join(ROOT, "_build")
ARCH = os.environ.get("SA_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Wall", "-Wno-unused-function",
    # hipcc's own packed-FP32 selection is kept off (the host pass warns that it does
    # not know the feature; that warning is harmless)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Per-source extra flags: the indexer kernels keep their MFMA accumulators in VGPRs
# (the epilogue reads every accumulator element, so AGPR copies would cost VALU slots).
EXTRA_FLAGS = {
    "k_indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "k_indexer_topk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libsa)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [_hipcc(), *FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), *lang, "-c", src,
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def probe_sources():
    return sorted(os.path.join(PROBE, f) for f in os.listdir(PROBE) if f.endswith(".hip"))


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs, psrcs = sources(), probe_sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(psrcs))) as ex:
        objs = list(ex.map(_compile, srcs + psrcs))
    _link(objs[: len(srcs)], OUT)
    _link(objs[len(srcs):], PROBE_OUT)
    if verbose:
        print(f"built {OUT} and {PROBE_OUT}")
    return OUT


if __name__ == "__main__":
    build()
