"""Build the gfx950 HIP library ``libmhla.so`` in-tree with hipcc.

Every source under ``csrc/`` is compiled for gfx950 only; objects go to ``_build/`` at the
repository root and the shared library next to this file, where the binding loads it.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmhla.so")
# the benchmark's measured-peak probe, a library of its own outside the MHLA path
PEAK_SOURCE = "peak_probe.hip"
PEAK_LIB = os.path.join(PKG, "libmhla_peak.so")

SOURCES = ["summary.hip", "summary_dma.hip", "mix.hip", "mix_mfma.hip", "readout.hip", "bwd.hip", "causal.hip", "causal_slice.hip", "decode.hip",
           "mhla_host.cpp", "noalloc.hip", "stacks.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the MHLA library)")


COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # packed fp32 instructions stay off: ordinary float code is compiled to scalar VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str, build_dir: str = BUILD, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    lang = [] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [hipcc(), *COMMON, *[f"-D{d}" for d in defines], "-I", INCLUDE, "-I", CSRC, *lang, "-c",
           os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = False, out: str = LIB, build_dir: str = BUILD, defines=()) -> str:
    """Compile every source and link `out`.  `defines` are extra -D macros (build variants)."""
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, defines), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}", file=sys.stderr)
    if out == LIB:
        build_peak_probe(build_dir)
    return out


def build_peak_probe(build_dir: str = BUILD) -> str:
    """The benchmark's MFMA-loop probe as its own shared library (``libmhla_peak.so``)."""
    os.makedirs(build_dir, exist_ok=True)
    obj = _compile(PEAK_SOURCE, build_dir)
    tmp = PEAK_LIB + ".tmp"
    res = subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, obj],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, PEAK_LIB)
    return PEAK_LIB


if __name__ == "__main__":
    build(verbose=True)
