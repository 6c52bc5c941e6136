"""Builds libtq.so in-tree: every csrc/*.hip and csrc/*.cpp compiled by hipcc for gfx950,
then linked into one shared library next to this file."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtq.so")

ARCH = "gfx950"
# packed-fp32 VALU forms are disabled for every HIP translation unit
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I", INCLUDE, "-I", CSRC]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


# per-source extra flags: the search, prefill and token-sliced decode scans keep their MFMA
# accumulators in VGPRs (they read them back every tile; the AGPR form costs one copy per
# accumulator).  The token-sliced decode is compiled on the assumption that its float values
# are not NaN: fmaxf then needs no quieting of operands that come from lane exchanges (one
# instruction each); the one place where NaN products can arise (zero weights times the
# unbounded norms of masked tokens) selects on the bits.
EXTRA = {"tq_search.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "tq_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "tq_decode_mx.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, hipcc: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc, *COMMON, *DEVICE, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc, *COMMON, "-x", "hip", *DEVICE, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        print(res.stderr, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile and link libtq.so (always rebuilds).  Returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
