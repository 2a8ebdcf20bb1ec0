"""Build the gfx950 C-ABI library ``libeagle3.so`` in-tree with hipcc.

Every .hip file under csrc/ is compiled to an object (in parallel) and
linked into eagle_draft_tree_amd/libeagle3.so.  Always rebuilds.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libeagle3.so")
ARCH = os.environ.get("EAGLE3_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result", "-ffp-contract=fast"]
# The tiled GEMM's epilogues walk a fully unrolled 8 x 8 accumulator grid; a
# higher full-unroll budget keeps the accumulators in registers (no
# dynamically indexed copy in scratch).
EXTRA = {"ttt.hip": ["-mllvm", "-pragma-unroll-threshold=200000"],
         "ttt_bwd.hip": ["-mllvm", "-pragma-unroll-threshold=200000"]}


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + EXTRA.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    return obj, err


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        res = list(ex.map(_compile, srcs))
    if verbose:
        for (o, err) in res:
            if err.strip():
                print(err)
    objs = [o for o, _ in res]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
