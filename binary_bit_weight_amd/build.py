"""Builds the gfx950 C-ABI library ``liblowbit.so`` in-tree with hipcc.

Every HIP translation unit is compiled with ``-Xclang -target-feature
-Xclang -packed-fp32-ops`` (no packed fp32 instructions) and
``-ffp-contract=off`` (every fp32 multiply and add is its own IEEE
operation unless the source asks for an fma), then linked into one shared
object next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblowbit.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-fPIC", "-std=c++17", "-ffp-contract=off", "-Wall", "-Wno-unused-function",
          "-I", INCLUDE, "-I", CSRC]
DEVICE = ["-x", "hip", "--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def sources():
    hip = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    cpp = sorted(f for f in os.listdir(CSRC) if f.endswith(".cpp"))
    return hip, cpp


def _compile(src: str, obj: str, device: bool):
    cmd = [HIPCC, *COMMON, *(DEVICE if device else ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include"]), "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    return err


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hip, cpp = sources()
    jobs = [(s, os.path.join(BUILD, s + ".o"), True) for s in hip] + \
           [(s, os.path.join(BUILD, s + ".o"), False) for s in cpp]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        futs = {ex.submit(_compile, *j): j[0] for j in jobs}
        for f in cf.as_completed(futs):
            msg = f.result()
            if verbose and msg.strip():
                print("[%s]\n%s" % (futs[f], msg), file=sys.stderr)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *[j[1] for j in jobs]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
