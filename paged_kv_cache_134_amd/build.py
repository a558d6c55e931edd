"""Build libpagedattn.so in-tree with hipcc for gfx950.

Usage: python paged_kv_cache_134_amd/build.py   (or __graft_entry__.build())

Every HIP source is compiled with packed FP32 instructions disabled
(-target-feature -packed-fp32-ops); the host-only block pool is compiled with
g++.  Objects go to paged_kv_cache_134_amd/_build/, the library next to this
file.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpagedattn.so")

ARCH = "gfx950"
HIP_SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))  # every HIP source
CXX_SOURCES = ["pool.cpp"]


def _hipcc() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    common = ["-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC]
    cmds = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, f"--offload-arch={ARCH}", *common,
                     "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                     "-munsafe-fp-atomics", "-c", os.path.join(CSRC, src), "-o", obj])
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src.replace(".cpp", ".o"))
        objs.append(obj)
        cmds.append(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC,
                     "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        outs = list(ex.map(_run, cmds))
    if verbose:
        for c, o in zip(cmds, outs):
            print(" ".join(c))
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
