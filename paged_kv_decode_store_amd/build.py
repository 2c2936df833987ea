"""Build libpkv.so (HIP for gfx950) in-tree with hipcc.

    python -m paged_kv_decode_store_amd.build

Device code is compiled with packed-fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops); the host pass warns that
it does not know the feature, which is harmless.  No fast-math: the sampler
relies on IEEE fp32 division.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build", "pkv")
LIB_PATH = os.path.join(PKG, "libpkv.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
DEVICE_SOURCES = ["slot_store.hip", "decode_attention.hip", "decode_attention_mfma.hip",
                  "varlen_attention.hip", "sampler.hip", "static_scratch.hip", "probe.hip"]
HOST_SOURCES = ["api.cpp"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I" + os.path.join(ROOT, "include")]
DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang",
                "-packed-fp32-ops"]
# Per-file extras.  The varlen attention kernel masks by position (a select,
# never arithmetic on NaN), so NaN semantics are dropped there: its fmaxf on
# matrix-core results then needs no quieting instruction per operand.
FILE_FLAGS = {"varlen_attention.hip": ["-fno-honor-nans"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if out.strip() and verbose:
        print(out, file=sys.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    objs = []
    for src in DEVICE_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append([HIPCC, "-x", "hip", "-c", *COMMON, *DEVICE_FLAGS, *FILE_FLAGS.get(src, []),
                     os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append([HIPCC, "-c", *COMMON, os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(4, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
