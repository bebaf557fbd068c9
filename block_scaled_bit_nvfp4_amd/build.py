"""Build libnvfp4.so (gfx950 HIP kernels + C ABI) in-tree with hipcc.

    python -m block_scaled_bit_nvfp4_amd.build
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
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libnvfp4.so")
# The measurement aid bench.py times the products against (nvfp4_probe.h).
PROBE_SRC = os.path.join(PKG, "probe", "nvfp4_probe.hip")
PROBE_LIB_PATH = os.path.join(PKG, "libnvfp4_probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-ffp-contract=off",                       # every fused multiply-add is written out
    # dot2 as the three-operand VOP3P form: a chain can start from the inline
    # constant 0 instead of a register copy of it
    "-Xclang", "-target-feature", "-Xclang", "-dot13-insts",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I" + INCLUDE, "-I" + CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC] + CFLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l and "dot13-insts" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, out):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    """Compile every .hip source for gfx950 and link libnvfp4.so, and the
    measurement probe into libnvfp4_probe.so (always rebuilds)."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError("hipcc not found (%s)" % HIPCC)
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources() + [PROBE_SRC]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:-1], LIB_PATH)
    _link(objs[-1:], PROBE_LIB_PATH)
    if verbose:
        print("built", LIB_PATH, "and", PROBE_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build()
