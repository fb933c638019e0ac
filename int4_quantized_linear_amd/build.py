"""Build libconvrot.so (the gfx950 HIP kernels + C-ABI) in-tree with hipcc.

Usage: python -m int4_quantized_linear_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libconvrot.so")
ARCH = "gfx950"

SOURCES = ["convrot_abi.hip", "rotate_quant.hip", "gemm_i8.hip", "gemv_i8.hip", "gemm_w4a4.hip", "gemv_w4a8.hip"]

# Packed-fp32 VALU forms are disabled on purpose: plain fp32 code is emitted instead.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-Wno-unused-command-line-argument"]
# Per-source extras.  The W4A4 GEMM keeps its group fold where it is written: machine sinking
# would move it past the load-issue branches, after the barrier, and spill.
SOURCE_FLAGS = {"gemm_w4a4.hip": ["-mllvm", "-disable-machine-sink"]}


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def _compile(src: str, obj: str) -> None:
    cmd = [_hipcc(), *COMMON, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))


def build(verbose: bool = False) -> str:
    """Compile every kernel source for gfx950 and link libconvrot.so (always rebuilds)."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        list(ex.map(_compile, SOURCES, objs))
    tmp = LIB + ".tmp%d" % os.getpid()
    # the version script keeps the internal C++ launchers local: only convrot_* is exported
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH,
           "-Wl,--version-script=" + os.path.join(CSRC, "libconvrot.map"), "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
