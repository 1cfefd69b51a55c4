"""Build ``libmamba2.so`` (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmamba2.so")
OBJ = os.path.join(ROOT, "_build")
ARCH = os.environ.get("MAMBA2_OFFLOAD_ARCH", "gfx950")

SOURCES = ["api.hip", "timing.hip", "conv1d.hip", "gated_rmsnorm.hip", "scan_decode.hip", "snapshots.hip", "padded.hip", "linear.hip",
           "ssd_common.hip", "ssd_generic.hip", "ssd_mfma.hip", "mamba3.hip"]

FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", "-c", os.path.join(CSRC, src), "-o", obj] + FLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    noisy = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noisy:
        sys.stderr.write("\n".join(noisy) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link libmamba2.so (always recompiles)."""
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "-shared", "--offload-arch=" + ARCH, "-o", tmp] + objs
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
