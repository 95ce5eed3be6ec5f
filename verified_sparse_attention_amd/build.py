"""Builds libvattn.so (the gfx950 HIP library behind include/vattn.h) in-tree."""
import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = [os.path.join(PKG, "csrc", f) for f in ("vattn_kernels.hip", "vattn_api.cpp")]
LIB = os.path.join(PKG, "libvattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",            # every fma in the pinned arithmetic is explicit
    "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
    "-I", os.path.join(PKG, "csrc"),
]


def source_hash() -> str:
    """Short digest of the kernel sources; hardware-counter summaries record it so a
    summary taken before a kernel change is recognised as stale."""
    h = hashlib.sha1()
    for f in ("vattn_kernels.hip", "vattn_device.hpp", "vattn_plan.hpp"):
        with open(os.path.join(PKG, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:12]


def build(verbose=False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-x", "hip"] + SRC + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
