"""Build libfgq.so (gfx950) in place with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libfgq.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-fp32 instructions anywhere in the library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division / sqrt (the quantiser's codes depend on it)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc] + HIPCC_FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")] + \
        sources() + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
