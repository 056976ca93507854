"""Build libfgq.so (gfx950) in place with hipcc: every source is compiled to
an object of its own (in parallel, with its own extra flags), then linked."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libfgq.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-fp32 instructions anywhere in the library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division / sqrt (the quantiser's codes depend on it)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall",
]


# Extra flags per source file.  The grouped-query attention keeps its matrix
# core accumulators in ordinary VGPRs (its softmax reads and rescales them
# every block; in AGPRs each access costs a copy).
EXTRA_FLAGS = {
    "gqa_attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + out)
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    tmpdir = tempfile.mkdtemp(prefix="fgq_build_")
    try:
        jobs = []
        for src in sources():
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd = [hipcc] + HIPCC_FLAGS + EXTRA_FLAGS.get(os.path.basename(src), []) + inc + ["-c", src, "-o", obj]
            jobs.append((cmd, obj))
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
            list(ex.map(lambda j: _run(j[0], verbose), jobs))
        tmp = LIB + ".tmp%d" % os.getpid()
        _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + [o for _, o in jobs] + ["-o", tmp], verbose)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
