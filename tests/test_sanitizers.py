"""AddressSanitizer + UndefinedBehaviorSanitizer runs of the host code (no GPU):

* the CPU oracle (oracle/oracle.c, built with gcc) driven by
  tests/sanitize/oracle_checks.c: small ragged shapes in exactly-sized heap
  buffers, the edge cases and the rejected arguments;
* libfgq's host side (argument validation and size queries; the kernels are
  compiled as usual, only the host code is instrumented) driven by
  tests/sanitize/abi_checks.c: every entry point with arguments it must
  reject before any HIP call, and the size queries over extreme values.

Any sanitizer report aborts the driver (-fno-sanitize-recover=all), and the
drivers also check every returned status.
"""
import concurrent.futures
import os
import subprocess

import pytest

from int4_group_quantized_fgq_amd import build as hip_build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN_DIR = os.path.join(HERE, "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
# host-only instrumentation on every hipcc line
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all".split()
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")


def _run(cmd, timeout, env=None):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=timeout, env=env)
    return res.returncode, res.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    rc, out = _run(["gcc", "-std=c99", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-ffp-contract=off", "-fopenmp", os.path.join(ROOT, "oracle", "oracle.c"),
                    os.path.join(SAN_DIR, "oracle_checks.c"), "-lm", "-o", exe], 120)
    assert rc == 0, out
    rc, out = _run([exe], 300, SAN_ENV)
    assert rc == 0 and "oracle checks ok" in out, out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs hipcc and clang")
def test_library_host_validation_under_asan_ubsan(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(hip_build.HERE, "csrc")]
    flags = [f for f in hip_build.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"] + HOST_SAN
    jobs = []
    for src in hip_build.sources():
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        jobs.append(([HIPCC] + flags + hip_build.EXTRA_FLAGS.get(os.path.basename(src), []) + inc +
                     ["-c", src, "-o", obj], obj))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        results = list(ex.map(lambda j: _run(j[0], 600), jobs))
    for (rc, out), (cmd, _) in zip(results, jobs):
        assert rc == 0, " ".join(cmd) + "\n" + out
    lib = str(tmp_path / "libfgq_san.so")
    rc, out = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + HOST_SAN[:4] + [o for _, o in jobs] +
                   ["-o", lib], 300)
    assert rc == 0, out
    exe = str(tmp_path / "abi_checks")
    rc, out = _run([CLANG, "-std=c99", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "include"), os.path.join(SAN_DIR, "abi_checks.c"), lib,
                    "-Wl,-rpath," + str(tmp_path), "-o", exe], 120)
    assert rc == 0, out
    rc, out = _run([exe], 300, SAN_ENV)
    assert rc == 0 and "abi checks ok" in out, out
