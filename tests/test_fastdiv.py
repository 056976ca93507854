"""Host-side check of the invariant-divisor division the kernels use to
decode positions (multiply-high + shifts, Granlund and Montgomery, PLDI 1994,
section 4): the same header compiled by the host compiler, against exact
division on edge divisors (1, powers of two and their neighbours, 2^31 + 1,
2^32 - 1), numerators around multiples of the divisor, and random pairs."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "int4_group_quantized_fgq_amd", "csrc")

SRC = r'''
#include "fastdiv.h"
#include <cstdio>
#include <random>
int main() {
    std::mt19937_64 rng(1);
    unsigned long long bad = 0, checks = 0;
    const uint32_t ds[] = {1u, 2u, 3u, 5u, 7u, 24u, 48u, 96u, 127u, 128u, 129u, 512u, 513u, 544u, 1000u, 4096u,
                           16416u, 65535u, 65536u, 65537u, 1000003u, 0x7fffffffu, 0x80000000u, 0x80000001u,
                           0xfffffffeu, 0xffffffffu};
    for (uint32_t d : ds) {
        const fgq::FastDiv f = fgq::make_fastdiv(d);
        for (int i = 0; i < 200000; ++i) {
            const uint32_t n = i < 1000 ? (uint32_t)i : (i < 2000 ? 0xffffffffu - (uint32_t)(i - 1000) : (uint32_t)rng());
            ++checks; bad += fgq::fastdiv(n, f) != n / d;
        }
        for (uint64_t k = 0; k < 4096; ++k)
            for (int e = -1; e <= 1; ++e) {
                const uint64_t v = k * d + e;
                if (v > 0xffffffffull) continue;
                ++checks; bad += fgq::fastdiv((uint32_t)v, f) != (uint32_t)v / d;
            }
    }
    for (int i = 0; i < 1000000; ++i) {
        uint32_t d = (uint32_t)rng() >> (rng() % 32);
        if (!d) d = 1;
        const uint32_t n = (uint32_t)rng();
        ++checks; bad += fgq::fastdiv(n, fgq::make_fastdiv(d)) != n / d;
    }
    std::printf("%llu %llu\n", checks, bad);
    return bad != 0;
}
'''


def test_fastdiv_matches_exact_division(tmp_path):
    src = tmp_path / "t.cpp"
    src.write_text(SRC)
    exe = tmp_path / "t"
    try:
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-I", CSRC, str(src), "-o", str(exe)])
    except (OSError, subprocess.CalledProcessError):
        pytest.skip("no host C++ compiler")
    out = subprocess.run([str(exe)], stdout=subprocess.PIPE, text=True)
    checks, bad = map(int, out.stdout.split())
    assert out.returncode == 0 and bad == 0 and checks > 5_000_000
