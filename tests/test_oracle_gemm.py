"""Pins of the oracle's dequantise-then-multiply weight GEMM.

The block of m GPU batches of g rows each (paper-graph-ui FlexGen summary, section
3.4 "Compute Schedule": block size = GPU batch size x number of GPU batches,
and one load of a layer's weights serves the whole block; FlexGen review on
jaehun.me, "A block is the unit of weight reuse": B = g*m) multiplies one
weight matrix whose groups of 64 run along the output channel.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


def _weights(K, N, seed, sigma=0.02):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((K, N)) * sigma).astype(np.float16)


def test_on_grid_weights_equal_numpy_matmul():
    K, N, M = 192, 256, 12
    rng = np.random.default_rng(1)
    k = rng.integers(0, 16, (K, N // 64, 64))
    k[..., 0], k[..., 1] = 0, 15
    e = rng.integers(-12, -4, (K, N // 64, 1))
    W = ((k - 8) * 2.0 ** e).reshape(K, N).astype(np.float16)
    X = rng.standard_normal((M, K)).astype(np.float16)
    codes, meta = oracle.quantize_g64(W)
    Y = oracle.dequant_gemm(X, 4, 3, codes, meta)
    ref = X.astype(np.float64) @ W.astype(np.float64)
    assert np.allclose(Y, ref, rtol=2.0 ** -23, atol=1e-30)


def test_exact_tiny_gemm_rational():
    """The tiny workload's 4 x 128 x 512 product in exact rationals over the
    stored reconstructions, rounded once; the oracle's fp64 sum rounds to fp32
    within one ulp of it."""
    w = synth.WORKLOADS["tiny"]
    W = synth.weight(w, 0)
    X = synth.gemm_x(w, 0, 1)
    codes, meta = oracle.quantize_g64(W)
    What = oracle.dequant_g64(codes, meta)
    Y = oracle.dequant_gemm(X, w.g, w.m, codes, meta)
    # exact: all values are dyadic; scale to integers
    Xi = [[int(Fraction(float(v)) * 2 ** 24) for v in row] for row in X]
    Wi = (What.astype(np.float64) * 2.0 ** 40)
    assert np.all(Wi == np.round(Wi))    # reconstructions are multiples of 2^-40 here
    Wi = Wi.astype(object)
    for r in range(X.shape[0]):
        for n in range(0, W.shape[1], 7):
            exact = Fraction(sum(Xi[r][k] * int(Wi[k, n]) for k in range(W.shape[0])), 2 ** 64)
            got = Fraction(float(Y[r, n]))
            assert abs(got - exact) <= abs(exact) * Fraction(1, 2 ** 23) + Fraction(1, 2 ** 100), (r, n)


def test_block_identity_g_times_m():
    """Rows are independent: (g, m) equals the m GPU batches of g rows run one
    at a time, bit for bit."""
    K, N, g, m = 256, 320, 5, 4
    W = _weights(K, N, 2)
    rng = np.random.default_rng(3)
    X = rng.standard_normal((g * m, K)).astype(np.float16)
    codes, meta = oracle.quantize_g64(W)
    Y = oracle.dequant_gemm(X, g, m, codes, meta)
    parts = [oracle.dequant_gemm(X[j * g:(j + 1) * g], g, 1, codes, meta) for j in range(m)]
    assert np.array_equal(Y, np.concatenate(parts))


def test_row_permutation_and_linearity():
    K, N, M = 128, 192, 8
    W = _weights(K, N, 4)
    codes, meta = oracle.quantize_g64(W)
    rng = np.random.default_rng(5)
    X1 = rng.standard_normal((M, K)).astype(np.float16)
    perm = rng.permutation(M)
    Y = oracle.dequant_gemm(X1, M, 1, codes, meta)
    assert np.array_equal(oracle.dequant_gemm(X1[perm], M, 1, codes, meta), Y[perm])
    # linearity on inputs whose sum is exact in fp16 (halves of each other)
    Xa = (X1.astype(np.float32) * 0.5).astype(np.float16)
    Ya = oracle.dequant_gemm(Xa, M, 1, codes, meta)
    assert np.allclose(2.0 * Ya, Y, rtol=1e-6, atol=1e-7)


def test_weight_groups_run_along_output_channel():
    """Scaling one 64-column group of one input row changes only that group's
    reconstruction: the output columns outside it are untouched."""
    K, N, M = 64, 256, 4
    W = _weights(K, N, 6)
    X = np.random.default_rng(7).standard_normal((M, K)).astype(np.float16)
    c0, m0 = oracle.quantize_g64(W)
    W2 = W.copy()
    W2[10, 64:128] *= np.float16(3.0)
    c1, m1 = oracle.quantize_g64(W2)
    assert np.array_equal(np.delete(m1, 1, axis=1), np.delete(m0, 1, axis=1))
    Y0 = oracle.dequant_gemm(X, M, 1, c0, m0)
    Y1 = oracle.dequant_gemm(X, M, 1, c1, m1)
    cols = np.r_[0:64, 128:256]
    assert np.array_equal(Y0[:, cols], Y1[:, cols])
    assert not np.array_equal(Y0[:, 64:128], Y1[:, 64:128])


def test_identity_input_rows_read_back_the_weights():
    K, N = 128, 256
    W = _weights(K, N, 8)
    codes, meta = oracle.quantize_g64(W)
    X = np.eye(K, dtype=np.float16)[:16]
    Y = oracle.dequant_gemm(X, 16, 1, codes, meta)
    assert np.array_equal(Y, oracle.dequant_g64(codes, meta)[:16])


def test_empty_block():
    W = _weights(64, 64, 9)
    codes, meta = oracle.quantize_g64(W)
    Y = oracle.dequant_gemm(np.zeros((0, 64), np.float16), 0, 4, codes, meta)
    assert Y.shape == (0, 64)
