"""GPU parity of fgq_dequant_gemm, the block GEMM straight from the
quantiser's codes [K][N/2] and metadata [K][N/64], against the CPU oracle.

Bar: the GPU's codes and metadata are first asserted equal to the oracle's;
then max|gpu - oracle| <= 1e-2 and ||gpu - oracle||_2 / ||oracle||_2 <= 1e-3
against the oracle's fp64 product of the fp32 reconstruction of the same
codes.  Shapes cover the workloads' weight matrices (whole, or sampled
whole-group column slices where the oracle would take minutes), ragged row
counts and partial last column tiles, split-K plans with both k-phase
settings, and fp16 output.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

try:
    import torch
    _HAS_GPU = torch.cuda.is_available()
except ImportError:   # pragma: no cover
    _HAS_GPU = False

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not _HAS_GPU, reason="needs an MI355X GPU")]

W = synth.WORKLOADS


def _quantized(Wt):
    """GPU quantisation of W (device codes/meta), checked bit-exact against the oracle."""
    torch = gu.torch_cuda()
    K, N = Wt.shape
    wd = gu.to_dev(Wt)
    codes = torch.empty((K, N // 2), dtype=torch.uint8, device="cuda")
    meta = torch.empty((K, N // 64), dtype=torch.int32, device="cuda")
    gu.fgq.fgq_quantize_g64(wd, K, N, N, codes, meta)
    torch.cuda.synchronize()
    del wd
    return codes, meta


@pytest.mark.parametrize("M,K,N", [(1, 64, 64), (5, 128, 320), (16, 64, 256), (17, 192, 64), (37, 256, 512),
                                   (144, 128, 192), (145, 192, 128), (300, 64, 64), (33, 576, 320),
                                   (145, 4160, 1088), (150, 8256, 576), (64, 4096, 4160)])
def test_canonical_gemm_ragged_shapes(M, K, N):
    rng = np.random.default_rng(M * 13 + K + N)
    Wt = (rng.standard_normal((K, N)) * 0.02).astype(np.float16)
    X = rng.standard_normal((M, K)).astype(np.float16)
    gu.note("canonical gemm M=%d K=%d N=%d" % (M, K, N))
    codes, meta = _quantized(Wt)
    rc, rm = oracle.quantize_g64(Wt)
    assert np.array_equal(gu.to_host(codes), rc) and np.array_equal(gu.to_host(meta, np.uint32), rm)
    y = gu.gemm_canonical(X, M, 1, codes, meta, K, N)
    gu.assert_close(y, oracle.dequant_gemm(X, M, 1, rc, rm), "canonical gemm %dx%dx%d" % (M, K, N))


@pytest.mark.parametrize("M", [8, 40, 72, 104, 136])
def test_canonical_gemm_row_tile_counts(M):
    """Row-tile counts 1, 3, 5, 7 and 9 with several ring turns, a split plan
    and a ragged last column block: two-phase workgroups of up to 8 m-tiles
    take slots of two chunks per wave, 9 m-tiles one."""
    K, N = 8192, 640
    rng = np.random.default_rng(M + 23)
    Wt = (rng.standard_normal((K, N)) * 0.02).astype(np.float16)
    X = rng.standard_normal((M, K)).astype(np.float16)
    gu.note("canonical gemm row tiles M=%d" % M)
    codes, meta = _quantized(Wt)
    rc, rm = oracle.quantize_g64(Wt)
    y = gu.gemm_canonical(X, M, 1, codes, meta, K, N)
    gu.assert_close(y, oracle.dequant_gemm(X, M, 1, rc, rm), "canonical gemm %dx%dx%d" % (M, K, N))


def test_canonical_gemm_empty_k_is_zero():
    torch = gu.torch_cuda()
    M, N = 4, 64
    dummy = torch.empty(16, dtype=torch.int32, device="cuda")
    X = np.zeros((M, 0), np.float16)
    gu.note("canonical gemm K=0")
    y = gu.gemm_canonical(X, M, 1, dummy, dummy, 0, N, xd=dummy)
    assert np.all(y == 0)


@pytest.mark.parametrize("name,idx", [("tiny", 0), ("opt-6.7b", 0), ("opt-6.7b", 4), ("opt-6.7b", 5),
                                      ("opt-30b", 0)])
def test_canonical_gemm_workload_full(name, idx):
    w = W[name]
    K, N = w.weights[idx]
    gu.note("canonical gemm %s[%d] M=%d K=%d N=%d" % (name, idx, w.batch, K, N))
    Wt = synth.weight(w, idx)
    X = synth.gemm_x(w, idx, 1)
    codes, meta = _quantized(Wt)
    rc, rm = oracle.quantize_g64(Wt)
    assert np.array_equal(gu.to_host(codes), rc) and np.array_equal(gu.to_host(meta, np.uint32), rm)
    y = gu.gemm_canonical(X, w.g, w.m, codes, meta, K, N)
    gu.assert_close(y, oracle.dequant_gemm(X, w.g, w.m, rc, rm), "canonical gemm %s[%d]" % (name, idx))


@pytest.mark.parametrize("name,idx", [("opt-30b", 4), ("opt-30b", 5), ("opt-175b", 0), ("opt-175b", 4),
                                      ("opt-175b", 5)])
def test_canonical_gemm_sampled_columns(name, idx):
    """Full-size weights with the workload's block (M = g*m rows); the oracle
    quantises and multiplies three whole-group 256-column slices on its own
    (groups run along N, so a slice of whole groups has the same codes)."""
    w = W[name]
    K, N = w.weights[idx]
    gu.note("canonical gemm %s[%d] M=%d K=%d N=%d (sampled columns)" % (name, idx, w.batch, K, N))
    Wt = synth.weight(w, idx)
    X = synth.gemm_x(w, idx, 1)
    codes, meta = _quantized(Wt)
    hc, hm = gu.to_host(codes), gu.to_host(meta, np.uint32)
    y = gu.gemm_canonical(X, w.g, w.m, codes, meta, K, N)
    del codes, meta
    for n0 in (0, N // 2 + 64, N - 256):
        rc, rm = oracle.quantize_g64(np.ascontiguousarray(Wt[:, n0:n0 + 256]))
        assert np.array_equal(hc[:, n0 // 2:(n0 + 256) // 2], rc), n0
        assert np.array_equal(hm[:, n0 // 64:(n0 + 256) // 64], rm), n0
        gu.assert_close(y[:, n0:n0 + 256], oracle.dequant_gemm(X, w.g, w.m, rc, rm),
                        "canonical %s[%d] cols %d.." % (name, idx, n0))


def test_canonical_and_packed_layouts_agree():
    """The same weight through both entry points (one read of the canonical
    codes, one of the offline packed layout), against each other and the
    oracle; bitwise repeatable."""
    w = W["opt-6.7b"]
    K, N = w.weights[5]
    Wt = synth.weight(w, 5)
    X = synth.gemm_x(w, 5, 3)
    gu.note("canonical vs packed 16384x4096, M=64")
    codes, meta = _quantized(Wt)
    pc, pm = gu.pack(codes, meta, K, N)
    yc = gu.gemm_canonical(X, w.g, w.m, codes, meta, K, N)
    yc2 = gu.gemm_canonical(X, w.g, w.m, codes, meta, K, N)
    assert np.array_equal(yc, yc2)
    yp = gu.gemm(X, w.g, w.m, pc, pm, K, N)
    rc, rm = oracle.quantize_g64(Wt)
    exp = oracle.dequant_gemm(X, w.g, w.m, rc, rm)
    gu.assert_close(yc, exp, "canonical vs oracle")
    gu.assert_close(yp, exp, "packed vs oracle")
    gu.assert_close(yc, yp, "canonical vs packed")


def test_canonical_gemm_wide_ranging_groups_and_fp16_output():
    """Column groups whose steps span fp16 from tiny to near-overflow (the
    canonical path restores fp16(min + q*step) directly, with no per-group
    exponent); constant groups (step 0).  Each column group is compared on its
    own scale: the restored weights reach 65000, so the products do too."""
    rng = np.random.default_rng(41)
    K, N, g, m = 256, 384, 8, 2
    Wt = (rng.standard_normal((K, N)) * 0.02).astype(np.float16)
    Wt[:, 64:128] *= np.float16(400.0)
    Wt[:, 128:192] = (rng.standard_normal((K, 64)) * 20000).clip(-65000, 65000).astype(np.float16)
    Wt[:, 192:256] *= np.float16(1e-3)
    Wt[:, 256:320] = np.float16(0.75)
    X = (rng.standard_normal((g * m, K)) * 0.01).astype(np.float16)
    gu.note("canonical gemm wide-ranging groups")
    codes, meta = _quantized(Wt)
    rc, rm = oracle.quantize_g64(Wt)
    assert np.array_equal(gu.to_host(codes), rc) and np.array_equal(gu.to_host(meta, np.uint32), rm)
    y = gu.gemm_canonical(X, g, m, codes, meta, K, N)
    exp = oracle.dequant_gemm(X, g, m, rc, rm)
    for c in range(N // 64):
        sl = slice(64 * c, 64 * c + 64)
        s = max(1.0, float(np.abs(exp[:, sl]).max()))
        gu.assert_close(y[:, sl] / s, exp[:, sl] / s, "group %d (scaled by %.3g)" % (c, s))
    # fp16 output of an N(0,1) x N(0, 0.02) product (|Y| < 8: rounding within 2^-9)
    w = W["opt-6.7b"]
    K2, N2 = w.weights[0]
    Wt2 = synth.weight(w, 0)
    X2 = synth.gemm_x(w, 0, 2)
    codes2, meta2 = _quantized(Wt2)
    rc2, rm2 = oracle.quantize_g64(Wt2)
    y16 = gu.gemm_canonical(X2, w.g, w.m, codes2, meta2, K2, N2, y_f16=True)
    gu.assert_close(y16, oracle.dequant_gemm(X2, w.g, w.m, rc2, rm2), "canonical gemm fp16 out")
