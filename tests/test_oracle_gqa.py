"""Pins of the oracle's grouped-query (GQA) and multi-query (MQA) decode
attention over the compressed cache.

What is computed: the vTensor page on papercache.org, background section "GQA
and MQA optimisation": with MQA all query heads share one key head and one
value head; with GQA the query heads are divided into groups, each sharing one
key head and one value head.  The reading taken (the pages do not say which
heads form a group) is consecutive query heads: query head hq reads cache head
hq // R, R = q_heads / kv_heads.  The pins check the function against brute
force in 50-digit arithmetic, against the (separately pinned) multi-head oracle
on a cache whose heads are repeated R times, against torch's attention with
grouped heads on exactly representable inputs, and against special cases.
"""
import dataclasses
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch

import oracle
import synth


def _fill(B, Hkv, D, L, seed=0, cap_extra=3):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, L, Hkv * D)).astype(np.float16)
    v = rng.standard_normal((B, L, Hkv * D)).astype(np.float16)
    kv = oracle.KVCache(B, Hkv, D, L + cap_extra)
    oracle.kv_append(kv, k, v, 0)
    return kv


def _repeat_heads(kv, R):
    """The same cache with every K/V head stored R times in a row (an MHA cache)."""
    big = oracle.KVCache(kv.batch, kv.heads * R, kv.head_dim, kv.cap)
    for a in ("k_codes", "k_meta", "v_codes", "v_meta"):
        setattr(big, a, np.ascontiguousarray(np.repeat(getattr(kv, a), R, axis=1)))
    return big


def _recon(kv, which, L):
    codes = kv.k_codes if which == "k" else kv.v_codes
    meta = kv.k_meta if which == "k" else kv.v_meta
    B, H, _, _ = codes.shape
    D = kv.head_dim
    return oracle.dequant_g64(codes[:, :, :L].reshape(-1, D // 2),
                              meta[:, :, :L].reshape(-1, D // 64)).reshape(B, H, L, D)


@pytest.mark.parametrize("Hkv,R,D,L", [(2, 2, 64, 9), (3, 4, 128, 21), (1, 8, 128, 17), (2, 16, 64, 5)])
def test_equals_multi_head_oracle_on_repeated_heads(Hkv, R, D, L):
    """A cache whose heads are each repeated R times is an MHA cache with one
    head per query head; the grouped oracle over the small cache must equal the
    MHA oracle over the repeated one (same loops, so bit for bit).  Taking the
    group of a query head as hq % kv_heads instead of hq // R fails here."""
    B = 2
    kv = _fill(B, Hkv, D, L, seed=Hkv * 100 + R)
    q = np.random.default_rng(R).standard_normal((B, Hkv * R * D)).astype(np.float16)
    got = oracle.decode_attn_gqa(kv, q, Hkv * R, L)
    ref = oracle.decode_attn(_repeat_heads(kv, R), q, L)
    assert np.array_equal(got, ref)


def test_on_grid_cache_reduces_to_torch_grouped_attention():
    """K, V on the 16-level grid of their group reconstruct exactly, so the
    oracle must agree with torch's attention with grouped K/V heads
    (enable_gqa) on the original fp16 values."""
    B, Hkv, R, D, L = 2, 3, 4, 128, 33
    rng = np.random.default_rng(5)

    def grid(shape):
        k = rng.integers(0, 16, shape + (D // 64, 64))
        k[..., 0], k[..., 1] = 0, 15
        e = rng.integers(-6, 2, shape + (D // 64, 1))
        return ((k - 8) * 2.0 ** e).reshape(shape + (D,)).astype(np.float16)

    kh = grid((B, L, Hkv))
    vh = grid((B, L, Hkv))
    q = rng.standard_normal((B, Hkv * R * D)).astype(np.float16)
    kv = oracle.KVCache(B, Hkv, D, L)
    oracle.kv_append(kv, kh.reshape(B, L, Hkv * D), vh.reshape(B, L, Hkv * D), 0)
    got = oracle.decode_attn_gqa(kv, q, Hkv * R, L)
    Q = torch.from_numpy(q.astype(np.float64)).reshape(B, Hkv * R, 1, D)
    Kt = torch.from_numpy(kh.astype(np.float64)).permute(0, 2, 1, 3).contiguous()
    Vt = torch.from_numpy(vh.astype(np.float64)).permute(0, 2, 1, 3).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, enable_gqa=True)
    assert np.allclose(got, ref.reshape(B, Hkv * R * D).numpy(), rtol=2.0 ** -23, atol=1e-30)


def test_brute_force_50_digits():
    """Exact rational scores (D = 64, scale 1/8), exp to 50 digits, two K/V
    heads shared by three query heads each."""
    B, Hkv, R, D, L = 1, 2, 3, 64, 6
    kv = _fill(B, Hkv, D, L, seed=11)
    q = np.random.default_rng(12).standard_normal((B, Hkv * R * D)).astype(np.float16)
    got = oracle.decode_attn_gqa(kv, q, Hkv * R, L)
    K = _recon(kv, "k", L)
    V = _recon(kv, "v", L)
    mpmath.mp.dps = 50
    for hq in range(Hkv * R):
        kh = hq // R
        qv = [Fraction(float(x)) for x in q[0, hq * D:(hq + 1) * D]]
        s = [sum(qv[d] * Fraction(float(K[0, kh, j, d])) for d in range(D)) / 8 for j in range(L)]
        mx = max(s)
        e = [mpmath.exp(mpmath.mpf(x.numerator) / x.denominator - mpmath.mpf(mx.numerator) / mx.denominator)
             for x in s]
        den = sum(e)
        for d in range(D):
            ref = float(sum(e[j] * mpmath.mpf(float(V[0, kh, j, d])) for j in range(L)) / den)
            assert abs(float(got[0, hq * D + d]) - ref) <= 2.0 ** -23 * abs(ref) + 1e-30, (hq, d)


def test_mqa_equal_queries_give_equal_outputs_and_single_head_rows():
    """MQA (one K/V head): query heads with equal queries produce equal rows,
    and each row equals single-head attention of that query over the cache."""
    B, R, D, L = 2, 8, 128, 40
    kv = _fill(B, 1, D, L, seed=21)
    rng = np.random.default_rng(22)
    q = rng.standard_normal((B, R * D)).astype(np.float16)
    q[:, 3 * D:4 * D] = q[:, 0:D]
    got = oracle.decode_attn_gqa(kv, q, R, L).reshape(B, R, D)
    assert np.array_equal(got[:, 3], got[:, 0])
    for hq in range(R):
        one = oracle.decode_attn(kv, np.ascontiguousarray(q[:, hq * D:(hq + 1) * D]), L)
        assert np.array_equal(got[:, hq], one)


def test_group_ratio_one_is_multi_head_attention():
    B, H, D, L = 2, 3, 64, 12
    kv = _fill(B, H, D, L, seed=31)
    q = np.random.default_rng(32).standard_normal((B, H * D)).astype(np.float16)
    assert np.array_equal(oracle.decode_attn_gqa(kv, q, H, L), oracle.decode_attn(kv, q, L))


def test_grouped_heads_outlier_workload_against_float64_reference():
    """Heavy-tailed data with outlier channels and constant groups (the
    long-context recipe on a grouped cache): the oracle equals a numpy fp64
    softmax over its own reconstructions, an independent formulation."""
    w = dataclasses.replace(synth.WORKLOADS["long-t3"], heads=16, kv_heads=4)
    L = 40
    k = synth.prompt_kv(w, "k", nb=1, nt=L)
    v = synth.prompt_kv(w, "v", nb=1, nt=L)
    q = synth.step_q(w, 1)[:1]
    kv = oracle.KVCache(1, w.n_kv_heads, w.head_dim, L)
    oracle.kv_append(kv, k, v, 0)
    got = oracle.decode_attn_gqa(kv, q, w.heads, L).reshape(w.heads, w.head_dim)
    R = w.heads // w.n_kv_heads
    K = np.repeat(_recon(kv, "k", L)[0].astype(np.float64), R, axis=0)
    V = np.repeat(_recon(kv, "v", L)[0].astype(np.float64), R, axis=0)
    Q = q.astype(np.float64).reshape(w.heads, 1, w.head_dim)
    s = (Q @ K.transpose(0, 2, 1))[:, 0] / np.sqrt(w.head_dim)
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    ref = np.einsum("hj,hjd->hd", p, V)
    assert np.allclose(got, ref, rtol=1e-5, atol=1e-5 * np.abs(ref).max())


def test_rejects_heads_that_do_not_divide():
    kv = _fill(1, 3, 64, 4)
    q = np.zeros((1, 4 * 64), np.float16)
    with pytest.raises(oracle.OracleError):
        oracle.decode_attn_gqa(kv, q, 4, 4)
    q = np.zeros((1, 2 * 64), np.float16)
    with pytest.raises(oracle.OracleError):
        oracle.decode_attn_gqa(kv, q, 2, 4)     # fewer query heads than K/V heads
