"""Pins of the oracle's KV append and decode attention.

Decode attention over the compressed cache is, by definition, softmax attention
of one new query over every cached position, computed on the reconstructed K
and V (FlexGen review on blog.gzher.com, section 3.4: restore to FP16 before
compute; paper-graph-ui FlexGen summary, section 3.4 "Computation delegation":
decode attention reads the whole per-layer cache).  The pins below check the
oracle against brute force in 50-digit arithmetic, against torch's attention
on exactly representable inputs, and against closed-form special cases.
"""
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch

import oracle
import synth


def _fill(B, H, D, L, seed=0, scale=1.0):
    rng = np.random.default_rng(seed)
    k = (rng.standard_normal((B, L, H * D)) * scale).astype(np.float16)
    v = (rng.standard_normal((B, L, H * D)) * scale).astype(np.float16)
    q = rng.standard_normal((B, H * D)).astype(np.float16)
    kv = oracle.KVCache(B, H, D, L + 3)
    oracle.kv_append(kv, k, v, 0)
    return kv, q, k, v


def _recon(kv, which, L):
    codes = kv.k_codes if which == "k" else kv.v_codes
    meta = kv.k_meta if which == "k" else kv.v_meta
    B, H, cap, _ = codes.shape
    D = kv.head_dim
    c = codes[:, :, :L].reshape(-1, D // 2)
    m = meta[:, :, :L].reshape(-1, D // 64)
    return oracle.dequant_g64(c, m).reshape(B, H, L, D)


def test_append_layout_matches_row_quantisation():
    B, H, D, L = 2, 3, 128, 5
    kv, q, k, v = _fill(B, H, D, L, 1)
    for b in range(B):
        for h in range(H):
            rows = np.ascontiguousarray(k[b, :, h * D:(h + 1) * D])
            c, m = oracle.quantize_g64(rows)
            assert np.array_equal(kv.k_codes[b, h, :L], c)
            assert np.array_equal(kv.k_meta[b, h, :L], m)
            rows = np.ascontiguousarray(v[b, :, h * D:(h + 1) * D])
            c, m = oracle.quantize_g64(rows)
            assert np.array_equal(kv.v_codes[b, h, :L], c)
            assert np.array_equal(kv.v_meta[b, h, :L], m)
    assert np.all(kv.k_codes[:, :, L:] == 0) and np.all(kv.k_meta[:, :, L:] == 0)


def test_append_one_by_one_equals_bulk():
    B, H, D, L = 2, 2, 64, 9
    rng = np.random.default_rng(4)
    k = rng.standard_normal((B, L, H * D)).astype(np.float16)
    v = rng.standard_normal((B, L, H * D)).astype(np.float16)
    bulk = oracle.KVCache(B, H, D, L)
    oracle.kv_append(bulk, k, v, 0)
    one = oracle.KVCache(B, H, D, L)
    for t in range(L):
        oracle.kv_append(one, k[:, t:t + 1], v[:, t:t + 1], t)
    for a in ("k_codes", "k_meta", "v_codes", "v_meta"):
        assert np.array_equal(getattr(bulk, a), getattr(one, a))


def test_append_capacity_checked():
    kv = oracle.KVCache(1, 1, 64, 4)
    x = np.zeros((1, 2, 64), np.float16)
    with pytest.raises(oracle.OracleError):
        oracle.kv_append(kv, x, x, 3)


def test_brute_force_50_digits():
    """Every score is an exact rational (fp16 q times fp32 reconstructions, D=64
    so the 1/sqrt(D) scale is 1/8); exp is taken to 50 digits."""
    B, H, D, L = 2, 2, 64, 7
    kv, q, _, _ = _fill(B, H, D, L, 2)
    got = oracle.decode_attn(kv, q, L)
    K = _recon(kv, "k", L)
    V = _recon(kv, "v", L)
    mpmath.mp.dps = 50
    for b in range(B):
        for h in range(H):
            qv = [Fraction(float(x)) for x in q[b, h * D:(h + 1) * D]]
            s = []
            for j in range(L):
                acc = sum(qv[d] * Fraction(float(K[b, h, j, d])) for d in range(D))
                s.append(acc / 8)
            mx = max(s)
            e = [mpmath.exp(mpmath.mpf(x.numerator) / x.denominator - mpmath.mpf(mx.numerator) / mx.denominator)
                 for x in s]
            den = sum(e)
            for d in range(D):
                o = sum(e[j] * mpmath.mpf(float(V[b, h, j, d])) for j in range(L)) / den
                ref = float(o)
                assert abs(float(got[b, h * D + d]) - ref) <= 2.0 ** -23 * abs(ref) + 1e-30, (b, h, d)


def test_on_grid_cache_reduces_to_torch_attention():
    """K, V on the 16-level grid of their group reconstruct exactly, so the
    oracle must agree with torch's attention on the original fp16 values."""
    B, H, D, L = 2, 3, 128, 33
    rng = np.random.default_rng(5)

    def grid(shape):
        k = rng.integers(0, 16, shape + (D // 64, 64))
        k[..., 0], k[..., 1] = 0, 15
        e = rng.integers(-6, 2, shape + (D // 64, 1))
        return ((k - 8) * 2.0 ** e).reshape(shape + (D,)).astype(np.float16)

    kh = grid((B, L, H))
    vh = grid((B, L, H))
    q = rng.standard_normal((B, H * D)).astype(np.float16)
    kv = oracle.KVCache(B, H, D, L)
    oracle.kv_append(kv, kh.reshape(B, L, H * D), vh.reshape(B, L, H * D), 0)
    got = oracle.decode_attn(kv, q, L)
    Q = torch.from_numpy(q.astype(np.float64)).reshape(B, H, 1, D)
    Kt = torch.from_numpy(kh.astype(np.float64)).permute(0, 2, 1, 3).contiguous()
    Vt = torch.from_numpy(vh.astype(np.float64)).permute(0, 2, 1, 3).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt).reshape(B, H * D).numpy()
    assert np.allclose(got, ref, rtol=2.0 ** -23, atol=1e-30)


def test_single_position_returns_its_value_row():
    B, H, D, L = 2, 2, 128, 1
    kv, q, _, _ = _fill(B, H, D, L, 6)
    got = oracle.decode_attn(kv, q, 1)
    V = _recon(kv, "v", 1)
    assert np.array_equal(got.reshape(B, H, D), V[:, :, 0])


def test_zero_query_averages_values():
    B, H, D, L = 1, 2, 64, 13
    kv, q, _, _ = _fill(B, H, D, L, 7)
    q[:] = 0
    got = oracle.decode_attn(kv, q, L).reshape(B, H, D)
    V = _recon(kv, "v", L).astype(np.float64)
    assert np.allclose(got, V.mean(axis=2), rtol=1e-6, atol=1e-7)


def test_position_permutation_invariance():
    B, H, D, L = 1, 2, 128, 17
    kv, q, _, _ = _fill(B, H, D, L, 8)
    base = oracle.decode_attn(kv, q, L)
    perm = np.random.default_rng(0).permutation(L)
    kv2 = oracle.KVCache(B, H, D, kv.cap)
    for a in ("k_codes", "k_meta", "v_codes", "v_meta"):
        src = getattr(kv, a)
        dst = getattr(kv2, a)
        dst[:, :, :L] = src[:, :, perm]
    got = oracle.decode_attn(kv2, q, L)
    assert np.allclose(got, base, rtol=1e-6, atol=1e-7)


def test_kv_len_prefix_ignores_later_positions():
    B, H, D, L = 1, 1, 64, 10
    kv, q, _, _ = _fill(B, H, D, L, 9)
    a = oracle.decode_attn(kv, q, 6)
    kv.k_codes[:, :, 6:] ^= 0x5A
    kv.v_codes[:, :, 6:] ^= 0xA5
    b = oracle.decode_attn(kv, q, 6)
    assert np.array_equal(a, b)


def test_scale_argument():
    B, H, D, L = 1, 2, 64, 5
    kv, q, _, _ = _fill(B, H, D, L, 10)
    default = oracle.decode_attn(kv, q, L)
    explicit = oracle.decode_attn(kv, q, L, 1.0 / 8.0)
    assert np.array_equal(default, explicit)
    hot = oracle.decode_attn(kv, q, L, 1e-9)          # scores ~ 0 -> plain mean
    V = _recon(kv, "v", L).astype(np.float64)
    assert np.allclose(hot.reshape(B, H, D), V.mean(axis=2), rtol=1e-6, atol=1e-6)


def test_outlier_workload_attention_against_float64_reference():
    """On the long-context workload's heavy-tailed data (outlier channels and
    constant groups), the oracle equals a numpy fp64 softmax over its own
    reconstructions (a second, independent formulation of the definition)."""
    w = synth.WORKLOADS["long-t3"]
    L = 48
    k = synth.prompt_kv(w, "k", nb=1, nt=L)
    v = synth.prompt_kv(w, "v", nb=1, nt=L)
    q = synth.step_q(w, 1)[:1]
    kv = oracle.KVCache(1, w.heads, w.head_dim, L)
    oracle.kv_append(kv, k, v, 0)
    got = oracle.decode_attn(kv, q, L).reshape(w.heads, w.head_dim)
    K = _recon(kv, "k", L)[0].astype(np.float64)
    V = _recon(kv, "v", L)[0].astype(np.float64)
    Q = q.astype(np.float64).reshape(w.heads, 1, w.head_dim)
    s = (Q @ K.transpose(0, 2, 1))[:, 0] / np.sqrt(w.head_dim)
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    ref = np.einsum("hj,hjd->hd", p, V)
    assert np.allclose(got, ref, rtol=1e-5, atol=1e-5 * np.abs(ref).max())
