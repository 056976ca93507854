"""Pins of the oracle's prefill attention (causal attention of the prompt
over its own fp16 K and V, before compression; paper-graph-ui FlexGen
summary, section 3.4, token 0 of the computation grid is the prefill step;
FlexGen review on blog.gzher.com, section 1).  Checked against torch's
causal attention, 50-digit brute force, the decode-attention oracle (pinned
on its own) over a losslessly compressed cache, and closed-form cases.
"""
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch

import oracle


def _qkv(B, s, H, D, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, s, H * D)).astype(np.float16) for _ in range(3)]


def test_reduces_to_torch_causal_attention():
    B, s, H, D = 2, 37, 3, 64
    q, k, v = _qkv(B, s, H, D, 1)
    got = oracle.prefill_attn(q, k, v, H)

    def t(x):   # [B][s][H*D] -> [B][H][s][D], fp64
        return torch.from_numpy(x.astype(np.float64)).reshape(B, s, H, D).permute(0, 2, 1, 3).contiguous()

    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True)
    ref = ref.permute(0, 2, 1, 3).reshape(B, s, H * D).numpy()
    assert np.allclose(got, ref, rtol=2.0 ** -22, atol=1e-30)


def test_brute_force_50_digits():
    B, s, H, D = 1, 6, 2, 64
    q, k, v = _qkv(B, s, H, D, 2)
    got = oracle.prefill_attn(q, k, v, H)
    mpmath.mp.dps = 50
    for h in range(H):
        sl = slice(h * D, (h + 1) * D)
        for i in range(s):
            sc = [sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(q[0, i, sl], k[0, j, sl])) / 8
                  for j in range(i + 1)]
            mx = max(sc)
            e = [mpmath.exp(mpmath.mpf(x.numerator) / x.denominator - mpmath.mpf(mx.numerator) / mx.denominator)
                 for x in sc]
            den = sum(e)
            for d in range(D):
                ref = float(sum(e[j] * mpmath.mpf(float(v[0, j, h * D + d])) for j in range(i + 1)) / den)
                assert abs(float(got[0, i, h * D + d]) - ref) <= 2.0 ** -23 * abs(ref) + 1e-30, (h, i, d)


def test_row_i_is_decode_attention_over_positions_up_to_i():
    """With K and V on their groups' 16-level grid the compressed cache is
    lossless, so row i of prefill equals the decode-attention oracle of query
    i over cache positions 0..i."""
    B, s, H, D = 2, 20, 2, 128
    rng = np.random.default_rng(3)

    def grid():
        c = rng.integers(0, 16, (B, s, H, D // 64, 64))
        c[..., 0], c[..., 1] = 0, 15
        e = rng.integers(-5, 1, (B, s, H, D // 64, 1))
        return ((c - 8) * 2.0 ** e).reshape(B, s, H * D).astype(np.float16)

    k, v = grid(), grid()
    q = rng.standard_normal((B, s, H * D)).astype(np.float16)
    got = oracle.prefill_attn(q, k, v, H)
    kv = oracle.KVCache(B, H, D, s)
    oracle.kv_append(kv, k, v, 0)
    for i in (0, 1, 7, s - 1):
        dec = oracle.decode_attn(kv, np.ascontiguousarray(q[:, i]), i + 1)
        assert np.allclose(got[:, i], dec, rtol=1e-6, atol=1e-7), i


def test_first_row_is_the_first_value_row_and_causality():
    B, s, H, D = 1, 9, 2, 64
    q, k, v = _qkv(B, s, H, D, 4)
    got = oracle.prefill_attn(q, k, v, H)
    assert np.array_equal(got[:, 0], v[:, 0].astype(np.float32))
    k2, v2 = k.copy(), v.copy()
    k2[:, 5:] = np.float16(3.0)
    v2[:, 5:] = np.float16(-7.0)
    got2 = oracle.prefill_attn(q, k2, v2, H)
    assert np.array_equal(got[:, :5], got2[:, :5])
    assert not np.allclose(got[:, 5:], got2[:, 5:])


def test_row_range_and_scale():
    B, s, H, D = 1, 12, 2, 64
    q, k, v = _qkv(B, s, H, D, 5)
    full = oracle.prefill_attn(q, k, v, H)
    part = oracle.prefill_attn(q, k, v, H, rows=(4, 9))
    assert np.array_equal(part[:, 4:9], full[:, 4:9])
    assert np.all(np.isnan(part[:, :4])) and np.all(np.isnan(part[:, 9:]))
    assert np.array_equal(oracle.prefill_attn(q, k, v, H, scale=1.0 / 8.0), full)
    cold = oracle.prefill_attn(q, k, v, H, scale=1e-12)      # every score ~ 0: the running mean of v
    ref = np.cumsum(v.astype(np.float64), axis=1) / np.arange(1, s + 1)[None, :, None]
    assert np.allclose(cold, ref, rtol=1e-6, atol=1e-6)


def test_rejects_bad_row_range():
    q, k, v = _qkv(1, 4, 1, 64, 6)
    with pytest.raises(oracle.OracleError):
        oracle.prefill_attn(q, k, v, 1, rows=(2, 5))
