"""GPU parity of grouped-query (GQA) and multi-query (MQA) decode attention
over the compressed cache, against the CPU oracle on the same codes.

The cache is written by the GPU's own append, and its bytes are checked equal
to the oracle's before attention is compared (max |gpu - oracle| <= 1e-2 and
relative L2 <= 1e-3 on fp32 outputs).  Cases span group ratios 2..32 (one and
two 16-head column tiles, ratios that leave padding columns), head_dim 64 and
128, lengths with ragged ends inside a 32-token block and across the four
waves of a workgroup, split plans with several partial states, the
heavy-tailed long-context recipe, and sampled sequences of the full grouped
workload (16 sequences x 16K positions, 32 query heads over 8 or 1 K/V heads).
"""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

try:
    import torch
    _HAS_GPU = torch.cuda.is_available()
except Exception:  # pragma: no cover
    _HAS_GPU = False

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not _HAS_GPU, reason="needs an MI355X GPU")]

W = synth.WORKLOADS


def _shape(base, B, Hkv, R, D, L):
    return dataclasses.replace(base, g=B, m=1, heads=Hkv * R, kv_heads=Hkv, head_dim=D, prompt=L, steps=1)


def _case(w):
    """Prompt bulk append on the GPU and in the oracle; the cache bytes must agree."""
    B, Hkv, D, cap = w.batch, w.n_kv_heads, w.head_dim, w.capacity
    dev = gu.DevKV(B, Hkv, D, cap)
    ref = oracle.KVCache(B, Hkv, D, cap)
    pk, pv = synth.prompt_kv(w, "k"), synth.prompt_kv(w, "v")
    dev.append(pk, pv, 0)
    oracle.kv_append(ref, pk, pv, 0)
    h = dev.host()
    for a in ("k_codes", "k_meta", "v_codes", "v_meta"):
        assert np.array_equal(h[a], getattr(ref, a)), a
    return dev, ref


def _check(dev, ref, w, L, what, out_f16=False, scale=0.0, t=1):
    q = synth.step_q(w, t)
    gu.note("gqa %s Hq=%d Hkv=%d D=%d L=%d" % (what, w.heads, w.n_kv_heads, w.head_dim, L))
    got = dev.attend_gqa(q, w.heads, L, scale, out_f16)
    exp = oracle.decode_attn_gqa(ref, q, w.heads, L, scale)
    gu.assert_close(got, exp, "%s L=%d" % (what, L))


@pytest.mark.parametrize("Hkv,R,D", [(2, 2, 64), (2, 4, 128), (1, 8, 128), (4, 16, 128), (1, 32, 128),
                                     (2, 3, 64), (1, 17, 128), (3, 32, 64), (2, 5, 128)])
def test_gqa_ratios_and_ragged_lengths(Hkv, R, D):
    w = _shape(W["gqa"], 2, Hkv, R, D, 300)
    dev, ref = _case(w)
    for L in (1, 2, 31, 32, 33, 127, 128, 129, 300):
        _check(dev, ref, w, L, "R=%d" % R)


@pytest.mark.parametrize("B,Hkv,R,L", [(1, 1, 8, 2000), (1, 2, 4, 4100), (2, 1, 32, 3000)])
def test_gqa_split_plans(B, Hkv, R, L):
    """Few (sequence, K/V head) pairs over long contexts: several splits merged."""
    assert gu.fgq.fgq_decode_attn_gqa_ws_bytes(B, Hkv * R, Hkv, 128, L) > 0
    w = _shape(W["gqa"], B, Hkv, R, 128, L)
    dev, ref = _case(w)
    for Lq in (L, L - 77, 513):
        _check(dev, ref, w, Lq, "split")


@pytest.mark.parametrize("B,Hkv,R,D,L,Ls", [
    (2, 1, 16, 64, 600, (1, 33, 255, 256, 257, 600)),   # ragged splits; waves 1..3 empty at L = 1
    (2, 2, 12, 128, 300, (31, 224, 256, 300)),          # padding columns (12 of 16 heads)
    (1, 1, 16, 128, 3000, (3000, 2923, 513)),           # several splits
    (1, 3, 10, 64, 5000, (5000, 4097)),                 # head_dim 64, padding columns
])
def test_gqa_wide_groups_few_pairs(B, Hkv, R, D, L, Ls):
    """9..16 query heads per K/V head with few pairs: one workgroup per
    (sequence, K/V head, split), lengths that leave some of its waves without
    a block, padding columns, head_dim 64, several splits; bitwise repeatable."""
    w = _shape(W["gqa"], B, Hkv, R, D, L)
    if L >= 3000:
        assert gu.fgq.fgq_decode_attn_gqa_ws_bytes(B, Hkv * R, Hkv, D, L) > 0
    dev, ref = _case(w)
    for Lq in Ls:
        _check(dev, ref, w, Lq, "wide group R=%d" % R)
    q = synth.step_q(w, 1)
    assert np.array_equal(dev.attend_gqa(q, w.heads, L), dev.attend_gqa(q, w.heads, L))


def test_gqa_long_context_outliers_and_constant_groups():
    w = dataclasses.replace(W["long-t3"], g=2, heads=96, kv_heads=12, prompt=4096, steps=1)
    dev, ref = _case(w)
    _check(dev, ref, w, 4096, "long-t3 R=8")
    _check(dev, ref, w, 1000, "long-t3 R=8")


def test_gqa_fp16_output_and_scale():
    w = _shape(W["gqa"], 2, 2, 8, 128, 700)
    dev, ref = _case(w)
    _check(dev, ref, w, 700, "fp16 out", out_f16=True)
    _check(dev, ref, w, 650, "scale 0.05", scale=0.05)


def test_gqa_ratio_one_is_the_multi_head_call():
    w = _shape(W["gqa"], 3, 4, 1, 128, 200)
    dev, ref = _case(w)
    q = synth.step_q(w, 1)
    a = dev.attend_gqa(q, w.heads, 200)
    b = dev.attend(q, 200)
    assert np.array_equal(a, b)
    gu.assert_close(a, oracle.decode_attn_gqa(ref, q, w.heads, 200), "R=1")


def test_gqa_repeatable_bitwise():
    w = _shape(W["gqa"], 1, 2, 8, 128, 3000)
    dev, _ = _case(w)
    q = synth.step_q(w, 1)
    a = dev.attend_gqa(q, w.heads, 3000)
    b = dev.attend_gqa(q, w.heads, 3000)
    assert np.array_equal(a, b)


def _full_size(w, t, samples):
    """The workload at full size: prompt bulk-appended in chunks of sequences,
    t decode-step appends, attention at kv_len = prompt + t; sampled sequences
    checked against the oracle (codes first, then the output rows)."""
    B, Hkv, D, cap = w.batch, w.n_kv_heads, w.head_dim, w.capacity
    gu.note("full-size gqa %s B=%d Hq=%d Hkv=%d L=%d" % (w.name, B, w.heads, Hkv, w.kv_len(t)))
    dev = gu.DevKV(B, Hkv, D, cap)
    chunk = 4
    for b0 in range(0, B, chunk):
        nb = min(chunk, B - b0)
        sub = gu.fgq.kv_struct(dev.k_codes[b0:b0 + nb], dev.v_codes[b0:b0 + nb], dev.k_meta[b0:b0 + nb],
                               dev.v_meta[b0:b0 + nb], nb, Hkv, D, cap)
        kd = gu.to_dev(synth.prompt_kv(w, "k", b0=b0, nb=nb))
        vd = gu.to_dev(synth.prompt_kv(w, "v", b0=b0, nb=nb))
        gu.fgq.fgq_kv_append(sub, kd, vd, 0, w.prompt)
        del kd, vd
    for s in range(1, t + 1):
        dev.append(synth.step_kv(w, "k", s), synth.step_kv(w, "v", s), w.prompt + s - 1)
    q = synth.step_q(w, t)
    got = dev.attend_gqa(q, w.heads, w.kv_len(t))
    for b in samples:
        ref = oracle.KVCache(1, Hkv, D, cap)
        oracle.kv_append(ref, synth.prompt_kv(w, "k", b0=b, nb=1), synth.prompt_kv(w, "v", b0=b, nb=1), 0)
        for s in range(1, t + 1):
            oracle.kv_append(ref, synth.step_kv(w, "k", s)[b:b + 1], synth.step_kv(w, "v", s)[b:b + 1],
                             w.prompt + s - 1)
        for a in ("k_codes", "k_meta", "v_codes", "v_meta"):
            assert np.array_equal(gu.to_host(getattr(dev, a)[b], np.uint32 if "meta" in a else None),
                                  getattr(ref, a)[0]), (a, b)
        exp = oracle.decode_attn_gqa(ref, q[b:b + 1], w.heads, w.kv_len(t))
        gu.assert_close(got[b:b + 1], exp, "%s full-size seq %d" % (w.name, b))


@pytest.mark.parametrize("kv_heads,t,samples", [(8, 2, (0, 15)), (2, 3, (7,)), (1, 1, (5,))])
def test_gqa_workload_full_size_sampled(kv_heads, t, samples):
    _full_size(dataclasses.replace(W["gqa"], kv_heads=kv_heads), t, samples)


@pytest.mark.parametrize("B,Hkv,R,D,L", [(64, 32, 2, 128, 300), (64, 32, 4, 64, 257)])
def test_gqa_one_wave_per_item_plan(B, Hkv, R, D, L):
    """At least 2048 (sequence, K/V head) pairs: one wave per pair, no split."""
    assert gu.fgq.fgq_decode_attn_gqa_ws_bytes(B, Hkv * R, Hkv, D, L) == 0
    w = _shape(W["gqa"], B, Hkv, R, D, L)
    dev, ref = _case(w)
    for Lq in (L, L - 1, 33):
        _check(dev, ref, w, Lq, "one wave per pair")
