"""GPU parity of top-K sparse decode attention (through the C ABI) against
the oracle on the same seeded inputs and the same codes.

The kept set is an integer decision taken on floating-point scores: the GPU
ranks its fp32 scores, the oracle its fp64 scores rounded once to fp32.
Where the two selections agree (all but near-ties at the cut) the outputs
are held to the attention bar (max-abs 1e-2, rel-L2 1e-3).  Where they differ,
the GPU's selection must still be a valid one - every kept score at least
every dropped score, to within a bound on the GPU's fp32 score error - and its
output may differ from the oracle's only by the weight of the swapped
positions.  Exact ties (bit-identical K rows) are decided identically on both
sides, so with well-separated distinct rows the selections must be equal.
"""
import math

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
# bound on |GPU fp32 score - exact score| as a fraction of scale * max_j sum_d |q_d K^_{j,d}|
SCORE_ERR = 2.0 ** -16


def _kv_case(w, nb, steps):
    cap = w.prompt + steps
    dev = gu.DevKV(nb, w.heads, w.head_dim, cap)
    ref = oracle.KVCache(nb, w.heads, w.head_dim, cap)
    pk = synth.prompt_kv(w, "k", nb=nb)
    pv = synth.prompt_kv(w, "v", nb=nb)
    dev.append(pk, pv, 0)
    oracle.kv_append(ref, pk, pv, 0)
    for t in range(1, steps + 1):
        sk = synth.step_kv(w, "k", t)[:nb]
        sv = synth.step_kv(w, "v", t)[:nb]
        dev.append(sk, sv, w.prompt + t - 1)
        oracle.kv_append(ref, sk, sv, w.prompt + t - 1)
    return dev, ref


def _recon(ref, which, L):
    codes = ref.k_codes if which == "k" else ref.v_codes
    meta = ref.k_meta if which == "k" else ref.v_meta
    B, H = codes.shape[:2]
    D = ref.head_dim
    return oracle.dequant_g64(codes[:, :, :L].reshape(-1, D // 2),
                              meta[:, :, :L].reshape(-1, D // 64)).reshape(B, H, L, D).astype(np.float64)


def _topk_check(dev, ref, q, L, k, what, scale=0.0, out_f16=False, max_swapped_frac=0.01):
    gu.note("top-k attention %s kv_len %d top_k %d" % (what, L, k))
    B, H, D = ref.batch, ref.heads, ref.head_dim
    kk = min(k, L)
    got, gsel = dev.attend_topk(q, L, k, scale, out_f16)
    exp, osel = oracle.decode_attn_topk(ref, q, L, k, scale)
    assert np.all(np.isfinite(got)), what
    assert gsel.shape == (B, H, kk)
    sc = scale if scale > 0 else 1.0 / math.sqrt(D)
    K = _recon(ref, "k", L)
    V = _recon(ref, "v", L)
    Q = q.astype(np.float64).reshape(B, H, D, 1)
    s = (K @ Q)[..., 0] * sc                                   # [B][H][L]
    eps = SCORE_ERR * sc * (np.abs(K) @ np.abs(Q))[..., 0].max(-1)   # [B][H]
    same = np.all(gsel == osel, axis=-1)
    g3, e3 = got.reshape(B, H, D), exp.reshape(B, H, D)
    for b, h in zip(*np.nonzero(~same)):
        g = gsel[b, h]
        assert np.all(np.diff(g) > 0) and g[0] >= 0 and g[-1] < L, (what, b, h, "malformed selection")
        keep = np.zeros(L, bool)
        keep[g] = True
        if kk < L:
            assert s[b, h][keep].min() >= s[b, h][~keep].max() - eps[b, h], (what, b, h, "invalid selection")
        # the output differs from the oracle's only through the swapped positions
        ok = np.zeros(L, bool)
        ok[osel[b, h]] = True
        m = s[b, h].max()
        den = np.exp(s[b, h][ok] - m).sum()
        swapped = keep ^ ok
        wsw = np.exp(s[b, h][swapped] - m) / den
        # |o_T' - o_T| <= sum over swapped j of w_j (|V^_j| + |o|), doubled for rounding
        bound = 2.0 * np.max((wsw[:, None] * (np.abs(V[b, h][swapped]) + np.abs(e3[b, h])[None])).sum(0)) + gu.ATOL
        assert np.max(np.abs(g3[b, h] - e3[b, h])) <= bound, (what, b, h, "swap bound")
    n_swapped = int((~same).sum())
    gu.note("%s: %d of %d (seq, head) selections differ at a near-tie" % (what, n_swapped, B * H))
    assert n_swapped <= max(1, max_swapped_frac * B * H), (what, n_swapped)
    gu.assert_close(g3[same], e3[same], what)
    return got, gsel


def test_topk_tiny_all_lengths_and_counts():
    w = W["tiny"]
    dev, ref = _kv_case(w, w.batch, 1)
    q = synth.step_q(w, 1)
    for L in (1, 2, 63, 64, 65, 127, 128, 129):
        for k in sorted({1, 3, math.ceil(L / 10), L, L + 7}):
            _topk_check(dev, ref, q, L, k, "tiny(D=64)")


def test_topk_opt67b_reduced_batch_steps():
    w = W["opt-6.7b"]
    nb, steps = 3, 32
    dev, ref = _kv_case(w, nb, steps)
    for t in (1, 17, 32):
        L = w.kv_len(t)
        q = synth.step_q(w, t)[:nb]
        for k in (1, math.ceil(L / 10), L // 2, L - 1):
            _topk_check(dev, ref, q, L, k, "opt-6.7b b=3 t=%d" % t)


def test_topk_long_context_outliers_and_constant_groups():
    w = W["long-t3"]
    nb, steps = 2, 2
    dev, ref = _kv_case(w, nb, steps)
    for t in (1, 2):
        L = w.kv_len(t)
        q = synth.step_q(w, t)[:nb]
        _topk_check(dev, ref, q, L, math.ceil(L / 10), "long-t3 b=2 t=%d" % t)


@pytest.mark.parametrize("L", [300, 2500])
def test_topk_exact_ties_decided_like_the_oracle(L):
    """K rows drawn from five distinct rows per (sequence, head): every score
    is one of five well-separated values, each shared by many positions, so
    every cut falls inside a run of bit-identical scores (one wavefront per
    (sequence, head) at L = 300, one workgroup at L = 2500)."""
    B, H, D = 2, 3, 128
    rng = np.random.default_rng(21)
    base = rng.standard_normal((B, H, 5, D)).astype(np.float16)
    pick = rng.integers(0, 5, (B, H, L))
    k16 = np.take_along_axis(base, pick[..., None].repeat(D, -1), axis=2)        # [B][H][L][D]
    k16 = np.ascontiguousarray(k16.transpose(0, 2, 1, 3).reshape(B, L, H * D))
    v16 = rng.standard_normal((B, L, H * D)).astype(np.float16)
    q = rng.standard_normal((B, H * D)).astype(np.float16)
    dev = gu.DevKV(B, H, D, L)
    ref = oracle.KVCache(B, H, D, L)
    dev.append(k16, v16, 0)
    oracle.kv_append(ref, k16, v16, 0)
    K = _recon(ref, "k", L)
    s = (K @ q.astype(np.float64).reshape(B, H, D, 1))[..., 0]
    for b in range(B):
        for h in range(H):
            u = np.unique(s[b, h])
            assert len(u) == 5 and np.min(np.diff(u)) > 1e-3, "distinct rows must score far apart"
    for k in (1, 7, 50, L // 2, L - 1):
        got, gsel = dev.attend_topk(q, L, k)
        exp, osel = oracle.decode_attn_topk(ref, q, L, k)
        gu.note("exact ties top_k %d" % k)
        assert np.array_equal(gsel, osel), k
        gu.assert_close(got, exp, "exact ties k=%d" % k)


@pytest.mark.parametrize("L", [2047, 2048, 2049, 3001])
def test_topk_lengths_around_the_kernel_switch(L):
    """Contexts up to 2048 run one wavefront per (sequence, head), longer ones
    one workgroup: both sides of the switch against the oracle."""
    w = W["opt-6.7b"]
    B, H, D = 2, 4, w.head_dim
    rng = np.random.default_rng(L)
    k16 = rng.standard_normal((B, L, H * D)).astype(np.float16)
    v16 = rng.standard_normal((B, L, H * D)).astype(np.float16)
    q = rng.standard_normal((B, H * D)).astype(np.float16)
    dev = gu.DevKV(B, H, D, L)
    ref = oracle.KVCache(B, H, D, L)
    dev.append(k16, v16, 0)
    oracle.kv_append(ref, k16, v16, 0)
    for k in (1, math.ceil(L / 10), L - 1):
        _topk_check(dev, ref, q, L, k, "L=%d" % L)


def test_topk_keeping_everything_is_dense_attention():
    w = W["opt-6.7b"]
    dev, ref = _kv_case(w, 2, 1)
    q = synth.step_q(w, 1)[:2]
    L = w.kv_len(1)
    got, gsel = _topk_check(dev, ref, q, L, L, "dense limit")
    dense = dev.attend(q, L)
    gu.assert_close(got, dense, "top-k (all kept) vs dense kernel")
    gu.assert_close(got, oracle.decode_attn(ref, q, L), "top-k (all kept) vs dense oracle")
    assert np.array_equal(gsel, np.broadcast_to(np.arange(L, dtype=np.int32), gsel.shape))


def test_topk_fp16_output_scale_and_optional_selection():
    w = W["opt-6.7b"]
    nb = 2
    dev, ref = _kv_case(w, nb, 1)
    q = synth.step_q(w, 1)[:nb]
    L = w.kv_len(1)
    _topk_check(dev, ref, q, L, 52, "fp16 out", out_f16=True)
    _topk_check(dev, ref, q, 300, 30, "scale 0.05", scale=0.05)
    a, sa = dev.attend_topk(q, L, 52)
    b, _ = dev.attend_topk(q, L, 52, want_sel=False)
    c, sc = dev.attend_topk(q, L, 52)
    assert np.array_equal(a, b) and np.array_equal(a, c) and np.array_equal(sa, sc)


@pytest.mark.parametrize("name,t,samples", [("opt-175b", 3, (0, 77, 143))])
def test_topk_full_size_sampled(name, t, samples):
    """The full workload's batch and heads in one launch (the configuration
    the benchmark times), sampled sequences checked against the oracle."""
    w = W[name]
    B, H, D, cap = w.batch, w.heads, w.head_dim, w.capacity
    L = w.kv_len(t)
    k = math.ceil(L / 10)
    gu.note("full-size top-k attention %s B=%d H=%d L=%d k=%d" % (name, B, H, L, k))
    dev = gu.DevKV(B, H, D, cap)
    for b0 in range(0, B, 8):
        nb = min(8, B - b0)
        sub = gu.fgq.kv_struct(dev.k_codes[b0:b0 + nb], dev.v_codes[b0:b0 + nb], dev.k_meta[b0:b0 + nb],
                               dev.v_meta[b0:b0 + nb], nb, H, D, cap)
        gu.fgq.fgq_kv_append(sub, gu.to_dev(synth.prompt_kv(w, "k", b0=b0, nb=nb)),
                             gu.to_dev(synth.prompt_kv(w, "v", b0=b0, nb=nb)), 0, w.prompt)
    for s_ in range(1, t + 1):
        dev.append(synth.step_kv(w, "k", s_), synth.step_kv(w, "v", s_), w.prompt + s_ - 1)
    q = synth.step_q(w, t)
    got, gsel = dev.attend_topk(q, L, k)
    for b in samples:
        ref = oracle.KVCache(1, H, D, cap)
        oracle.kv_append(ref, synth.prompt_kv(w, "k", b0=b, nb=1), synth.prompt_kv(w, "v", b0=b, nb=1), 0)
        for s_ in range(1, t + 1):
            oracle.kv_append(ref, synth.step_kv(w, "k", s_)[b:b + 1], synth.step_kv(w, "v", s_)[b:b + 1],
                             w.prompt + s_ - 1)

        class _One:   # the full launch's outputs of sequence b, in the shape _topk_check expects
            def attend_topk(self, q_, L_, k_, scale=0.0, out_f16=False):
                return got[b:b + 1], gsel[b:b + 1]

        _topk_check(_One(), ref, q[b:b + 1], L, k, "%s full-size seq %d" % (name, b))


def test_topk_repeatable_bitwise():
    w = W["long-t3"]
    dev, ref = _kv_case(w, 1, 1)
    q = synth.step_q(w, 1)[:1]
    L = w.kv_len(1)
    gu.note("top-k repeatability")
    a, sa = dev.attend_topk(q, L, 410)
    b, sb = dev.attend_topk(q, L, 410)
    assert np.array_equal(a, b) and np.array_equal(sa, sb)


def _random_case(B, H, D, L, seed):
    rng = np.random.default_rng(seed)
    k16 = rng.standard_normal((B, L, H * D)).astype(np.float16)
    v16 = rng.standard_normal((B, L, H * D)).astype(np.float16)
    q = rng.standard_normal((B, H * D)).astype(np.float16)
    dev = gu.DevKV(B, H, D, L)
    ref = oracle.KVCache(B, H, D, L)
    dev.append(k16, v16, 0)
    oracle.kv_append(ref, k16, v16, 0)
    return dev, ref, q


@pytest.mark.parametrize("L,D", [(14000, 128), (16416, 128), (40000, 64), (65536, 128)])
def test_topk_long_contexts(L, D):
    """Long contexts at 10% kept, a few, half, and everything: while the fp32
    scores and kept list fit 19840 positions (77.5 KB of LDS) the fp32
    workgroup kernel runs (above 64 KB of dynamic LDS at 14000 and 16416
    positions), beyond that the 16-bit-key kernel (candidate refinement
    inside the cut's bucket, P.V in buffered passes)."""
    dev, ref, q = _random_case(1, 2, D, L, L + D)
    for k in (math.ceil(L / 10), 3, L // 2):
        _topk_check(dev, ref, q, L, k, "long L=%d D=%d" % (L, D))
    got, gsel = _topk_check(dev, ref, q, L, L, "long L=%d D=%d, all kept" % (L, D))
    gu.assert_close(got, dev.attend(q, L), "long top-k (all kept) vs dense kernel")
    assert np.array_equal(gsel, np.broadcast_to(np.arange(L, dtype=np.int32), gsel.shape))


def test_topk_long_context_exact_ties_span_buffers():
    """Five distinct K rows per (sequence, head) over 20000 positions: the cut
    falls inside a run of ~4000 bit-identical scores, more candidates than one
    LDS buffer holds; the kept set must equal the oracle's (lower positions
    first)."""
    B, H, D, L = 1, 2, 128, 20000
    rng = np.random.default_rng(5)
    base = rng.standard_normal((B, H, 5, D)).astype(np.float16)
    pick = rng.integers(0, 5, (B, H, L))
    k16 = np.take_along_axis(base, pick[..., None].repeat(D, -1), axis=2)
    k16 = np.ascontiguousarray(k16.transpose(0, 2, 1, 3).reshape(B, L, H * D))
    v16 = rng.standard_normal((B, L, H * D)).astype(np.float16)
    q = rng.standard_normal((B, H * D)).astype(np.float16)
    dev = gu.DevKV(B, H, D, L)
    ref = oracle.KVCache(B, H, D, L)
    dev.append(k16, v16, 0)
    oracle.kv_append(ref, k16, v16, 0)
    for k in (1, 2000, 6500, L - 1):
        got, gsel = dev.attend_topk(q, L, k)
        exp, osel = oracle.decode_attn_topk(ref, q, L, k)
        gu.note("long exact ties top_k %d" % k)
        assert np.array_equal(gsel, osel), k
        gu.assert_close(got, exp, "long exact ties k=%d" % k)


@pytest.mark.parametrize("kk", [1840, 1841])
def test_topk_exact_ties_at_the_fp32_bound(kk):
    """kv_len + kk = 19840 is the largest selection the fp32 workgroup kernel
    holds (77.5 KB of dynamic LDS); one more kept position takes the
    16-bit-key kernel.  Five distinct K rows per (sequence, head) make runs of
    bit-identical scores at the cut; on both sides of the bound the kept
    positions must be the oracle's (ties to the lower position)."""
    B, H, D, L = 1, 2, 128, 18000
    gu.note("fp32 bound L=%d kk=%d" % (L, kk))
    rng = np.random.default_rng(kk)
    base = rng.standard_normal((B, H, 5, D)).astype(np.float16)
    pick = rng.integers(0, 5, (B, H, L))
    k16 = np.take_along_axis(base, pick[..., None].repeat(D, -1), axis=2)
    k16 = np.ascontiguousarray(k16.transpose(0, 2, 1, 3).reshape(B, L, H * D))
    v16 = rng.standard_normal((B, L, H * D)).astype(np.float16)
    q = rng.standard_normal((B, H * D)).astype(np.float16)
    dev = gu.DevKV(B, H, D, L)
    ref = oracle.KVCache(B, H, D, L)
    dev.append(k16, v16, 0)
    oracle.kv_append(ref, k16, v16, 0)
    got, gsel = dev.attend_topk(q, L, kk)
    exp, osel = oracle.decode_attn_topk(ref, q, L, kk)
    assert np.array_equal(gsel, osel)
    gu.assert_close(got, exp, "fp32 bound exact ties kk=%d" % kk)


def test_topk_long_context_all_scores_equal():
    """A zero query makes every score 0: the whole context is one candidate
    bucket; the first kk positions are kept and the output is their mean V."""
    B, H, D, L = 2, 2, 64, 30000
    dev, ref, _ = _random_case(B, H, D, L, 9)
    q = np.zeros((B, H * D), np.float16)
    kk = 3000
    got, gsel = dev.attend_topk(q, L, kk)
    exp, osel = oracle.decode_attn_topk(ref, q, L, kk)
    assert np.array_equal(gsel, np.broadcast_to(np.arange(kk, dtype=np.int32), gsel.shape))
    assert np.array_equal(osel, gsel)
    gu.assert_close(got, exp, "all scores equal")


def test_topk_16k_context_full_heads_sampled():
    """The grouped-query workload's context (16 sequences, 32 heads, 16416
    positions) as multi-head attention: one launch, three sequences against
    the oracle at 10% kept."""
    B, H, D, L = 16, 32, 128, 16416
    gu.note("top-k 16k context B=%d H=%d L=%d" % (B, H, L))
    rng = np.random.default_rng(77)
    dev = gu.DevKV(B, H, D, L)
    ks, vs = [], []
    for b in range(B):
        k16 = rng.standard_normal((1, L, H * D)).astype(np.float16)
        v16 = rng.standard_normal((1, L, H * D)).astype(np.float16)
        sub = gu.fgq.kv_struct(dev.k_codes[b:b + 1], dev.v_codes[b:b + 1], dev.k_meta[b:b + 1], dev.v_meta[b:b + 1],
                               1, H, D, L)
        gu.fgq.fgq_kv_append(sub, gu.to_dev(k16), gu.to_dev(v16), 0, L)
        ks.append(k16)
        vs.append(v16)
    q = rng.standard_normal((B, H * D)).astype(np.float16)
    k = math.ceil(L / 10)
    got, gsel = dev.attend_topk(q, L, k)
    for b in (0, 7, 15):
        ref = oracle.KVCache(1, H, D, L)
        oracle.kv_append(ref, ks[b], vs[b], 0)

        class _One:
            def attend_topk(self, q_, L_, k_, scale=0.0, out_f16=False):
                return got[b:b + 1], gsel[b:b + 1]

        _topk_check(_One(), ref, q[b:b + 1], L, k, "16k context seq %d" % b)
