"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bar: codes and meta bit-exact; attention and GEMM outputs within
max|gpu - oracle| <= 1e-2 and ||gpu - oracle||_2 / ||oracle||_2 <= 1e-3,
computed by the oracle on the same codes.  Sizes span several tiles and
ragged tails; the full-size workloads are checked on sampled outputs that the
oracle computes one sequence / one column group at a time.
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


def _special_groups():
    rng = np.random.default_rng(0)
    rows = []
    rows.append(np.full(64, 1.5))                           # constant
    rows.append(np.full(64, -0.0))                          # constant -0
    z = np.zeros(64); z[:32] = -0.0; z[40] = 2.0; rows.append(z)  # signed zeros at the min
    rows.append(np.r_[65504.0, -65504.0, rng.standard_normal(62)])
    rows.append(rng.standard_normal(64) * 2.0 ** -20)      # subnormal fp16 values
    sub = np.zeros(64); sub[1] = 2.0 ** -24; rows.append(sub)  # step underflows to 0
    rows.append(np.r_[0.0, 30.0, np.arange(1, 30, 2), np.zeros(64 - 17)])                 # tie ladder G1
    rows.append(np.r_[-8.0, 7.0, np.arange(-7.5, 7.0, 1.0), np.full(64 - 17, -8.0)])     # tie ladder G2
    k = rng.integers(0, 16, 64); k[0], k[1] = 0, 15; rows.append((k - 8) * 0.25)          # on-grid
    rows.append(rng.standard_normal(64) * 1000.0)
    return np.array(rows).astype(np.float16)


def test_quantize_bit_exact_random_and_special():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((333, 64 * 7)) * 3.0).astype(np.float16)
    sp = _special_groups()                                   # [10][64]
    x[:10, 64:128] = sp
    x[20:30, 0:64] = sp
    gu.note("quantize 333x448 random + special groups")
    c, m = gu.quantize(x)
    rc, rm = oracle.quantize_g64(x)
    assert np.array_equal(c, rc) and np.array_equal(m, rm)


def test_quantize_leading_dimension():
    rng = np.random.default_rng(2)
    full = rng.standard_normal((37, 256 + 64)).astype(np.float16)
    gu.note("quantize with ld_x > cols")
    torch = gu.torch_cuda()
    xd = gu.to_dev(full)
    codes = torch.empty((37, 128), dtype=torch.uint8, device="cuda")
    meta = torch.empty((37, 4), dtype=torch.int32, device="cuda")
    gu.fgq.fgq_quantize_g64(xd, 37, 256, 320, codes, meta)
    torch.cuda.synchronize()
    rc, rm = oracle.quantize_g64(np.ascontiguousarray(full[:, :256]))
    assert np.array_equal(gu.to_host(codes), rc)
    assert np.array_equal(gu.to_host(meta, np.uint32), rm)


@pytest.mark.parametrize("name,idx", [("tiny", 0), ("opt-6.7b", 0), ("opt-6.7b", 5), ("opt-30b", 4),
                                      ("opt-175b", 0), ("opt-175b", 4)])
def test_quantize_bit_exact_workload_weights(name, idx):
    w = W[name]
    K, N = w.weights[idx]
    gu.note("quantize weight %s[%d] %dx%d" % (name, idx, K, N))
    x = synth.weight(w, idx)
    c, m = gu.quantize(x)
    rc, rm = oracle.quantize_g64(x)
    assert np.array_equal(c, rc), "codes differ"
    assert np.array_equal(m, rm), "meta differs"


def _kv_case(w, nb, steps):
    """Prompt bulk append then `steps` one-token appends, GPU and oracle."""
    B, H, D = nb, w.heads, w.head_dim
    cap = w.prompt + steps
    dev = gu.DevKV(B, H, D, cap)
    ref = oracle.KVCache(B, H, D, cap)
    pk = synth.prompt_kv(w, "k", nb=nb)
    pv = synth.prompt_kv(w, "v", nb=nb)
    dev.append(pk, pv, 0)
    oracle.kv_append(ref, pk, pv, 0)
    del pk, pv
    for t in range(1, steps + 1):
        sk = synth.step_kv(w, "k", t)[:nb]
        sv = synth.step_kv(w, "v", t)[:nb]
        dev.append(sk, sv, w.prompt + t - 1)
        oracle.kv_append(ref, sk, sv, w.prompt + t - 1)
    return dev, ref


@pytest.mark.parametrize("name,nb,steps", [("tiny", 4, 1), ("opt-6.7b", 3, 4), ("long-t3", 2, 2)])
def test_kv_append_bit_exact(name, nb, steps):
    w = W[name]
    gu.note("kv_append %s batch %d steps %d" % (name, nb, steps))
    dev, ref = _kv_case(w, nb, steps)
    h = dev.host()
    for a in ("k_codes", "k_meta", "v_codes", "v_meta"):
        assert np.array_equal(h[a], getattr(ref, a)), a


def test_append_one_by_one_equals_bulk_on_gpu():
    w = W["opt-6.7b"]
    nb, L = 2, 40
    k = synth.prompt_kv(w, "k", nb=nb, nt=L)
    v = synth.prompt_kv(w, "v", nb=nb, nt=L)
    gu.note("append one-by-one vs bulk")
    a = gu.DevKV(nb, w.heads, w.head_dim, L)
    a.append(k, v, 0)
    b = gu.DevKV(nb, w.heads, w.head_dim, L)
    for t in range(L):
        b.append(np.ascontiguousarray(k[:, t:t + 1]), np.ascontiguousarray(v[:, t:t + 1]), t)
    ha, hb = a.host(), b.host()
    for key in ha:
        assert np.array_equal(ha[key], hb[key]), key


def _attn_check(dev, ref, q, L, what, out_f16=False, scale=0.0):
    gu.note("attention %s kv_len %d" % (what, L))
    got = dev.attend(q, L, scale, out_f16)
    exp = oracle.decode_attn(ref, q, L, scale)
    gu.assert_close(got, exp, what)


def test_attention_tiny_all_lengths():
    w = W["tiny"]
    dev, ref = _kv_case(w, w.batch, 1)
    q = synth.step_q(w, 1)
    for L in (1, 2, 63, 64, 65, 127, 128, 129):
        _attn_check(dev, ref, q, L, "tiny(D=64)")


def test_attention_opt67b_reduced_batch_all_steps():
    w = W["opt-6.7b"]
    nb, steps = 3, 32
    dev, ref = _kv_case(w, nb, steps)
    for t in (1, 2, 17, 31, 32):
        q = synth.step_q(w, t)[:nb]
        _attn_check(dev, ref, q, w.kv_len(t), "opt-6.7b b=3 t=%d" % t)


def test_attention_long_context_outliers_and_constant_groups():
    w = W["long-t3"]
    nb, steps = 2, 2
    dev, ref = _kv_case(w, nb, steps)
    for t in (1, 2):
        q = synth.step_q(w, t)[:nb]
        _attn_check(dev, ref, q, w.kv_len(t), "long-t3 b=2 t=%d" % t)


def test_attention_fp16_output_and_scale():
    w = W["opt-6.7b"]
    nb = 2
    dev, ref = _kv_case(w, nb, 1)
    q = synth.step_q(w, 1)[:nb]
    _attn_check(dev, ref, q, 513, "fp16 out", out_f16=True)
    _attn_check(dev, ref, q, 300, "scale 0.05", scale=0.05)


def _full_size_attention_rows(name, t, samples):
    w = W[name]
    B, H, D, cap = w.batch, w.heads, w.head_dim, w.capacity
    gu.note("full-size attention %s B=%d H=%d L=%d" % (name, B, H, w.kv_len(t)))
    dev = gu.DevKV(B, H, D, cap)
    chunk = 8
    for b0 in range(0, B, chunk):
        nb = min(chunk, B - b0)
        sub = gu.fgq.kv_struct(dev.k_codes[b0:b0 + nb], dev.v_codes[b0:b0 + nb], dev.k_meta[b0:b0 + nb],
                               dev.v_meta[b0:b0 + nb], nb, H, D, cap)
        kd = gu.to_dev(synth.prompt_kv(w, "k", b0=b0, nb=nb))
        vd = gu.to_dev(synth.prompt_kv(w, "v", b0=b0, nb=nb))
        gu.fgq.fgq_kv_append(sub, kd, vd, 0, w.prompt)
        del kd, vd
    for s in range(1, t + 1):
        dev.append(synth.step_kv(w, "k", s), synth.step_kv(w, "v", s), w.prompt + s - 1)
    q = synth.step_q(w, t)
    got = dev.attend(q, w.kv_len(t))
    h = dev.host()
    for b in samples:
        ref = oracle.KVCache(1, H, D, cap)
        oracle.kv_append(ref, synth.prompt_kv(w, "k", b0=b, nb=1), synth.prompt_kv(w, "v", b0=b, nb=1), 0)
        for s in range(1, t + 1):
            oracle.kv_append(ref, synth.step_kv(w, "k", s)[b:b + 1], synth.step_kv(w, "v", s)[b:b + 1],
                             w.prompt + s - 1)
        for a in ("k_codes", "k_meta", "v_codes", "v_meta"):
            assert np.array_equal(h[a][b], getattr(ref, a)[0]), (a, b)
        exp = oracle.decode_attn(ref, q[b:b + 1], w.kv_len(t))
        gu.assert_close(got[b:b + 1], exp, "%s full-size seq %d" % (name, b))


@pytest.mark.parametrize("name,t,samples", [("opt-175b", 3, (0, 77, 143)), ("long-t3", 2, (0, 31)),
                                           ("opt-30b", 2, (0, 50, 95)), ("opt-6.7b", 32, (0, 63))])
def test_attention_full_size_sampled(name, t, samples):
    _full_size_attention_rows(name, t, samples)


@pytest.mark.parametrize("B,H,D,L", [(8, 256, 64, 3100), (16, 128, 128, 4100)])
def test_attention_long_chunk_plan_sampled(B, H, D, L):
    """2048 (sequence, head) pairs over 3-4K positions: one workgroup of four
    waves per pair (each wave takes every fourth chunk), no split, the
    long-chunk launch with a ragged last chunk; sampled sequences against the
    oracle on the same codes."""
    import dataclasses
    w = dataclasses.replace(W["long-t3"], g=B, m=1, heads=H, head_dim=D, prompt=L, steps=1)
    gu.note("long-chunk plan B=%d H=%d D=%d L=%d" % (B, H, D, L))
    dev = gu.DevKV(B, H, D, L)
    for b0 in range(0, B, 4):
        nb = min(4, B - b0)
        sub = gu.fgq.kv_struct(dev.k_codes[b0:b0 + nb], dev.v_codes[b0:b0 + nb], dev.k_meta[b0:b0 + nb],
                               dev.v_meta[b0:b0 + nb], nb, H, D, L)
        gu.fgq.fgq_kv_append(sub, gu.to_dev(synth.prompt_kv(w, "k", b0=b0, nb=nb)),
                             gu.to_dev(synth.prompt_kv(w, "v", b0=b0, nb=nb)), 0, L)
    q = synth.step_q(w, 1)
    got = dev.attend(q, L)
    for b in (0, B - 1):
        ref = oracle.KVCache(1, H, D, L)
        oracle.kv_append(ref, synth.prompt_kv(w, "k", b0=b, nb=1), synth.prompt_kv(w, "v", b0=b, nb=1), 0)
        gu.assert_close(got[b:b + 1], oracle.decode_attn(ref, q[b:b + 1], L), "long-chunk seq %d" % b)


def _small_long_cache(B, H, D, L):
    import dataclasses
    w = dataclasses.replace(W["long-t3"], g=B, m=1, heads=H, head_dim=D, prompt=L, steps=1)
    dev = gu.DevKV(B, H, D, L)
    ref = oracle.KVCache(B, H, D, L)
    k = synth.prompt_kv(w, "k", nb=B)
    v = synth.prompt_kv(w, "v", nb=B)
    dev.append(k, v, 0)
    oracle.kv_append(ref, k, v, 0)
    return w, dev, ref


@pytest.mark.parametrize("B,H,D,L,splits", [
    (2, 3, 64, 8065, 7),      # last split: 1 token, so waves 1-3 of its items stream nothing
    (2, 3, 128, 12673, 12),   # the same at head_dim 128
    (1, 2, 128, 10563, 10),   # last split: 2 whole chunks + 3 tokens, wave 3 idle
    (1, 2, 128, 1024, 1),     # the shortest sequence that takes four waves per pair: no split
    (1, 2, 128, 2048, 2),     # two splits of 1056 and 992 positions
    (3, 32, 64, 5000, 4),     # 7 chunks per split (wave 3 takes one fewer), last 5 + 8 tokens
])
def test_attention_four_waves_per_item(B, H, D, L, splits):
    """Few (sequence, head) pairs over >= 2048 positions: one workgroup of four
    waves per work item, merged in LDS, combined with a split of the sequence
    (the split count is read back from the workspace size).  Every sequence
    against the oracle on the same codes, and bitwise repeatable."""
    assert gu.fgq.fgq_decode_attn_ws_bytes(B, H, D, L) == (B * H * splits * (D + 4) * 4 if splits > 1 else 0)
    gu.note("four waves per item B=%d H=%d D=%d L=%d splits=%d" % (B, H, D, L, splits))
    w, dev, ref = _small_long_cache(B, H, D, L)
    q = synth.step_q(w, 1)
    got = dev.attend(q, L)
    gu.assert_close(got, oracle.decode_attn(ref, q, L), "four-wave items")
    assert np.array_equal(got, dev.attend(q, L))


def test_attention_one_wave_and_four_wave_items_agree():
    """8 x 32 pairs: at 1023 positions a pair is one wave's item (three splits
    of 384, 384 and 255 tokens), at 1024 one workgroup's with no split; both
    against the oracle on the same cache."""
    B, H, D = 8, 32, 128
    assert gu.fgq.fgq_decode_attn_ws_bytes(B, H, D, 1023) == B * H * 3 * (D + 4) * 4
    assert gu.fgq.fgq_decode_attn_ws_bytes(B, H, D, 1024) == 0
    nb = 2
    w, dev, ref = _small_long_cache(nb, H, D, 1024)
    q = synth.step_q(w, 1)
    wide = gu.DevKV(B, H, D, 1024)
    for a in ("k_codes", "k_meta", "v_codes", "v_meta"):
        getattr(wide, a)[:nb].copy_(getattr(dev, a))
        getattr(wide, a)[nb:].copy_(getattr(dev, a)[:1].expand(B - nb, -1, -1, -1))
    qw = np.concatenate([q, np.repeat(q[:1], B - nb, axis=0)])
    for L in (1023, 1024):
        gu.note("one- vs four-wave items at L=%d" % L)
        gu.assert_close(wide.attend(qw, L)[:nb], oracle.decode_attn(ref, q, L), "L=%d" % L)


def test_attention_result_does_not_depend_on_batch_split_plan():
    """The same sequences attended alone (long splits merged) and inside a wide
    batch (one split) agree within tolerance, and each matches the oracle."""
    w = W["opt-6.7b"]
    dev, ref = _kv_case(w, 2, 1)
    q = synth.step_q(w, 1)[:2]
    L = w.kv_len(1)
    gu.note("split-plan independence")
    wide = gu.DevKV(64, w.heads, w.head_dim, dev.cap)
    for a in ("k_codes", "k_meta", "v_codes", "v_meta"):
        getattr(wide, a)[:2].copy_(getattr(dev, a))
        getattr(wide, a)[2:].copy_(getattr(dev, a)[:1].expand(62, -1, -1, -1))
    qw = np.concatenate([q, np.repeat(q[:1], 62, axis=0)])
    a1 = dev.attend(q, L)
    a2 = wide.attend(qw, L)[:2]
    exp = oracle.decode_attn(ref, q, L)
    gu.assert_close(a1, exp, "narrow plan")
    gu.assert_close(a2, exp, "wide plan")
    assert gu.fgq.fgq_decode_attn_ws_bytes(2, w.heads, w.head_dim, L) > 0
    assert gu.fgq.fgq_decode_attn_ws_bytes(64, w.heads, w.head_dim, L) >= 0


def test_attention_repeatable_bitwise():
    w = W["long-t3"]
    dev, ref = _kv_case(w, 1, 1)
    q = synth.step_q(w, 1)[:1]
    gu.note("attention repeatability")
    a = dev.attend(q, w.kv_len(1))
    b = dev.attend(q, w.kv_len(1))
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------- GEMM

def _gemm_case(x16, g, m, Wt):
    K, N = Wt.shape
    codes, meta = gu.quantize(Wt)
    rc, rm = oracle.quantize_g64(Wt)
    assert np.array_equal(codes, rc) and np.array_equal(meta, rm)
    pc, pm = gu.pack(gu.to_dev(codes), gu.to_dev(meta), K, N)
    return rc, rm, pc, pm


def test_pack_matches_layout_definition():
    """Column groups of very different ranges (exponents 0 up to 24, fp16
    subnormal minima after scaling) packed bit for bit as the header says."""
    rng = np.random.default_rng(3)
    Wt = (rng.standard_normal((96, 320)) * 0.02).astype(np.float16)
    Wt[:, 64:128] *= np.float16(400.0)                      # steps ~ 2.5: e = 16
    Wt[:, 128:192] = (rng.standard_normal((96, 64)) * 20000).clip(-65000, 65000).astype(np.float16)
    Wt[:, 192:256] *= np.float16(1e-3)                      # tiny steps: e = 0
    gu.note("pack layout 96x320")
    codes, meta = oracle.quantize_g64(Wt)
    pc, pm = gu.pack(gu.to_dev(codes), gu.to_dev(meta), 96, 320)
    ec, em = gu.pack_reference(codes, meta)
    assert em.size == gu.fgq.fgq_pack_weight_meta_words(96, 320)
    assert np.array_equal(gu.to_host(pc, np.uint32), ec)
    assert np.array_equal(gu.to_host(pm, np.uint32), em)
    assert em[-5:].min() == 0 and em[-5:].max() >= 20      # the tiny and the huge column groups


def test_gemm_on_wide_ranging_column_groups():
    """The GEMM undoes each column group's power of two: groups whose steps
    need exponents from 0 to 24 against the oracle."""
    rng = np.random.default_rng(31)
    K, N, g, m = 256, 384, 8, 2
    Wt = (rng.standard_normal((K, N)) * 0.02).astype(np.float16)
    Wt[:, 64:128] *= np.float16(400.0)
    Wt[:, 128:192] = (rng.standard_normal((K, 64)) * 20000).clip(-65000, 65000).astype(np.float16)
    Wt[:, 192:256] *= np.float16(1e-3)
    Wt[:, 256:320] = np.float16(0.75)                       # constant groups: step 0
    X = (rng.standard_normal((g * m, K)) * 0.01).astype(np.float16)
    rc, rm, pc, pm = _gemm_case(X, g, m, Wt)
    ex = gu.to_host(pm, np.uint32)[-(N // 64):]
    gu.note("gemm wide-ranging groups, exponents %s" % ex.tolist())
    assert ex.min() == 0 and ex.max() >= 20
    y = gu.gemm(X, g, m, pc, pm, K, N)
    exp = oracle.dequant_gemm(X, g, m, rc, rm)
    for c in range(N // 64):   # each column group against the bar on its own scale
        sl = slice(64 * c, 64 * c + 64)
        s = max(1.0, float(np.abs(exp[:, sl]).max()))
        gu.assert_close(y[:, sl] / s, exp[:, sl] / s, "group %d (scaled by %.3g)" % (c, s))


# The last three take two k-phases per workgroup: an odd chunk count with no
# split (33 x 544), an odd per-split chunk count with 8 splits and a last
# workgroup holding one valid column group (145 x 4128 x 1088), and 17 splits
# whose last one has a single chunk, so one phase has no work (150 x 8224).
@pytest.mark.parametrize("M,K,N", [(1, 32, 64), (5, 96, 320), (16, 64, 256), (17, 160, 64), (37, 256, 512),
                                   (144, 128, 192), (145, 96, 128), (300, 64, 64), (4, 0, 64),
                                   (33, 544, 320), (145, 4128, 1088), (150, 8224, 576)])
def test_gemm_ragged_shapes(M, K, N):
    rng = np.random.default_rng(M * 7 + K + N)
    Wt = (rng.standard_normal((K, N)) * 0.02).astype(np.float16)
    X = rng.standard_normal((M, K)).astype(np.float16)
    gu.note("gemm ragged M=%d K=%d N=%d" % (M, K, N))
    if K == 0:
        torch = gu.torch_cuda()
        pc = torch.empty(16, dtype=torch.int32, device="cuda")
        y = gu.gemm(X, M, 1, pc, pc, K, N)
        assert np.all(y == 0)
        return
    rc, rm, pc, pm = _gemm_case(X, M, 1, Wt)
    y = gu.gemm(X, M, 1, pc, pm, K, N)
    gu.assert_close(y, oracle.dequant_gemm(X, M, 1, rc, rm), "gemm %dx%dx%d" % (M, K, N))


# Every row-tile count (1..9 m-tiles) with a K long enough for several ring
# turns and a split plan: k-phased workgroups of up to 8 m-tiles take slots
# of two of a wave's chunks where three slots fit in LDS, so this covers both
# slot sizes, the ring's tail and a ragged last column block (N = 640).
@pytest.mark.parametrize("M", [8, 24, 40, 56, 72, 88, 104, 120, 136])
def test_gemm_every_row_tile_count(M):
    K, N = 8192, 640
    rng = np.random.default_rng(M + 11)
    Wt = (rng.standard_normal((K, N)) * 0.02).astype(np.float16)
    X = rng.standard_normal((M, K)).astype(np.float16)
    gu.note("gemm row tiles M=%d K=%d N=%d" % (M, K, N))
    rc, rm, pc, pm = _gemm_case(X, M, 1, Wt)
    y = gu.gemm(X, M, 1, pc, pm, K, N)
    gu.assert_close(y, oracle.dequant_gemm(X, M, 1, rc, rm), "gemm %dx%dx%d" % (M, K, N))


@pytest.mark.parametrize("name,idx", [("tiny", 0), ("opt-6.7b", 0), ("opt-6.7b", 4), ("opt-6.7b", 5),
                                      ("opt-30b", 0)])
def test_gemm_workload_full(name, idx):
    w = W[name]
    K, N = w.weights[idx]
    gu.note("gemm %s[%d] M=%d K=%d N=%d" % (name, idx, w.batch, K, N))
    Wt = synth.weight(w, idx)
    X = synth.gemm_x(w, idx, 1)
    rc, rm, pc, pm = _gemm_case(X, w.g, w.m, Wt)
    y = gu.gemm(X, w.g, w.m, pc, pm, K, N)
    gu.assert_close(y, oracle.dequant_gemm(X, w.g, w.m, rc, rm), "gemm %s[%d]" % (name, idx))


def _sampled_columns_check(Wt, X, g, m, slices, what):
    """GEMM of the full weight on the GPU; the oracle quantises and multiplies
    whole-group column slices on its own (groups run along N, so a slice of
    whole groups has the same codes), after the GPU's codes of each slice are
    checked equal to the oracle's."""
    K, N = Wt.shape
    codes, meta = gu.quantize(Wt)
    refs = []
    for n0 in slices:
        rc, rm = oracle.quantize_g64(np.ascontiguousarray(Wt[:, n0:n0 + 256]))
        assert np.array_equal(codes[:, n0 // 2:(n0 + 256) // 2], rc), (what, n0)
        assert np.array_equal(meta[:, n0 // 64:(n0 + 256) // 64], rm), (what, n0)
        refs.append((n0, rc, rm))
    pc, pm = gu.pack(gu.to_dev(codes), gu.to_dev(meta), K, N)
    del codes, meta
    y = gu.gemm(X, g, m, pc, pm, K, N)
    for n0, rc, rm in refs:
        gu.assert_close(y[:, n0:n0 + 256], oracle.dequant_gemm(X, g, m, rc, rm), "%s cols %d.." % (what, n0))


@pytest.mark.parametrize("idx", [4, 5])
def test_gemm_opt30b_sampled_columns(idx):
    """OPT-30B FFN weights (7168 x 28672 and 28672 x 7168) at full size with the
    block of M = 96 = 24 x 4 rows; the oracle recomputes three 256-column slices."""
    w = W["opt-30b"]
    K, N = w.weights[idx]
    gu.note("gemm opt-30b[%d] M=%d K=%d N=%d" % (idx, w.batch, K, N))
    _sampled_columns_check(synth.weight(w, idx), synth.gemm_x(w, idx, 1), w.g, w.m,
                           (0, N // 2 + 64, N - 256), "opt-30b[%d]" % idx)


@pytest.mark.parametrize("idx", [0, 4, 5])
def test_gemm_opt175b_sampled_columns(idx):
    """Bench launch configuration (M = 144 = 36 x 4) at full size; the oracle
    recomputes three 256-column slices (whole weight groups)."""
    w = W["opt-175b"]
    K, N = w.weights[idx]
    gu.note("gemm opt-175b[%d] M=%d K=%d N=%d" % (idx, w.batch, K, N))
    _sampled_columns_check(synth.weight(w, idx), synth.gemm_x(w, idx, 1), w.g, w.m,
                           (0, N // 2 + 64, N - 256), "opt-175b[%d]" % idx)


# Large ragged shapes at full size, checked on sampled columns: two k-phases
# with three M blocks and an odd chunk count; a partial last column tile with
# one M block; two M blocks and a partial last tile.  Slices cover the first
# column tile, a tile boundary and the last (partial) tile.
@pytest.mark.parametrize("M,K,N,tc", [(290, 8416, 14592, 256), (144, 8416, 33600, 256), (150, 9472, 33600, 512)])
def test_gemm_large_ragged_sampled_columns(M, K, N, tc):
    gu.note("gemm large ragged M=%d K=%d N=%d" % (M, K, N))
    Wt = synth.to_f16(synth.normal(synth.stream_key(90, M, K, N), K * N, 0.02)).reshape(K, N)
    X = synth.to_f16(synth.normal(synth.stream_key(91, M, K, N), M * K)).reshape(M, K)
    _sampled_columns_check(Wt, X, M, 1, (0, 5 * tc - 128, N - 256), "gemm %dx%dx%d" % (M, K, N))


@pytest.mark.parametrize("K,N", [(1024, 512), (4128, 1088)])
def test_gemm_block_identity_and_determinism(K, N):
    """Y(g, m) against the m GPU batches run one at a time (within tolerance:
    the launch plan differs), and bitwise repeatability (the second shape
    sums two k-phases per workgroup and eight K splits)."""
    rng = np.random.default_rng(9)
    g, m = 36, 4
    Wt = (rng.standard_normal((K, N)) * 0.02).astype(np.float16)
    X = rng.standard_normal((g * m, K)).astype(np.float16)
    rc, rm, pc, pm = _gemm_case(X, g, m, Wt)
    gu.note("gemm block identity K=%d N=%d" % (K, N))
    y = gu.gemm(X, g, m, pc, pm, K, N)
    y2 = gu.gemm(X, g, m, pc, pm, K, N)
    assert np.array_equal(y, y2)
    parts = np.concatenate([gu.gemm(np.ascontiguousarray(X[j * g:(j + 1) * g]), g, 1, pc, pm, K, N)
                            for j in range(m)])
    gu.assert_close(y, parts, "block vs per-batch")
    gu.assert_close(y, oracle.dequant_gemm(X, g, m, rc, rm), "block vs oracle")


def test_gemm_fp16_output():
    w = W["opt-6.7b"]
    K, N = w.weights[0]
    Wt = synth.weight(w, 0)
    X = synth.gemm_x(w, 0, 2)
    rc, rm, pc, pm = _gemm_case(X, w.g, w.m, Wt)
    gu.note("gemm fp16 output")
    y = gu.gemm(X, w.g, w.m, pc, pm, K, N, y_f16=True)
    exp = oracle.dequant_gemm(X, w.g, w.m, rc, rm)
    # fp16 rounding of |Y| up to ~8 adds up to 2^-11 relative on top of the fp32 bar
    gu.assert_close(y, exp, "gemm fp16 out")


def test_gpu_rejects_capacity_overflow_without_writing():
    w = W["tiny"]
    dev = gu.DevKV(2, w.heads, w.head_dim, 8)
    k = np.ones((2, 3, w.hidden), np.float16)
    gu.note("capacity error")
    with pytest.raises(gu.fgq.FgqError) as e:
        dev.append(k, k, 6)
    assert e.value.status == gu.fgq.FGQ_ERR_CAPACITY
    h = dev.host()
    assert all(np.all(v == 0) for v in h.values())
