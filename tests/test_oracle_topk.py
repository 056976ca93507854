"""Pins of the oracle's top-K sparse decode attention.

The pages name the approximation (read only the top 10% of the value cache:
FlexGen review on blog.gzher.com, section 3.4; paper-graph-ui FlexGen summary,
section 3.3, the paper's section-5 approximate methods) but give no formula.
The reading pinned here: score every position over the compressed K as dense
decode attention does, keep the top_k largest scores (compared as fp32
values, equal scores going to the lower position), softmax over the kept
positions only.  Each pin checks the oracle against something other than
itself: exact rational scores with 50-digit exponentials, torch's topk and
softmax on exactly representable inputs, the dense oracle (pinned on its own)
when every position is kept, the argmax row when one is kept, and hand-built
exact ties.
"""
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch

import oracle
import synth


def _fill(B, H, D, L, seed, cap_extra=2):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, L, H * D)).astype(np.float16)
    v = rng.standard_normal((B, L, H * D)).astype(np.float16)
    q = rng.standard_normal((B, H * D)).astype(np.float16)
    kv = oracle.KVCache(B, H, D, L + cap_extra)
    oracle.kv_append(kv, k, v, 0)
    return kv, q


def _recon(kv, which, L):
    codes = kv.k_codes if which == "k" else kv.v_codes
    meta = kv.k_meta if which == "k" else kv.v_meta
    B, H = codes.shape[:2]
    D = kv.head_dim
    c = codes[:, :, :L].reshape(-1, D // 2)
    m = meta[:, :, :L].reshape(-1, D // 64)
    return oracle.dequant_g64(c, m).reshape(B, H, L, D)


def _scores64(kv, q, L):
    """fp64 scores from numpy's matmul of the reconstructions (a library routine)."""
    B, H, D = kv.batch, kv.heads, kv.head_dim
    K = _recon(kv, "k", L).astype(np.float64)
    Q = q.astype(np.float64).reshape(B, H, D, 1)
    return (K @ Q)[..., 0] / np.sqrt(D)                   # [B][H][L]


def test_keeping_every_position_is_dense_attention_bit_for_bit():
    B, H, D, L = 2, 3, 128, 37
    kv, q = _fill(B, H, D, L, 11)
    dense = oracle.decode_attn(kv, q, L)
    for k in (L, L + 5):
        out, sel = oracle.decode_attn_topk(kv, q, L, k)
        assert np.array_equal(out, dense)
        assert sel.shape == (B, H, L) and np.array_equal(sel, np.broadcast_to(np.arange(L), (B, H, L)))


def test_keeping_one_position_returns_the_argmax_value_row():
    B, H, D, L = 2, 2, 64, 29
    kv, q = _fill(B, H, D, L, 12)
    out, sel = oracle.decode_attn_topk(kv, q, L, 1)
    s = _scores64(kv, q, L)
    V = _recon(kv, "v", L)
    for b in range(B):
        for h in range(H):
            j = int(np.argmax(s[b, h]))
            assert sel[b, h, 0] == j
            assert np.array_equal(out[b, h * D:(h + 1) * D], V[b, h, j])


def test_brute_force_exact_scores_50_digit_softmax():
    """Exact rational scores (fp16 q times fp32 reconstructions, D = 64, scale
    1/8), the exact top-k set with the lower-position rule, exp to 50 digits."""
    B, H, D, L, k = 2, 2, 64, 11, 4
    kv, q = _fill(B, H, D, L, 13)
    got, sel = oracle.decode_attn_topk(kv, q, L, k)
    K = _recon(kv, "k", L)
    V = _recon(kv, "v", L)
    mpmath.mp.dps = 50
    for b in range(B):
        for h in range(H):
            qv = [Fraction(float(x)) for x in q[b, h * D:(h + 1) * D]]
            s = [sum(qv[d] * Fraction(float(K[b, h, j, d])) for d in range(D)) / 8 for j in range(L)]
            order = sorted(range(L), key=lambda j: (-s[j], j))
            keep = sorted(order[:k])
            # the exact set is also the fp32 set here: no two scores near the cut
            gap = s[order[k - 1]] - s[order[k]]
            assert gap > Fraction(1, 2 ** 10), "inputs must not tie at the cut"
            assert list(sel[b, h]) == keep
            mx = max(s)
            e = {j: mpmath.exp(mpmath.mpf(s[j].numerator) / s[j].denominator -
                               mpmath.mpf(mx.numerator) / mx.denominator) for j in keep}
            den = sum(e.values())
            for d in range(D):
                ref = float(sum(e[j] * mpmath.mpf(float(V[b, h, j, d])) for j in keep) / den)
                assert abs(float(got[b, h * D + d]) - ref) <= 2.0 ** -23 * abs(ref) + 1e-30, (b, h, d)


def test_on_grid_cache_reduces_to_torch_topk_softmax():
    """K, V on their groups' 16-level grid reconstruct exactly; then the oracle
    equals torch.topk on the fp64 scores, softmax over the kept scores, and
    the weighted sum of the kept fp16 V rows."""
    B, H, D, L, k = 2, 3, 128, 40, 7
    rng = np.random.default_rng(14)

    def grid(shape):
        c = rng.integers(0, 16, shape + (D // 64, 64))
        c[..., 0], c[..., 1] = 0, 15
        e = rng.integers(-6, 2, shape + (D // 64, 1))
        return ((c - 8) * 2.0 ** e).reshape(shape + (D,)).astype(np.float16)

    kh, vh = grid((B, L, H)), grid((B, L, H))
    q = rng.standard_normal((B, H * D)).astype(np.float16)
    kv = oracle.KVCache(B, H, D, L)
    oracle.kv_append(kv, kh.reshape(B, L, H * D), vh.reshape(B, L, H * D), 0)
    got, sel = oracle.decode_attn_topk(kv, q, L, k)
    Q = torch.from_numpy(q.astype(np.float64)).reshape(B, H, D, 1)
    Kt = torch.from_numpy(kh.astype(np.float64)).permute(0, 2, 1, 3).contiguous()   # [B][H][L][D]
    Vt = torch.from_numpy(vh.astype(np.float64)).permute(0, 2, 1, 3).contiguous()
    s = torch.matmul(Kt, Q)[..., 0] / np.sqrt(D)                                     # [B][H][L]
    top = torch.topk(s, k, dim=-1)
    srt = torch.sort(s, dim=-1, descending=True).values
    assert torch.all(srt[..., k - 1] - srt[..., k] > 1e-6), "inputs must not tie at the cut"
    p = torch.softmax(top.values, dim=-1)                                             # [B][H][k]
    rows = torch.gather(Vt, 2, top.indices[..., None].expand(B, H, k, D))
    ref = (p[..., None] * rows).sum(2).reshape(B, H * D).numpy()
    assert np.array_equal(sel, np.sort(top.indices.numpy(), axis=-1))
    assert np.allclose(got, ref, rtol=2.0 ** -22, atol=1e-30)


def test_exact_ties_go_to_the_lower_position():
    """Duplicated K rows give bit-identical scores; the cut falls inside a run
    of equal scores, and the lower positions of the run are the ones kept."""
    B, H, D = 1, 1, 64
    rng = np.random.default_rng(15)
    base = rng.standard_normal((8, D)).astype(np.float16)
    q = rng.standard_normal((1, D)).astype(np.float16)
    s8 = base.astype(np.float64) @ q[0].astype(np.float64)
    hi = int(np.argmax(s8))
    mid = int(np.argsort(s8)[3])                       # a row that is neither the best nor the worst
    lo = int(np.argmin(s8))
    # positions: 0 lo, 1 mid, 2 hi, 3 mid, 4 lo, 5 mid, 6 mid, 7 lo
    rows = np.stack([base[i] for i in (lo, mid, hi, mid, lo, mid, mid, lo)])
    v = rng.standard_normal((8, D)).astype(np.float16)
    kv = oracle.KVCache(B, H, D, 8)
    oracle.kv_append(kv, rows[None], v[None], 0)
    for k, want in ((1, [2]), (2, [1, 2]), (3, [1, 2, 3]), (4, [1, 2, 3, 5]), (5, [1, 2, 3, 5, 6]),
                    (6, [0, 1, 2, 3, 5, 6]), (7, [0, 1, 2, 3, 4, 5, 6])):
        out, sel = oracle.decode_attn_topk(kv, q, 8, k)
        assert list(sel[0, 0]) == want, k


def test_permuting_positions_permutes_the_selection():
    B, H, D, L, k = 1, 2, 128, 23, 5
    kv, q = _fill(B, H, D, L, 16)
    base, sel = oracle.decode_attn_topk(kv, q, L, k)
    perm = np.random.default_rng(1).permutation(L)
    kv2 = oracle.KVCache(B, H, D, kv.cap)
    for a in ("k_codes", "k_meta", "v_codes", "v_meta"):
        getattr(kv2, a)[:, :, :L] = getattr(kv, a)[:, :, perm]
    got, sel2 = oracle.decode_attn_topk(kv2, q, L, k)
    assert np.allclose(got, base, rtol=1e-6, atol=1e-7)
    inv = np.argsort(perm)                             # old position -> new position
    assert np.array_equal(np.sort(inv[sel], axis=-1), sel2)


def test_kept_scores_dominate_dropped_scores():
    """On the long-context workload's heavy-tailed data: every kept fp32 score
    is >= every dropped one (fp64 scores of numpy's matmul rounded to fp32)."""
    w = synth.WORKLOADS["long-t3"]
    L = 300
    kv = oracle.KVCache(1, w.heads, w.head_dim, L)
    oracle.kv_append(kv, synth.prompt_kv(w, "k", nb=1, nt=L), synth.prompt_kv(w, "v", nb=1, nt=L), 0)
    q = synth.step_q(w, 1)[:1]
    k = 30
    _, sel = oracle.decode_attn_topk(kv, q, L, k)
    s32 = _scores64(kv, q, L).astype(np.float32)[0]
    for h in range(w.heads):
        keep = np.zeros(L, bool)
        keep[sel[0, h]] = True
        assert keep.sum() == k and np.all(np.diff(sel[0, h]) > 0)
        assert s32[h][keep].min() >= s32[h][~keep].max(), h


def test_rejects_nonpositive_top_k():
    kv, q = _fill(1, 1, 64, 4, 17)
    with pytest.raises(oracle.OracleError):
        oracle.decode_attn_topk(kv, q, 4, 0)
