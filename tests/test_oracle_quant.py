"""Pins of the oracle's quantiser, fp16 conversion and reconstruction.

Each test checks the oracle against something other than itself: exact integer
arithmetic, hand-worked fixtures, numpy's IEEE conversion, closed forms and
invariants of the min-max group quantiser (FlexGen review on jaehun.me,
section "Is 4-bit compression the same as integer-arithmetic acceleration?",
paper section 5; FlexGen review on blog.gzher.com, section 3.4).
"""
import functools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def unpack(codes: np.ndarray) -> np.ndarray:
    q = np.zeros(codes.shape[:-1] + (codes.shape[-1] * 2,), np.int64)
    q[..., 0::2] = codes & 15
    q[..., 1::2] = codes >> 4
    return q


def exact_codes(x16: np.ndarray):
    """Codes of the min-max reading in exact integer arithmetic.

    fp16 values are integer multiples of 2^-24, so with X = x * 2^24 the scaled
    offset 15 (x - a) / (b - a) is the exact rational 15 (X - A) / (B - A);
    round half to even is taken on that rational.  Returns (codes, num, den).
    """
    X = (x16.astype(np.float64) * 2.0 ** 24).astype(np.int64)
    X = X.reshape(-1, 64)
    A = X.min(axis=1, keepdims=True)
    B = X.max(axis=1, keepdims=True)
    den = np.where(B > A, B - A, 1)
    num = 15 * (X - A)
    q0 = num // den
    r = num - q0 * den
    up = (2 * r > den) | ((2 * r == den) & (q0 % 2 == 1))
    q = np.where(B > A, q0 + up, 0)
    return q, num, den


# ---------------------------------------------------------------- fp16 format

def test_f16_to_f32_all_patterns_match_numpy():
    lib = oracle._load()
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([lib.oracle_f16_to_f32(int(b)) for b in bits], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_f16_rne_matches_numpy_on_ties_and_random_patterns():
    lib = oracle._load()
    finite = np.arange(65536, dtype=np.uint16).view(np.float16)
    finite = finite[np.isfinite(finite)].astype(np.float64)
    vals = np.sort(np.unique(finite))
    mids = (vals[:-1] + vals[1:]) / 2.0           # exact ties between neighbours
    mids = mids.astype(np.float32)
    near = np.concatenate([np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf))])
    rng = np.random.default_rng(7)
    rand = rng.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    edge = np.array([65504.0, 65519.99, 65520.0, 65536.0, 1e9, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
                     2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, -0.0, 0.0, np.inf, -np.inf], np.float32)
    xs = np.concatenate([vals.astype(np.float32), mids, near, rand, edge])
    xs = xs[~np.isnan(xs)]
    ref = xs.astype(np.float16).view(np.uint16)
    got = np.array([lib.oracle_f32_to_f16(float(v)) for v in xs], np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(xs[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


# ---------------------------------------------------------------- worked fixtures

def test_tie_ladders_fixture():
    spec = json.load(open(os.path.join(GOLDEN, "tie_ladders.json")))
    for grp in spec["groups"]:
        head = grp["head"]
        x = np.array([head + [grp["pad"]] * (64 - len(head))], np.float16)
        codes, meta = oracle.quantize_g64(x)
        q = unpack(codes)[0]
        assert q[: len(head)].tolist() == grp["codes_head"], grp["name"]
        assert np.all(q[len(head):] == 0)
        assert int(meta[0, 0]) & 0xFFFF == int(grp["min_h"], 16), grp["name"]
        assert int(meta[0, 0]) >> 16 == int(grp["step_h"], 16), grp["name"]


def test_nibble_order_low_nibble_is_even_element():
    x = np.zeros((1, 64), np.float16)
    x[0, 1] = 15.0   # odd element at the max, even elements at the min
    codes, meta = oracle.quantize_g64(x)
    assert codes[0, 0] == 0xF0
    assert np.all(codes[0, 1:] == 0)


# ---------------------------------------------------------------- exact arithmetic

@functools.lru_cache(maxsize=None)
def _sample_tensors():
    out = []
    for name in ("tiny", "opt-6.7b", "long-t3"):
        w = synth.WORKLOADS[name]
        k = synth.prompt_kv(w, "k", nb=1, nt=min(w.prompt, 256))
        out.append((name + ":k", k.reshape(-1, w.hidden)))
        out.append((name + ":q", synth.step_q(w, 1)))
        if w.weights:
            out.append((name + ":w", synth.weight(w, len(w.weights) - 1, rows=(0, 16))))
    return out


@pytest.mark.parametrize("idx", range(8))
def test_codes_equal_exact_rational_rounding(idx):
    tensors = _sample_tensors()
    if idx >= len(tensors):
        pytest.skip("no tensor")
    name, x = tensors[idx]
    x = np.ascontiguousarray(x)
    codes, meta = oracle.quantize_g64(x)
    q = unpack(codes).reshape(-1, 64)
    qe, num, den = exact_codes(x)
    mism = np.nonzero(q != qe)
    # The fp32 sequence (x-a)/d*15 may only part from exact rounding at a
    # near-tie; on these draws none occurs.
    assert mism[0].size == 0, (name, mism[0].size)


def test_exact_ties_round_to_even_in_sampled_data():
    w = synth.WORKLOADS["opt-6.7b"]
    x = synth.prompt_kv(w, "k", nb=1, nt=800).reshape(-1, 64)
    qe, num, den = exact_codes(x)
    ties = (2 * (num % den) == den)
    assert ties.sum() > 0            # the data does exercise exact ties
    codes, _ = oracle.quantize_g64(x.reshape(-1, 64))
    q = unpack(codes).reshape(-1, 64)
    assert np.all(q[ties] % 2 == 0)
    assert np.array_equal(q[ties], qe[ties])


# ---------------------------------------------------------------- invariants

def _groups(seed=3, n=4000, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, 64)) * scale).astype(np.float16)


def test_endpoints_and_range():
    x = _groups()
    codes, _ = oracle.quantize_g64(x)
    q = unpack(codes)
    xf = x.astype(np.float32)
    assert np.all(q[np.arange(len(x)), xf.argmin(1)] == 0)
    assert np.all(q[np.arange(len(x)), xf.argmax(1)] == 15)
    assert q.min() >= 0 and q.max() <= 15


def test_monotone_within_group():
    x = _groups(5)
    codes, _ = oracle.quantize_g64(x)
    q = unpack(codes)
    order = np.argsort(x.astype(np.float32), axis=1, kind="stable")
    qs = np.take_along_axis(q, order, axis=1)
    assert np.all(np.diff(qs, axis=1) >= 0)


def test_meta_is_min_and_step():
    x = _groups(11)
    codes, meta = oracle.quantize_g64(x)
    xf = x.astype(np.float32)
    a, b = xf.min(1), xf.max(1)
    min_h = (meta[:, 0] & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float32)
    step_h = (meta[:, 0] >> 16).astype(np.uint16).view(np.float16)
    assert np.array_equal(min_h, a)
    expect = ((b - a) / np.float32(15.0)).astype(np.float32).astype(np.float16)
    assert np.array_equal(step_h.view(np.uint16), expect.view(np.uint16))


@pytest.mark.parametrize("name", ["tiny", "opt-6.7b", "long-t3"])
def test_reconstruction_bound(name):
    """|x - x^| <= (b-a)/30 with the exact step; with the stored fp16 step the
    error adds at most q * |step_h - (b-a)/15|."""
    w = synth.WORKLOADS[name]
    x = synth.prompt_kv(w, "k", nb=1, nt=min(w.prompt, 160)).reshape(-1, 64)
    codes, meta = oracle.quantize_g64(x)
    q = unpack(codes).astype(np.float64)
    xf = x.astype(np.float64)
    a, b = xf.min(1, keepdims=True), xf.max(1, keepdims=True)
    exact_step_err = np.abs(xf - (a + q * (b - a) / 15.0))
    assert np.all(exact_step_err <= (b - a) / 30.0 * (1 + 1e-6) + 1e-300)
    xhat = oracle.dequant_g64(codes.reshape(-1, 32), meta.reshape(-1, 1)).astype(np.float64)
    step_h = (meta >> 16).astype(np.uint16).view(np.float16).astype(np.float64).reshape(-1, 1)
    bound = (b - a) / 30.0 + q * np.abs(step_h - (b - a) / 15.0)
    assert np.all(np.abs(xf - xhat) <= bound * (1 + 1e-6) + 1e-7 * np.abs(xf))


def test_constant_group_is_exact():
    vals = np.array([0.0, -0.0, 1.5, -3.25, 65504.0, -65504.0, 6e-8, 2.0 ** -14], np.float16)
    x = np.repeat(vals[:, None], 64, axis=1)
    codes, meta = oracle.quantize_g64(x)
    assert np.all(codes == 0)
    assert np.all(meta >> 16 == 0)
    xhat = oracle.dequant_g64(codes, meta)
    assert np.array_equal(xhat.astype(np.float16).view(np.uint16)[:, 0],
                          (x[:, 0] + np.float16(0.0)).view(np.uint16))   # -0 stored as +0


def test_signed_zero_min_is_canonical():
    x = np.zeros((1, 64), np.float16)
    x[0, :32] = -0.0
    x[0, 40] = 2.0
    codes, meta = oracle.quantize_g64(x)
    assert int(meta[0, 0]) & 0xFFFF == 0x0000
    x2 = np.full((1, 64), -0.0, np.float16)
    _, meta2 = oracle.quantize_g64(x2)
    assert int(meta2[0, 0]) == 0


def test_on_grid_groups_reconstruct_exactly():
    rng = np.random.default_rng(1)
    for e in (-10, -3, 0, 2, 6):
        k = rng.integers(0, 16, (50, 64))
        k[:, 0], k[:, 1] = 0, 15
        x = ((k - 8) * 2.0 ** e).astype(np.float16)
        codes, meta = oracle.quantize_g64(x)
        assert np.array_equal(unpack(codes), k)
        xhat = oracle.dequant_g64(codes, meta)
        assert np.array_equal(xhat, x.astype(np.float32))


def test_step_underflow_keeps_codes():
    """b - a > 0 but (b - a)/15 below half the smallest fp16 subnormal: the codes
    are kept, the stored step is 0 and x^ = a, an error of at most b - a."""
    x = np.zeros((1, 64), np.float16)
    x[0, 1] = np.float16(2.0 ** -24)   # b - a = 2^-24, step 2^-24/15 rounds to 0
    codes, meta = oracle.quantize_g64(x)
    q = unpack(codes)[0]
    assert q[1] == 15 and q[0] == 0
    assert int(meta[0, 0]) >> 16 == 0
    xhat = oracle.dequant_g64(codes, meta)
    assert np.all(xhat == 0.0)


def test_dequant_is_min_plus_code_times_step_rounded_once():
    x = _groups(17, 300)
    codes, meta = oracle.quantize_g64(x)
    xhat = oracle.dequant_g64(codes, meta)
    q = unpack(codes)
    for r in range(0, 300, 37):
        mn = Fraction(float(np.uint16(meta[r, 0] & 0xFFFF).view(np.float16)))
        st = Fraction(float(np.uint16(meta[r, 0] >> 16).view(np.float16)))
        for c in range(64):
            exact = mn + int(q[r, c]) * st
            assert float(np.float32(float(exact))) == float(xhat[r, c]) or \
                abs(Fraction(float(xhat[r, c])) - exact) <= abs(exact) * Fraction(1, 2 ** 24)


def test_rejects_nonfinite_and_bad_shape():
    x = np.zeros((2, 64), np.float16)
    x[1, 5] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.quantize_g64(x)
    with pytest.raises(oracle.OracleError):
        oracle.quantize_g64(np.zeros((2, 96), np.float16))
