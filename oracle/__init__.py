"""CPU oracle (ctypes wrapper around oracle.c).

TEST INFRASTRUCTURE: only the test suite, the smoke check of
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  It shares no code with the GPU library and imports nothing from it.

The arithmetic lives in ``oracle.c`` (see its header for the page citations and
the reading of the dropped quantisation formula); this file only marshals
numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

OK, ERR_SHAPE, ERR_NONFINITE = 0, -2, -9


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile liboracle.so in place: gcc -O2, no FMA contraction, no fast-math."""
    if force or not os.path.exists(_LIB_PATH):
        src = os.path.join(_HERE, "oracle.c")
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                               "-fPIC", "-shared", src, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f32.restype = ctypes.c_float
        lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_f16.restype = ctypes.c_uint16
        lib.oracle_quantize_g64.argtypes = [vp, i64, i64, i64, vp, vp]
        lib.oracle_dequant_g64.argtypes = [vp, vp, i64, i64, vp]
        lib.oracle_kv_append.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp]
        lib.oracle_decode_attn.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, i32, dbl, vp]
        lib.oracle_dequant_gemm.argtypes = [vp, i32, i32, i64, i64, vp, vp, vp]
        lib.oracle_decode_attn_topk.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, i32, i32, dbl, vp, vp]
        lib.oracle_prefill_attn.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, dbl, vp]
        lib.oracle_decode_attn_gqa.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, i32, dbl, vp]
        for f in (lib.oracle_quantize_g64, lib.oracle_dequant_g64, lib.oracle_kv_append,
                  lib.oracle_decode_attn, lib.oracle_dequant_gemm, lib.oracle_decode_attn_topk,
                  lib.oracle_prefill_attn, lib.oracle_decode_attn_gqa):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != OK:
        raise OracleError("%s failed with code %d" % (what, rc))


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def f16_to_f32(bits: int) -> float:
    return float(_load().oracle_f16_to_f32(bits))


def f32_to_f16(x: float) -> int:
    return int(_load().oracle_f32_to_f16(x))


def quantize_g64(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """fp16 [rows][cols] -> (codes u8 [rows][cols/2], meta u32 [rows][cols/64])."""
    x = _c(x, np.float16)
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 2), np.uint8)
    meta = np.zeros((rows, cols // 64), np.uint32)
    _check(_load().oracle_quantize_g64(x.ctypes.data, rows, cols, cols, codes.ctypes.data, meta.ctypes.data),
           "quantize_g64")
    return codes, meta


def dequant_g64(codes: np.ndarray, meta: np.ndarray) -> np.ndarray:
    """(codes, meta) -> fp32 [rows][cols] reconstruction."""
    codes = _c(codes, np.uint8)
    meta = _c(meta, np.uint32)
    rows, half = codes.shape
    out = np.zeros((rows, half * 2), np.float32)
    _check(_load().oracle_dequant_g64(codes.ctypes.data, meta.ctypes.data, rows, half * 2, out.ctypes.data),
           "dequant_g64")
    return out


class KVCache:
    """Head-major compressed cache: codes [B][H][cap][D/2], meta [B][H][cap][D/64]."""

    def __init__(self, batch: int, heads: int, head_dim: int, cap: int):
        self.batch, self.heads, self.head_dim, self.cap = batch, heads, head_dim, cap
        self.k_codes = np.zeros((batch, heads, cap, head_dim // 2), np.uint8)
        self.v_codes = np.zeros((batch, heads, cap, head_dim // 2), np.uint8)
        self.k_meta = np.zeros((batch, heads, cap, head_dim // 64), np.uint32)
        self.v_meta = np.zeros((batch, heads, cap, head_dim // 64), np.uint32)


def kv_append(kv: KVCache, k_new: np.ndarray, v_new: np.ndarray, pos: int) -> None:
    """k_new, v_new fp16 [B][n_new][H*D]; writes cache positions [pos, pos+n_new)."""
    k_new = _c(k_new, np.float16)
    v_new = _c(v_new, np.float16)
    b, n_new, h = k_new.shape
    assert b == kv.batch and h == kv.heads * kv.head_dim and v_new.shape == k_new.shape
    _check(_load().oracle_kv_append(k_new.ctypes.data, v_new.ctypes.data, kv.batch, kv.heads, kv.head_dim,
                                    kv.cap, pos, n_new, kv.k_codes.ctypes.data, kv.k_meta.ctypes.data,
                                    kv.v_codes.ctypes.data, kv.v_meta.ctypes.data), "kv_append")


def decode_attn(kv: KVCache, q: np.ndarray, kv_len: int, scale: float = 0.0) -> np.ndarray:
    """q fp16 [B][H*D] -> fp32 [B][H*D]; scale <= 0 means 1/sqrt(D)."""
    q = _c(q, np.float16)
    if scale <= 0.0:
        scale = 1.0 / np.sqrt(kv.head_dim)
    out = np.zeros((kv.batch, kv.heads * kv.head_dim), np.float32)
    _check(_load().oracle_decode_attn(q.ctypes.data, kv.batch, kv.heads, kv.head_dim, kv.cap,
                                      kv.k_codes.ctypes.data, kv.k_meta.ctypes.data,
                                      kv.v_codes.ctypes.data, kv.v_meta.ctypes.data,
                                      kv_len, float(scale), out.ctypes.data), "decode_attn")
    return out


def decode_attn_gqa(kv: KVCache, q: np.ndarray, q_heads: int, kv_len: int, scale: float = 0.0) -> np.ndarray:
    """Grouped-query decode attention: the cache holds kv.heads K/V heads, q
    fp16 [B][q_heads*D] -> fp32 [B][q_heads*D]; query head hq reads cache head
    hq // (q_heads // kv.heads).  scale <= 0 means 1/sqrt(D)."""
    q = _c(q, np.float16)
    if scale <= 0.0:
        scale = 1.0 / np.sqrt(kv.head_dim)
    assert q.shape == (kv.batch, q_heads * kv.head_dim)
    out = np.zeros((kv.batch, q_heads * kv.head_dim), np.float32)
    _check(_load().oracle_decode_attn_gqa(q.ctypes.data, kv.batch, q_heads, kv.heads, kv.head_dim, kv.cap,
                                          kv.k_codes.ctypes.data, kv.k_meta.ctypes.data,
                                          kv.v_codes.ctypes.data, kv.v_meta.ctypes.data,
                                          kv_len, float(scale), out.ctypes.data), "decode_attn_gqa")
    return out


def decode_attn_topk(kv: KVCache, q: np.ndarray, kv_len: int, top_k: int, scale: float = 0.0):
    """Top-K sparse decode attention: q fp16 [B][H*D] -> (fp32 [B][H*D], kept
    positions int32 [B][H][min(top_k, kv_len)] ascending); scale <= 0 means 1/sqrt(D)."""
    q = _c(q, np.float16)
    if scale <= 0.0:
        scale = 1.0 / np.sqrt(kv.head_dim)
    out = np.zeros((kv.batch, kv.heads * kv.head_dim), np.float32)
    sel = np.zeros((kv.batch, kv.heads, max(min(top_k, kv_len), 0)), np.int32)
    _check(_load().oracle_decode_attn_topk(q.ctypes.data, kv.batch, kv.heads, kv.head_dim, kv.cap,
                                           kv.k_codes.ctypes.data, kv.k_meta.ctypes.data,
                                           kv.v_codes.ctypes.data, kv.v_meta.ctypes.data,
                                           kv_len, top_k, float(scale), out.ctypes.data, sel.ctypes.data),
           "decode_attn_topk")
    return out, sel


def prefill_attn(q: np.ndarray, k: np.ndarray, v: np.ndarray, heads: int, scale: float = 0.0,
                 rows=None) -> np.ndarray:
    """Causal prefill attention over fp16 q, k, v [B][s][H*D] -> fp32 [B][s][H*D];
    only query rows [rows[0], rows[1]) are computed (others are NaN).
    scale <= 0 means 1/sqrt(D)."""
    q, k, v = _c(q, np.float16), _c(k, np.float16), _c(v, np.float16)
    B, s, h = q.shape
    assert k.shape == q.shape and v.shape == q.shape and h % heads == 0
    D = h // heads
    if scale <= 0.0:
        scale = 1.0 / np.sqrt(D)
    r0, r1 = (0, s) if rows is None else rows
    out = np.full((B, s, h), np.nan, np.float32)
    _check(_load().oracle_prefill_attn(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, s, heads, D, r0, r1,
                                       float(scale), out.ctypes.data), "prefill_attn")
    return out


def dequant_gemm(x: np.ndarray, g: int, m: int, codes: np.ndarray, meta: np.ndarray) -> np.ndarray:
    """x fp16 [g*m][K], W codes [K][N/2] + meta [K][N/64] -> Y fp32 [g*m][N]."""
    x = _c(x, np.float16)
    codes = _c(codes, np.uint8)
    meta = _c(meta, np.uint32)
    M, K = x.shape
    assert M == g * m and codes.shape[0] == K
    N = codes.shape[1] * 2
    y = np.zeros((M, N), np.float32)
    _check(_load().oracle_dequant_gemm(x.ctypes.data, g, m, K, N, codes.ctypes.data, meta.ctypes.data,
                                       y.ctypes.data), "dequant_gemm")
    return y
