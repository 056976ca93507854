"""int4 group-wise (g=64) compressed decode path for MI355X (gfx950).

Thin ctypes binding over libfgq.so (the C ABI declared in include/fgq.h).
The functions keep the C names and only marshal arguments: torch tensors
(device memory) become pointers, the current torch stream becomes the HIP
stream.  Every step of the path runs in the library's HIP kernels; when the
library is missing, loading it raises instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfgq.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "fgq.h")

FGQ_OK = 0
FGQ_ERR_INVALID_ARG = -1
FGQ_ERR_SHAPE = -2
FGQ_ERR_ALIGN = -3
FGQ_ERR_CAPACITY = -4
FGQ_ERR_WORKSPACE = -5
FGQ_ERR_DTYPE = -6
FGQ_ERR_DEVICE = -7
FGQ_ERR_UNSUPPORTED = -8
FGQ_DTYPE_F32 = 0
FGQ_DTYPE_F16 = 1
FGQ_NOALLOC_SCRATCH_BYTES = 9 << 20
FGQ_GQA_MAX_GROUP = 32
FGQ_TOPK_MAX_POSITIONS = 65536

_lib = None


class FgqError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str):
        super().__init__("%s failed: %s (%d): %s" % (what, status_string(status), status, detail))
        self.status = status


class fgq_kv_cache(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("k_meta", ctypes.c_void_p), ("v_meta", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("capacity", ctypes.c_int32)]


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libfgq.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError("libfgq.so is not built (%s); run __graft_entry__.build() or "
                           "python int4_group_quantized_fgq_amd/build.py" % path)
    lib = declare(ctypes.CDLL(path))
    _lib = lib
    return lib


def declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    """Set the argument and result types of every entry point on a loaded
    copy of the library."""
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    kvp = ctypes.POINTER(fgq_kv_cache)
    sig = {
        "fgq_abi_version": ([], i32),
        "fgq_status_string": ([i32], ctypes.c_char_p),
        "fgq_last_error": ([], ctypes.c_char_p),
        "fgq_quantize_g64": ([vp, i64, i64, i64, vp, vp, vp], i32),
        "fgq_kv_append": ([kvp, vp, vp, i32, i32, vp], i32),
        "fgq_kv_append_ld": ([kvp, vp, vp, i64, i32, i32, vp], i32),
        "fgq_decode_attn_ws_bytes": ([i32, i32, i32, i32], sz),
        "fgq_decode_attn_q4kv": ([kvp, vp, i32, f32, vp, i32, vp, sz, vp], i32),
        "fgq_decode_attn_q4kv_ld": ([kvp, vp, i64, i32, f32, vp, i32, vp, sz, vp], i32),
        "fgq_decode_attn_q4kv_noalloc": ([kvp, vp, i32, f32, vp, i32, vp], i32),
        "fgq_decode_attn_topk_q4kv": ([kvp, vp, i32, i32, f32, vp, i32, vp, vp], i32),
        "fgq_decode_attn_gqa_ws_bytes": ([i32, i32, i32, i32, i32], sz),
        "fgq_decode_attn_gqa_q4kv": ([kvp, vp, i32, i32, f32, vp, i32, vp, sz, vp], i32),
        "fgq_prefill_attn_f16": ([vp, vp, vp, i32, i32, i32, i32, f32, vp, i32, vp], i32),
        "fgq_pack_weight_meta_words": ([i64, i64], sz),
        "fgq_pack_weight_g64": ([vp, vp, i64, i64, vp, vp, vp], i32),
        "fgq_dequant_gemm_ws_bytes": ([i64, i64, i64], sz),
        "fgq_dequant_gemm": ([vp, i32, i32, i64, i64, vp, vp, vp, i32, vp, sz, vp], i32),
        "fgq_dequant_gemm_packed": ([vp, i32, i32, i64, i64, vp, vp, vp, i32, vp, sz, vp], i32),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


def declared_symbols(header: str = HEADER_PATH):
    """Names of the functions include/fgq.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fgq_[a-z0-9_]+)\s*\(", text)))


def status_string(s: int) -> str:
    return load().fgq_status_string(s).decode()


def last_error() -> str:
    return load().fgq_last_error().decode()


def _check(status: int, what: str) -> None:
    if status != FGQ_OK:
        raise FgqError(status, what, last_error())


def _ptr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def kv_struct(k_codes, v_codes, k_meta, v_meta, batch, heads, head_dim, capacity) -> fgq_kv_cache:
    return fgq_kv_cache(_ptr(k_codes), _ptr(v_codes), _ptr(k_meta), _ptr(v_meta), batch, heads, head_dim,
                        capacity)


# --------------------------------------------------------------------------- entry points

def fgq_abi_version() -> int:
    return load().fgq_abi_version()


def fgq_quantize_g64(x, rows, cols, ld_x, codes, meta, stream=None) -> None:
    _check(load().fgq_quantize_g64(_ptr(x), rows, cols, ld_x, _ptr(codes), _ptr(meta), _stream(stream)),
           "fgq_quantize_g64")


def fgq_kv_append(kv: fgq_kv_cache, k_new, v_new, pos, n_new, stream=None) -> None:
    _check(load().fgq_kv_append(ctypes.byref(kv), _ptr(k_new), _ptr(v_new), pos, n_new, _stream(stream)),
           "fgq_kv_append")


def fgq_kv_append_ld(kv: fgq_kv_cache, k_new, v_new, ld_new, pos, n_new, stream=None) -> None:
    _check(load().fgq_kv_append_ld(ctypes.byref(kv), _ptr(k_new), _ptr(v_new), ld_new, pos, n_new, _stream(stream)),
           "fgq_kv_append_ld")


def fgq_decode_attn_ws_bytes(batch, heads, head_dim, kv_len) -> int:
    return load().fgq_decode_attn_ws_bytes(batch, heads, head_dim, kv_len)


def fgq_decode_attn_q4kv(kv: fgq_kv_cache, q, kv_len, softmax_scale, out, out_dtype, ws, ws_bytes,
                         stream=None) -> None:
    _check(load().fgq_decode_attn_q4kv(ctypes.byref(kv), _ptr(q), kv_len, softmax_scale, _ptr(out), out_dtype,
                                       _ptr(ws), ws_bytes, _stream(stream)), "fgq_decode_attn_q4kv")


def fgq_decode_attn_q4kv_ld(kv: fgq_kv_cache, q, ld_q, kv_len, softmax_scale, out, out_dtype, ws, ws_bytes,
                            stream=None) -> None:
    _check(load().fgq_decode_attn_q4kv_ld(ctypes.byref(kv), _ptr(q), ld_q, kv_len, softmax_scale, _ptr(out),
                                          out_dtype, _ptr(ws), ws_bytes, _stream(stream)), "fgq_decode_attn_q4kv_ld")


def fgq_decode_attn_q4kv_noalloc(kv: fgq_kv_cache, q, kv_len, softmax_scale, out, out_dtype, stream=None) -> None:
    _check(load().fgq_decode_attn_q4kv_noalloc(ctypes.byref(kv), _ptr(q), kv_len, softmax_scale, _ptr(out),
                                               out_dtype, _stream(stream)), "fgq_decode_attn_q4kv_noalloc")


def fgq_decode_attn_gqa_ws_bytes(batch, q_heads, kv_heads, head_dim, kv_len) -> int:
    return load().fgq_decode_attn_gqa_ws_bytes(batch, q_heads, kv_heads, head_dim, kv_len)


def fgq_decode_attn_gqa_q4kv(kv: fgq_kv_cache, q, q_heads, kv_len, softmax_scale, out, out_dtype, ws, ws_bytes,
                             stream=None) -> None:
    _check(load().fgq_decode_attn_gqa_q4kv(ctypes.byref(kv), _ptr(q), q_heads, kv_len, softmax_scale, _ptr(out),
                                           out_dtype, _ptr(ws), ws_bytes, _stream(stream)),
           "fgq_decode_attn_gqa_q4kv")


def fgq_decode_attn_topk_q4kv(kv: fgq_kv_cache, q, kv_len, top_k, softmax_scale, out, out_dtype, sel=None,
                              stream=None) -> None:
    _check(load().fgq_decode_attn_topk_q4kv(ctypes.byref(kv), _ptr(q), kv_len, top_k, softmax_scale, _ptr(out),
                                            out_dtype, _ptr(sel), _stream(stream)), "fgq_decode_attn_topk_q4kv")


def fgq_prefill_attn_f16(q, k, v, batch, seq, heads, head_dim, softmax_scale, out, out_dtype, stream=None) -> None:
    _check(load().fgq_prefill_attn_f16(_ptr(q), _ptr(k), _ptr(v), batch, seq, heads, head_dim, softmax_scale,
                                       _ptr(out), out_dtype, _stream(stream)), "fgq_prefill_attn_f16")


def fgq_pack_weight_meta_words(K, N) -> int:
    return load().fgq_pack_weight_meta_words(K, N)


def fgq_pack_weight_g64(codes, meta, K, N, packed_codes, packed_meta, stream=None) -> None:
    _check(load().fgq_pack_weight_g64(_ptr(codes), _ptr(meta), K, N, _ptr(packed_codes), _ptr(packed_meta),
                                      _stream(stream)), "fgq_pack_weight_g64")


def fgq_dequant_gemm_ws_bytes(M, K, N) -> int:
    return load().fgq_dequant_gemm_ws_bytes(M, K, N)


def fgq_dequant_gemm(x, g, m, K, N, w_codes, w_meta, y, y_dtype, ws, ws_bytes, stream=None) -> None:
    _check(load().fgq_dequant_gemm(_ptr(x), g, m, K, N, _ptr(w_codes), _ptr(w_meta), _ptr(y), y_dtype,
                                   _ptr(ws), ws_bytes, _stream(stream)), "fgq_dequant_gemm")


def fgq_dequant_gemm_packed(x, g, m, K, N, packed_codes, packed_meta, y, y_dtype, ws, ws_bytes, stream=None) -> None:
    _check(load().fgq_dequant_gemm_packed(_ptr(x), g, m, K, N, _ptr(packed_codes), _ptr(packed_meta), _ptr(y),
                                          y_dtype, _ptr(ws), ws_bytes, _stream(stream)), "fgq_dequant_gemm_packed")
