"""Helpers for the GPU parity tests: device allocation, calls through the C
ABI (via the package's ctypes binding) and the comparison metrics."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import int4_group_quantized_fgq_amd as fgq

ATOL = 1e-2     # max |gpu - oracle|
RTOL_L2 = 1e-3  # ||gpu - oracle||_2 / ||oracle||_2


def note(msg: str) -> None:
    print("[gpu] " + msg, flush=True)
    sys.stdout.flush()


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fgq.load()   # fail loudly if the HIP library is missing
    return torch


def to_dev(a: np.ndarray):
    torch = torch_cuda()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to("cuda")


def to_host(t, dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def metrics(gpu: np.ndarray, ref: np.ndarray):
    g = gpu.astype(np.float64)
    r = ref.astype(np.float64)
    max_abs = float(np.max(np.abs(g - r))) if g.size else 0.0
    nr = float(np.linalg.norm(r))
    rel = float(np.linalg.norm(g - r) / nr) if nr > 0 else float(np.linalg.norm(g - r))
    return max_abs, rel


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str) -> None:
    assert np.all(np.isfinite(gpu)), what + ": non-finite output"
    max_abs, rel = metrics(gpu, ref)
    note("%s: max_abs=%.3e rel_l2=%.3e" % (what, max_abs, rel))
    assert max_abs <= ATOL and rel <= RTOL_L2, (what, max_abs, rel)


# --------------------------------------------------------------------------- calls

def quantize(x16: np.ndarray, ld: int = None):
    """fp16 [rows][cols] host array -> (codes u8, meta u32) host arrays, via the GPU."""
    torch = torch_cuda()
    rows, cols = x16.shape
    xd = to_dev(x16)
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
    meta = torch.empty((rows, cols // 64), dtype=torch.int32, device="cuda")
    fgq.fgq_quantize_g64(xd, rows, cols, cols if ld is None else ld, codes, meta)
    torch.cuda.synchronize()
    return to_host(codes), to_host(meta, np.uint32)


class DevKV:
    def __init__(self, batch, heads, head_dim, cap):
        torch = torch_cuda()
        self.batch, self.heads, self.head_dim, self.cap = batch, heads, head_dim, cap
        self.k_codes = torch.zeros((batch, heads, cap, head_dim // 2), dtype=torch.uint8, device="cuda")
        self.v_codes = torch.zeros_like(self.k_codes)
        self.k_meta = torch.zeros((batch, heads, cap, head_dim // 64), dtype=torch.int32, device="cuda")
        self.v_meta = torch.zeros_like(self.k_meta)
        self.struct = fgq.kv_struct(self.k_codes, self.v_codes, self.k_meta, self.v_meta, batch, heads, head_dim,
                                    cap)

    def append(self, k16: np.ndarray, v16: np.ndarray, pos: int):
        kd, vd = to_dev(k16), to_dev(v16)
        fgq.fgq_kv_append(self.struct, kd, vd, pos, k16.shape[1])

    def attend(self, q16: np.ndarray, kv_len: int, scale: float = 0.0, out_f16: bool = False):
        torch = torch_cuda()
        qd = to_dev(q16)
        out = torch.empty((self.batch, self.heads * self.head_dim),
                          dtype=torch.float16 if out_f16 else torch.float32, device="cuda")
        wsb = fgq.fgq_decode_attn_ws_bytes(self.batch, self.heads, self.head_dim, kv_len)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
        fgq.fgq_decode_attn_q4kv(self.struct, qd, kv_len, scale, out,
                                 fgq.FGQ_DTYPE_F16 if out_f16 else fgq.FGQ_DTYPE_F32, ws, wsb)
        torch.cuda.synchronize()
        return to_host(out).astype(np.float32)

    def attend_gqa(self, q16: np.ndarray, q_heads: int, kv_len: int, scale: float = 0.0, out_f16: bool = False):
        """Grouped-query attention: q fp16 [B][q_heads*D] over this cache's K/V heads -> fp32 [B][q_heads*D]."""
        torch = torch_cuda()
        qd = to_dev(q16)
        out = torch.empty((self.batch, q_heads * self.head_dim),
                          dtype=torch.float16 if out_f16 else torch.float32, device="cuda")
        wsb = fgq.fgq_decode_attn_gqa_ws_bytes(self.batch, q_heads, self.heads, self.head_dim, kv_len)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
        fgq.fgq_decode_attn_gqa_q4kv(self.struct, qd, q_heads, kv_len, scale, out,
                                     fgq.FGQ_DTYPE_F16 if out_f16 else fgq.FGQ_DTYPE_F32, ws, wsb)
        torch.cuda.synchronize()
        return to_host(out).astype(np.float32)

    def attend_topk(self, q16: np.ndarray, kv_len: int, top_k: int, scale: float = 0.0, out_f16: bool = False,
                    want_sel: bool = True):
        """Top-K sparse attention -> (fp32 [B][H*D], kept positions int32 [B][H][kk] or None)."""
        torch = torch_cuda()
        qd = to_dev(q16)
        out = torch.empty((self.batch, self.heads * self.head_dim),
                          dtype=torch.float16 if out_f16 else torch.float32, device="cuda")
        kk = min(top_k, kv_len)
        sel = torch.full((self.batch, self.heads, kk), -1, dtype=torch.int32, device="cuda") if want_sel else None
        fgq.fgq_decode_attn_topk_q4kv(self.struct, qd, kv_len, top_k, scale, out,
                                      fgq.FGQ_DTYPE_F16 if out_f16 else fgq.FGQ_DTYPE_F32, sel)
        torch.cuda.synchronize()
        return to_host(out).astype(np.float32), (to_host(sel) if want_sel else None)

    def host(self):
        return {a: to_host(getattr(self, a), np.uint32 if "meta" in a else None)
                for a in ("k_codes", "k_meta", "v_codes", "v_meta")}


def pack(codes_d, meta_d, K, N):
    torch = torch_cuda()
    pc = torch.empty(K * N // 8, dtype=torch.int32, device="cuda")
    pm = torch.empty(fgq.fgq_pack_weight_meta_words(K, N), dtype=torch.int32, device="cuda")
    fgq.fgq_pack_weight_g64(codes_d, meta_d, K, N, pc, pm)
    return pc, pm


def gemm(x16: np.ndarray, g: int, m: int, pc, pm, K: int, N: int, y_f16: bool = False, xd=None):
    """Block GEMM over the packed layout (fgq_dequant_gemm_packed)."""
    torch = torch_cuda()
    M = g * m
    xd = to_dev(x16) if xd is None else xd
    y = torch.empty((M, N), dtype=torch.float16 if y_f16 else torch.float32, device="cuda")
    wsb = fgq.fgq_dequant_gemm_ws_bytes(M, K, N)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    fgq.fgq_dequant_gemm_packed(xd, g, m, K, N, pc, pm, y, fgq.FGQ_DTYPE_F16 if y_f16 else fgq.FGQ_DTYPE_F32, ws,
                                wsb)
    torch.cuda.synchronize()
    return to_host(y).astype(np.float32)


def gemm_canonical(x16: np.ndarray, g: int, m: int, codes_d, meta_d, K: int, N: int, y_f16: bool = False, xd=None):
    """Block GEMM straight from the quantiser's codes [K][N/2] and meta [K][N/64] (fgq_dequant_gemm)."""
    torch = torch_cuda()
    M = g * m
    xd = to_dev(x16) if xd is None else xd
    y = torch.empty((M, N), dtype=torch.float16 if y_f16 else torch.float32, device="cuda")
    wsb = fgq.fgq_dequant_gemm_ws_bytes(M, K, N)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    fgq.fgq_dequant_gemm(xd, g, m, K, N, codes_d, meta_d, y, fgq.FGQ_DTYPE_F16 if y_f16 else fgq.FGQ_DTYPE_F32, ws,
                         wsb)
    torch.cuda.synchronize()
    return to_host(y).astype(np.float32)


def _scale_f16_bits(h: np.ndarray, s: np.ndarray) -> np.ndarray:
    """fp16 bit patterns times 2^s (per element), rounded to fp16 (numpy's
    float32 -> float16 conversion rounds to nearest even)."""
    f = h.astype(np.uint16).view(np.float16).astype(np.float32) * np.exp2(s.astype(np.float32))
    return f.astype(np.float16).view(np.uint16).astype(np.uint32)


def pack_reference(codes: np.ndarray, meta: np.ndarray):
    """The packed layout of include/fgq.h, built with numpy: a re-layout of
    the stored codes, and the stored steps and minima times the powers of two
    the header defines (per column group g the smallest e >= 0 with
    max_k step * 2^(24-e) <= 65504), followed by the exponents."""
    K, half = codes.shape
    N = half * 2
    q = np.zeros((K, N), np.uint32)
    q[:, 0::2] = codes & 15
    q[:, 1::2] = codes >> 4
    kc_n, g_n = K // 32, N // 64
    lane = np.arange(64)
    out = np.zeros((kc_n, g_n, 64, 4), np.uint32)
    slot_of = [0, 4, 1, 5, 2, 6, 3, 7]
    for j in range(4):
        n = (np.arange(g_n)[:, None] * 64 + 16 * j + (lane % 16)[None, :])          # [g][lane]
        for i in range(8):
            k = (np.arange(kc_n)[:, None] * 32 + 8 * (lane // 16)[None, :] + i)     # [kc][lane]
            vals = q[k[:, None, :], n[None, :, :]]                                   # [kc][g][lane]
            out[:, :, :, j] |= vals << np.uint32(4 * slot_of[i])
    mins = (meta & 0xFFFF).astype(np.uint32)
    steps = (meta >> 16).astype(np.uint32)
    max_step = steps.astype(np.uint16).view(np.float16).astype(np.float64).max(axis=0)   # [g]
    e = np.zeros(g_n, np.int64)
    for g in range(g_n):
        while e[g] < 24 and max_step[g] * 2.0 ** (24 - e[g]) > 65504.0:
            e[g] += 1
    pm = np.zeros((kc_n, g_n, 4, 8), np.uint32)
    for kq in range(4):
        for t in range(4):
            k = np.arange(kc_n) * 32 + 8 * kq + 2 * t
            sh = np.broadcast_to((24 if t % 2 == 0 else 20) - e, (kc_n, g_n))
            pm[:, :, kq, t] = _scale_f16_bits(steps[k, :], sh) | (_scale_f16_bits(steps[k + 1, :], sh) << np.uint32(16))
            sm = np.broadcast_to(-e, (kc_n, g_n))
            pm[:, :, kq, t + 4] = _scale_f16_bits(mins[k, :], sm) | (_scale_f16_bits(mins[k + 1, :], sm) << np.uint32(16))
    return out.reshape(-1), np.concatenate([pm.reshape(-1), e.astype(np.uint32)])
