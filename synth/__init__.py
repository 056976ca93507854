"""Seeded synthetic inputs for the int4 group-wise (g=64) decode path.

This module only draws numbers and arranges them into the shapes of the
workloads.  It holds none of the compression method's arithmetic, and both the
GPU library's tests/bench and the CPU oracle take their inputs from here.

The workloads follow the evaluation setup of the FlexGen pages (OPT-6.7B /
30B / 175B layer shapes, prompt 512 or 1024 then 32 generated tokens, dummy
weights for throughput runs; FlexGen review on blog.gzher.com, section 4 and
section 6; FlexGen review on jaehun.me, "single-GPU performance figures").
Values are drawn, never taken from a dataset.

Streams: every tensor is its own Philox4x32-10 stream whose key folds
(seed, config, tensor id, layer instance, step) through splitmix64; element i
of a stream is a pure function of (key, i), so windows can be drawn in any
order and the same bytes come out.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import List, Optional, Tuple

import numpy as np

SEED = 230306865  # master seed (the arXiv number of the FlexGen paper)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

# tensor ids of the streams
T_PROMPT_K, T_PROMPT_V, T_STEP_K, T_STEP_V, T_STEP_Q = 1, 2, 3, 4, 5
T_GEMM_X = 6      # + weight index
T_WEIGHT = 20     # + weight index
T_OUTLIER = 40
T_CONST_MASK = 41
T_PROMPT_Q = 42


def build(force: bool = True) -> str:
    """Compile libsynth.so in place (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        src = os.path.join(_HERE, "synth.c")
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.synth_stream_key.restype = u64
        lib.synth_stream_key.argtypes = [u64] * 5
        for f in (lib.synth_normal_f32, lib.synth_student_t3_f32):
            f.argtypes = [u64, u64, i64, dbl, vp]
            f.restype = None
        lib.synth_uniform_f64.argtypes = [u64, u64, i64, vp]
        lib.synth_uniform_f64.restype = None
        lib.synth_philox4x32_10.argtypes = [vp, vp, vp]
        lib.synth_philox4x32_10.restype = None
        _lib = lib
    return _lib


def philox4x32_10(ctr, key) -> List[int]:
    """One Philox4x32-10 block (exposed for known-answer tests)."""
    lib = _load()
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    lib.synth_philox4x32_10(c, k, o)
    return list(o)


def stream_key(cfg: int, tensor: int, layer: int = 0, step: int = 0, seed: int = SEED) -> int:
    return int(_load().synth_stream_key(seed, cfg, tensor, layer, step))


def normal(key: int, n: int, sigma: float = 1.0, first: int = 0) -> np.ndarray:
    out = np.empty(int(n), np.float32)
    if n:
        _load().synth_normal_f32(key, first, int(n), float(sigma), out.ctypes.data)
    return out


def student_t3(key: int, n: int, sigma: float = 1.0, first: int = 0) -> np.ndarray:
    out = np.empty(int(n), np.float32)
    if n:
        _load().synth_student_t3_f32(key, first, int(n), float(sigma), out.ctypes.data)
    return out


def uniform(key: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(int(n), np.float64)
    if n:
        _load().synth_uniform_f64(key, first, int(n), out.ctypes.data)
    return out


def to_f16(x: np.ndarray) -> np.ndarray:
    """Store as fp16, saturating at the largest finite fp16 magnitude (65504)."""
    return np.clip(x, -65504.0, 65504.0).astype(np.float16)


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic decode layer.

    batch = g * m is the effective batch (block) whose GPU batches share one
    load of each weight matrix; heads x head_dim = hidden; `prompt` tokens are
    bulk-appended, then `steps` decode steps each append one K/V token per
    sequence and attend over prompt + t positions.
    """
    cid: int
    name: str
    g: int
    m: int
    heads: int
    head_dim: int
    prompt: int
    steps: int
    weights: Tuple[Tuple[int, int], ...]   # (K = in, N = out) per matrix
    kv_dist: str = "normal"                 # "normal" or "t3"
    outlier_channels: int = 0
    outlier_scale: float = 1.0
    const_group_frac: float = 0.0
    weight_sigma: float = 0.02
    kv_heads: int = 0                       # K/V heads; 0 means one per query head

    @property
    def batch(self) -> int:
        return self.g * self.m

    @property
    def hidden(self) -> int:
        """Query width: heads * head_dim."""
        return self.heads * self.head_dim

    @property
    def n_kv_heads(self) -> int:
        return self.kv_heads or self.heads

    @property
    def kv_hidden(self) -> int:
        """Width of one token's K (or V) row: kv_heads * head_dim."""
        return self.n_kv_heads * self.head_dim

    @property
    def capacity(self) -> int:
        return self.prompt + self.steps

    def kv_len(self, t: int) -> int:
        """Attended length after appending decode step t (1-based)."""
        return self.prompt + t


def _opt_layer(h: int) -> Tuple[Tuple[int, int], ...]:
    # Wq, Wk, Wv, Wout (h x h) and the MLP pair h x 4h, 4h x h, stored [in][out].
    return ((h, h),) * 4 + ((h, 4 * h), (4 * h, h))


WORKLOADS = {
    "tiny": Workload(1, "tiny", g=4, m=1, heads=2, head_dim=64, prompt=128, steps=1,
                     weights=((128, 512),)),
    "opt-6.7b": Workload(2, "opt-6.7b", g=16, m=4, heads=32, head_dim=128, prompt=512, steps=32,
                         weights=_opt_layer(4096)),
    "opt-30b": Workload(3, "opt-30b", g=24, m=4, heads=56, head_dim=128, prompt=1024, steps=32,
                        weights=_opt_layer(7168)),
    "opt-175b": Workload(4, "opt-175b", g=36, m=4, heads=96, head_dim=128, prompt=512, steps=32,
                         weights=_opt_layer(12288)),
    "long-t3": Workload(5, "long-t3", g=32, m=1, heads=96, head_dim=128, prompt=4096, steps=32,
                        weights=(), kv_dist="t3", outlier_channels=8, outlier_scale=20.0,
                        const_group_frac=0.01),
    # Grouped-query decode attention at the shape of the vTensor page's
    # decode-kernel evaluation (section "Decoding kernel evaluation", Figure 7:
    # 16K cached positions, batch up to 32, 32 query heads with 32 down to 1
    # K/V heads): batch 16, 32 query heads x 128 sharing 8 K/V heads.
    "gqa": Workload(6, "gqa", g=16, m=1, heads=32, kv_heads=8, head_dim=128, prompt=16384, steps=32,
                    weights=()),
}


def outlier_channels(w: Workload, layer: int = 0) -> np.ndarray:
    """The `outlier_channels` distinct hidden channels scaled in K and V."""
    if w.outlier_channels == 0:
        return np.zeros(0, np.int64)
    key = stream_key(w.cid, T_OUTLIER, layer)
    chosen: List[int] = []
    first = 0
    while len(chosen) < w.outlier_channels:
        for u in uniform(key, 64, first):
            c = int(u * w.kv_hidden)
            if c not in chosen:
                chosen.append(c)
                if len(chosen) == w.outlier_channels:
                    break
        first += 64
    return np.array(sorted(chosen), np.int64)


def _kv_rows(w: Workload, tensor: int, layer: int, step: int, ntok_full: int,
             b0: int, nb: int, t0: int, nt: int) -> np.ndarray:
    """fp16 [nb][nt][kv_hidden]: batch rows b0.., tokens t0.. of a K or V stream
    whose full layout is [batch][ntok_full][kv_hidden]."""
    h = w.kv_hidden
    key = stream_key(w.cid, tensor, layer, step)
    draw = student_t3 if w.kv_dist == "t3" else normal
    x = np.empty((nb, nt, h), np.float32)
    for i in range(nb):
        first = ((b0 + i) * ntok_full + t0) * h
        x[i] = draw(key, nt * h, 1.0, first).reshape(nt, h)
    if w.outlier_channels:
        x[:, :, outlier_channels(w, layer)] *= np.float32(w.outlier_scale)
    x16 = to_f16(x)
    if w.const_group_frac > 0.0:
        ng = h // 64
        mkey = stream_key(w.cid, T_CONST_MASK, layer, (tensor << 8) | step)
        u = np.empty((nb, nt, ng), np.float64)
        for i in range(nb):
            u[i] = uniform(mkey, nt * ng, ((b0 + i) * ntok_full + t0) * ng).reshape(nt, ng)
        g16 = x16.reshape(nb, nt, ng, 64)
        sel = u < w.const_group_frac
        g16[sel] = g16[sel][:, :1]
    return x16


def prompt_kv(w: Workload, which: str, layer: int = 0, b0: int = 0, nb: Optional[int] = None,
              t0: int = 0, nt: Optional[int] = None) -> np.ndarray:
    """Prompt K (which='k') or V ('v'): fp16 [nb][nt][kv_hidden], token-major;
    defaults cover every sequence and every prompt token."""
    nb = w.batch - b0 if nb is None else nb
    nt = w.prompt - t0 if nt is None else nt
    tid = T_PROMPT_K if which == "k" else T_PROMPT_V
    return _kv_rows(w, tid, layer, 0, w.prompt, b0, nb, t0, nt)


def step_kv(w: Workload, which: str, t: int, layer: int = 0) -> np.ndarray:
    """K or V of decode step t (1-based): fp16 [batch][1][kv_hidden]."""
    tid = T_STEP_K if which == "k" else T_STEP_V
    return _kv_rows(w, tid, layer, t, 1, 0, w.batch, 0, 1)


def step_q(w: Workload, t: int, layer: int = 0) -> np.ndarray:
    """Query of decode step t: fp16 [batch][hidden], N(0, 1)."""
    key = stream_key(w.cid, T_STEP_Q, layer, t)
    return to_f16(normal(key, w.batch * w.hidden)).reshape(w.batch, w.hidden)


def prompt_q(w: Workload, layer: int = 0, b0: int = 0, nb: Optional[int] = None) -> np.ndarray:
    """Queries of the prompt tokens (prefill): fp16 [nb][prompt][hidden], N(0, 1)."""
    nb = w.batch - b0 if nb is None else nb
    key = stream_key(w.cid, T_PROMPT_Q, layer)
    n = w.prompt * w.hidden
    x = np.empty((nb, w.prompt, w.hidden), np.float32)
    for i in range(nb):
        x[i] = normal(key, n, 1.0, (b0 + i) * n).reshape(w.prompt, w.hidden)
    return to_f16(x)


def weight(w: Workload, idx: int, layer: int = 0, rows: Optional[Tuple[int, int]] = None) -> np.ndarray:
    """Weight matrix idx: fp16 [K][N] ~ N(0, weight_sigma); `rows` selects a K-window."""
    K, N = w.weights[idx]
    r0, r1 = (0, K) if rows is None else rows
    key = stream_key(w.cid, T_WEIGHT + idx, layer)
    return to_f16(normal(key, (r1 - r0) * N, w.weight_sigma, r0 * N)).reshape(r1 - r0, N)


def gemm_x(w: Workload, idx: int, t: int, layer: int = 0) -> np.ndarray:
    """Activations entering weight idx at decode step t: fp16 [g*m][K] ~ N(0, 1)."""
    K, _ = w.weights[idx]
    key = stream_key(w.cid, T_GEMM_X + idx, layer, t)
    return to_f16(normal(key, w.batch * K)).reshape(w.batch, K)
