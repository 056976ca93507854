"""Algorithmic byte and flop counts of the decode path (the roofline numerators).

Counts what the method itself must move or compute, not what an implementation
happens to move:

* a compressed element costs 4 bits of code plus, per group of 64, an fp16
  minimum and an fp16 step: 0.5 + 4/64 = 0.5625 bytes (FlexGen review on
  jaehun.me, "Is 4-bit compression the same as integer-arithmetic
  acceleration?": the ideal 16-to-4-bit ratio differs from the real saving once
  the per-group metadata is counted);
* one decode step of attention reads every cached K and V position of every
  sequence once (paper-graph-ui FlexGen summary, section 3.4, "Computation
  delegation": the KV cache of one layer is 4*b*s*h1 bytes in FP16);
* the weight GEMM of one block reads each weight once for all g*m rows
  (paper-graph-ui FlexGen summary, section 3.4, "Compute Schedule"), and costs
  2*M*K*N flops.
"""
from __future__ import annotations

GROUP = 64
CODE_BYTES_PER_ELEM = 0.5
META_BYTES_PER_GROUP = 4          # fp16 min + fp16 step
PACKED_BYTES_PER_ELEM = CODE_BYTES_PER_ELEM + META_BYTES_PER_GROUP / GROUP   # 0.5625


def packed_bytes(n_elems: int) -> float:
    return n_elems * PACKED_BYTES_PER_ELEM


# --- the pages' fp16 byte model (FlexGen cost model, dtoc_g and cpu_comp_g terms)

def fp16_weight_bytes_per_layer(h1: int, h2: int) -> int:
    """8*h1^2 + 4*h1*h2: four h1 x h1 attention matrices and the h1 x h2 MLP pair."""
    return 8 * h1 * h1 + 4 * h1 * h2


def fp16_kv_bytes_per_layer(batch: int, seq: int, h1: int) -> int:
    """4*b*s*h1: keys and values, 2 bytes each."""
    return 4 * batch * seq * h1


def weight_transfer_bytes(layers: int, bytes_per_layer: float, gpu_batches: int, reuse: bool) -> float:
    """Weight bytes one generation step moves: once per GPU batch without block
    reuse, once per block with it."""
    return layers * bytes_per_layer * (1 if reuse else gpu_batches)


# --- this path's per-kernel algorithmic work

def attention_bytes(batch: int, hidden: int, kv_len: int, out_bytes: int = 4) -> float:
    """Compressed K and V over kv_len positions for every sequence (1.125*h per
    position), plus the fp16 query and the output row."""
    return 2 * packed_bytes(batch * hidden * kv_len) + batch * hidden * (2 + out_bytes)


def gqa_attention_bytes(batch: int, q_heads: int, kv_heads: int, head_dim: int, kv_len: int,
                        out_bytes: int = 4) -> float:
    """Grouped-query attention: the compressed K and V of the kv_heads cache
    heads over kv_len positions (read once for the whole group of query heads),
    plus the fp16 queries and the outputs of all q_heads."""
    return 2 * packed_bytes(batch * kv_heads * head_dim * kv_len) + batch * q_heads * head_dim * (2 + out_bytes)


def gqa_attention_flops(batch: int, q_heads: int, head_dim: int, kv_len: int) -> float:
    """q.k and p*v for every query head: two multiply-adds per cached element per head."""
    return 4.0 * batch * q_heads * head_dim * kv_len


def topk_attention_bytes(batch: int, hidden: int, kv_len: int, kept: int, out_bytes: int = 4) -> float:
    """Top-K sparse attention: the compressed K of every position, the
    compressed V of the kept positions only, plus the query and the output."""
    return packed_bytes(batch * hidden * (kv_len + min(kept, kv_len))) + batch * hidden * (2 + out_bytes)


def attention_flops(batch: int, hidden: int, kv_len: int) -> float:
    """q.k and p*v: two multiply-adds per cached element per sequence."""
    return 4.0 * batch * hidden * kv_len


def prefill_attention_flops(batch: int, hidden: int, seq: int) -> float:
    """Causal prefill attention: q.k and p*v, two multiply-adds per element
    for each of the seq*(seq+1)/2 (query, key) pairs of a sequence."""
    return 4.0 * batch * hidden * seq * (seq + 1) / 2


def append_bytes(batch: int, hidden: int, n_new: int = 1) -> float:
    """fp16 K and V rows in, compressed K and V rows out."""
    return batch * n_new * (2 * 2 * hidden + 2 * packed_bytes(hidden))


def quantize_bytes(rows: int, cols: int) -> float:
    return rows * cols * 2 + packed_bytes(rows * cols)


def gemm_bytes(M: int, K: int, N: int, y_bytes: int = 4) -> float:
    """Compressed weights once, fp16 activations in, outputs out."""
    return packed_bytes(K * N) + M * K * 2 + M * N * y_bytes


def gemm_flops(M: int, K: int, N: int) -> float:
    return 2.0 * M * K * N


def layer_gemm_flops(M: int, weights) -> float:
    return sum(gemm_flops(M, K, N) for K, N in weights)
