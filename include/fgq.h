/*
 * fgq.h - C ABI of libfgq: 4-bit asymmetric group-wise (64 elements per
 * group) compression of weights and KV cache, decode attention over the
 * compressed cache, and the dequantising weight GEMM of a block of GPU
 * batches, for AMD Instinct MI355X (gfx950).
 *
 * Method (pages on FlexGen, arXiv 2303.06865):
 *  - FlexGen review on jaehun.me, section "Is 4-bit compression the same as
 *    integer-arithmetic acceleration?" (paper section 5): weights and KV are
 *    stored as 4-bit integers and restored to FP16 before compute; groups of
 *    64 elements; weights grouped along the output channel, KV along the
 *    hidden dimension; asymmetric, from the group's minimum a and maximum b;
 *    a constant group needs separate handling.
 *  - FlexGen review on blog.gzher.com, section 3.4: fine-grained group-wise
 *    asymmetric quantisation of weights and KV cache, dequantised to FP16
 *    before computation; the aim is less storage and traffic, not INT4 math.
 *  - paper-graph-ui FlexGen summary, section 3.4 "Compute Schedule": a block
 *    is (GPU batch size g) x (number of GPU batches m); one load of a layer's
 *    weights serves every GPU batch of the block.
 *
 * Encoding (the formula is dropped from the pages; the plain min-max reading):
 *   per group of 64 fp16 values x_i:  a = min x_i, b = max x_i (signed zeros
 *   folded to +0); if a == b every code is 0 and the step is +0; otherwise
 *   q_i = roundTiesToEven(((x_i - a) / (b - a)) * 15) clamped to [0, 15], each
 *   operation a separate IEEE fp32 operation in that order; the group stores
 *   min = fp16(a) and step = fp16_RNE(fp32((b - a) / 15)).
 *   Reconstruction: x^ = min + q * step.
 *
 * Storage:
 *   codes  uint8 [rows][cols/2]; byte j holds element 2j in its low nibble and
 *          element 2j+1 in its high nibble.
 *   meta   uint32 [rows][cols/64]; low 16 bits fp16 min, high 16 bits fp16 step
 *          (a little-endian half2 {min, step}).
 *   0.5625 bytes per element (4-bit code plus 4 bytes of metadata per 64).
 *
 * Conventions for every call:
 *  - Every pointer is caller-owned device memory unless stated otherwise.
 *    The library never allocates, frees or retains memory and never
 *    synchronises; scratch space is a caller-provided workspace.
 *  - Every array must be 16-byte aligned (FGQ_ERR_ALIGN otherwise).
 *  - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL is
 *    the default stream).
 *  - Arguments are validated on the host before anything is enqueued; on any
 *    error nothing is enqueued and outputs are untouched.  A failed launch
 *    returns FGQ_ERR_DEVICE.  fgq_last_error() gives a text for the calling
 *    thread's last failure.
 *  - Size queries (the *_ws_bytes and *_words functions) return 0 for
 *    arguments the matching call rejects.
 *  - Inputs must be finite (precondition; the result is undefined otherwise).
 *  - Calls are reentrant; the library holds no mutable global state besides
 *    the per-thread error text and, for fgq_decode_attn_q4kv_noalloc only,
 *    one fixed scratch array per GPU (see there).
 */
#ifndef FGQ_H
#define FGQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FGQ_ABI_VERSION 3

typedef int32_t fgq_status;
#define FGQ_OK 0
#define FGQ_ERR_INVALID_ARG -1  /* null pointer or negative size */
#define FGQ_ERR_SHAPE -2        /* a size breaks a divisibility or range rule */
#define FGQ_ERR_ALIGN -3        /* an array (or leading dimension) is not 16-byte aligned */
#define FGQ_ERR_CAPACITY -4     /* KV positions beyond the cache capacity */
#define FGQ_ERR_WORKSPACE -5    /* workspace missing or smaller than the size query */
#define FGQ_ERR_DTYPE -6        /* unknown output dtype */
#define FGQ_ERR_DEVICE -7       /* the HIP runtime rejected a launch */
#define FGQ_ERR_UNSUPPORTED -8  /* valid but not implemented (e.g. head_dim not 64 or 128) */

/* Output element types. */
#define FGQ_DTYPE_F32 0
#define FGQ_DTYPE_F16 1

int32_t fgq_abi_version(void);
const char *fgq_status_string(fgq_status s);
/* Text describing the calling thread's most recent failure ("" if none). */
const char *fgq_last_error(void);

/*
 * fgq_quantize_g64 - compress an fp16 matrix, groups of 64 along its rows.
 *   x      fp16 [rows][ld_x], the first `cols` columns are read.
 *   codes  uint8 [rows][cols/2] out;  meta uint32 [rows][cols/64] out.
 * For a weight W [K = in][N = out] pass rows=K, cols=N: each group is 64
 * consecutive output channels at one input index.  For KV rows pass
 * [tokens][hidden]: each group is 64 consecutive hidden elements.
 * Requires cols % 64 == 0 and ld_x % 8 == 0, ld_x >= cols, rows * ld_x <= 2^48
 * (FGQ_ERR_SHAPE otherwise).  rows == 0 is a no-op.
 * Codes and meta equal, bit for bit, the encoding defined above.
 */
fgq_status fgq_quantize_g64(const void *x_f16, int64_t rows, int64_t cols, int64_t ld_x,
                            uint8_t *codes, uint32_t *meta, void *stream);

/*
 * Compressed KV cache of one layer, head-major:
 *   k_codes, v_codes  uint8  [batch][heads][capacity][head_dim/2]
 *   k_meta,  v_meta   uint32 [batch][heads][capacity][head_dim/64]
 * Groups run along the hidden dimension of one token's K (or V) row; with
 * head_dim a multiple of 64 a group never straddles two heads.  The caller
 * allocates the arrays; the library reads and writes them only in calls.
 * Every call that takes a cache requires capacity <= 2^30 and
 * batch * heads * capacity * head_dim <= 2^48 (FGQ_ERR_SHAPE otherwise).
 */
typedef struct fgq_kv_cache {
    uint8_t *k_codes;
    uint8_t *v_codes;
    uint32_t *k_meta;
    uint32_t *v_meta;
    int32_t batch;
    int32_t heads;
    int32_t head_dim;   /* 64 or 128 */
    int32_t capacity;   /* positions per sequence */
} fgq_kv_cache;

/*
 * fgq_kv_append - compress the K and V rows that a decode (or prompt) step
 * produced and write them at positions [pos, pos + n_new) of every sequence
 * (the cache persists and grows one token per decode step: paper-graph-ui
 * FlexGen summary, section 3.4, graph-traversal formulation; FlexGen review on
 * jaehun.me, "Is 4-bit compression ...": KV grouped along hidden).
 *   k_new, v_new  fp16 [batch][n_new][heads*head_dim], token-major.
 * Bit-exact with fgq_quantize_g64 on the same rows.  n_new == 0 or batch == 0
 * is a no-op.  pos + n_new > capacity -> FGQ_ERR_CAPACITY; k_new/v_new of
 * more than 2^48 elements (batch * n_new * row stride) -> FGQ_ERR_SHAPE.
 */
fgq_status fgq_kv_append(const fgq_kv_cache *kv, const void *k_new_f16, const void *v_new_f16,
                         int32_t pos, int32_t n_new, void *stream);

/*
 * fgq_kv_append_ld - fgq_kv_append over K and V rows that sit ld_new
 * elements apart: row (b * n_new + i) of k_new starts at element
 * (b * n_new + i) * ld_new.  This is how one fused projection writes them:
 * for a [rows][3 * hidden] output holding q | k | v side by side, pass
 * k_new = out + hidden, v_new = out + 2 * hidden, ld_new = 3 * hidden, so
 * the layer's Q/K/V product feeds the cache directly (the layer's output
 * feeds the next operation and its K and V persist in the cache:
 * paper-graph-ui FlexGen summary, section 3 "Technical Approach", the
 * computational graph of Figure 2).  Requires ld_new >= heads * head_dim
 * (FGQ_ERR_SHAPE) and ld_new % 8 == 0 (FGQ_ERR_ALIGN); otherwise as
 * fgq_kv_append, which is this call with ld_new = heads * head_dim.
 */
fgq_status fgq_kv_append_ld(const fgq_kv_cache *kv, const void *k_new_f16, const void *v_new_f16,
                            int64_t ld_new, int32_t pos, int32_t n_new, void *stream);

/*
 * fgq_decode_attn_q4kv - one decode step of attention for every sequence over
 * the compressed cache: for each (sequence, head)
 *   s_j = softmax_scale * sum_d q_d * K^_{j,d},  j in [0, kv_len)
 *   o_d = sum_j softmax(s)_j * V^_{j,d}
 * with K^, V^ reconstructed on the fly (paper-graph-ui FlexGen summary,
 * section 3.4 "Computation delegation": decode attention reads the whole
 * cache and is bound by I/O; FlexGen review on blog.gzher.com, section 3.4).
 *   q    fp16 [batch][heads*head_dim];  out [batch][heads*head_dim] in out_dtype.
 *   softmax_scale <= 0 selects 1/sqrt(head_dim).  Every sequence attends the
 *   same kv_len positions (no mask).  Requires 1 <= kv_len <= capacity.
 *   ws / ws_bytes: workspace of at least fgq_decode_attn_ws_bytes(...) bytes
 *   (may be NULL when that is 0): per-split partial softmax states.
 * The result depends on the split plan only through fp32 rounding.
 */
size_t fgq_decode_attn_ws_bytes(int32_t batch, int32_t heads, int32_t head_dim, int32_t kv_len);
fgq_status fgq_decode_attn_q4kv(const fgq_kv_cache *kv, const void *q_f16, int32_t kv_len,
                                float softmax_scale, void *out, int32_t out_dtype,
                                void *ws, size_t ws_bytes, void *stream);

/*
 * fgq_decode_attn_q4kv_ld - fgq_decode_attn_q4kv with the query of sequence b
 * at q_f16 + b * ld_q (elements), e.g. the q part of a fused [rows][3 *
 * hidden] Q/K/V product (ld_q = 3 * hidden).  Requires ld_q >= heads *
 * head_dim (FGQ_ERR_SHAPE) and ld_q % 8 == 0 (FGQ_ERR_ALIGN); out stays
 * [batch][heads*head_dim].  fgq_decode_attn_q4kv is this call with
 * ld_q = heads * head_dim.  batch * heads must stay below 2^31
 * (FGQ_ERR_SHAPE).
 */
fgq_status fgq_decode_attn_q4kv_ld(const fgq_kv_cache *kv, const void *q_f16, int64_t ld_q, int32_t kv_len,
                                   float softmax_scale, void *out, int32_t out_dtype,
                                   void *ws, size_t ws_bytes, void *stream);

/*
 * fgq_decode_attn_q4kv_noalloc - fgq_decode_attn_q4kv for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation): the same kernels and result, with the
 * per-split softmax states kept in a fixed scratch array inside the library
 * (FGQ_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends) instead of
 * a workspace argument.  It allocates nothing.  The split plan never needs
 * more than 8,650,224 bytes of states; a call that would is rejected with
 * FGQ_ERR_WORKSPACE.  Every call on one GPU shares that GPU's scratch: calls
 * that overlap on one GPU (two streams, or two threads) race and must be
 * ordered by the caller.  The first call on a device looks up the scratch's
 * device address (FGQ_ERR_DEVICE if that fails).
 */
#define FGQ_NOALLOC_SCRATCH_BYTES ((size_t)9 << 20)
fgq_status fgq_decode_attn_q4kv_noalloc(const fgq_kv_cache *kv, const void *q_f16, int32_t kv_len,
                                        float softmax_scale, void *out, int32_t out_dtype, void *stream);

/*
 * fgq_decode_attn_gqa_q4kv - decode attention with grouped K/V heads (GQA) or
 * one shared K/V head (MQA) over the compressed cache (vTensor page on
 * papercache.org, background section "GQA and MQA optimisation": the query
 * heads are divided into groups, each group sharing one key head and one
 * value head; MQA shares a single one).  The cache holds kv->heads K/V heads;
 * with R = q_heads / kv->heads, query head hq reads cache head hq / R
 * (consecutive query heads form a group).  For each (sequence, query head):
 *   s_j = softmax_scale * sum_d q_{hq,d} * K^_{hq/R,j,d},  j in [0, kv_len)
 *   o_d = sum_j softmax(s)_j * V^_{hq/R,j,d}
 *   q    fp16 [batch][q_heads*head_dim];  out [batch][q_heads*head_dim] in out_dtype.
 *   Requires q_heads a multiple of kv->heads (FGQ_ERR_SHAPE),
 *   R <= FGQ_GQA_MAX_GROUP and, for R > 1, capacity * head_dim / 2 < 2^32
 *   (FGQ_ERR_UNSUPPORTED); R == 1 is fgq_decode_attn_q4kv.  softmax_scale <= 0 selects 1/sqrt(head_dim); every
 *   sequence attends the same kv_len positions; 1 <= kv_len <= capacity.
 *   ws / ws_bytes: at least fgq_decode_attn_gqa_ws_bytes(...) bytes (may be
 *   NULL when that is 0): per-split partial softmax states.
 * Fp16 matrix cores with fp32 accumulation: the codes enter exactly, the
 * probabilities enter the p.v product as fp16(p * step).  The result depends
 * on the split plan only through fp32 rounding.
 */
#define FGQ_GQA_MAX_GROUP 32
size_t fgq_decode_attn_gqa_ws_bytes(int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                                    int32_t kv_len);
fgq_status fgq_decode_attn_gqa_q4kv(const fgq_kv_cache *kv, const void *q_f16, int32_t q_heads,
                                    int32_t kv_len, float softmax_scale, void *out, int32_t out_dtype,
                                    void *ws, size_t ws_bytes, void *stream);

/*
 * fgq_decode_attn_topk_q4kv - top-K sparse variant of fgq_decode_attn_q4kv:
 * the paper's optional approximation that reads only the top 10% of the value
 * cache (FlexGen review on blog.gzher.com, section 3.4; paper-graph-ui FlexGen
 * summary, section 3.3: a section-5 approximation meant to cut I/O).  For
 * each (sequence, head):
 *   s_j = softmax_scale * sum_d q_d * K^_{j,d},  j in [0, kv_len)
 *   T   = the kk = min(top_k, kv_len) positions with the largest s_j, scores
 *         compared as fp32 values (-0 as +0), equal scores going to the
 *         lower position
 *   o_d = sum_{j in T} exp(s_j - m) V^_{j,d} / sum_{j in T} exp(s_j - m),
 *         m = max_j s_j
 * Every K row is read; only the kk kept V rows are.  top_k >= kv_len is
 * dense attention.
 *   q fp16 [batch][heads*head_dim]; out [batch][heads*head_dim] in out_dtype.
 *   sel: NULL, or int32 [batch][heads][kk] receiving the kept positions of
 *   every (sequence, head) in ascending order.
 *   softmax_scale <= 0 selects 1/sqrt(head_dim).  Requires top_k >= 1
 *   (FGQ_ERR_INVALID_ARG), 1 <= kv_len <= capacity, and
 *   kv_len <= FGQ_TOPK_MAX_POSITIONS (FGQ_ERR_UNSUPPORTED: the selection
 *   state of one (sequence, head) lives in on-chip memory, 4 bytes per
 *   position while kv_len + kk <= 19840, 2.125 bytes beyond).  No workspace.
 */
#define FGQ_TOPK_MAX_POSITIONS 65536
fgq_status fgq_decode_attn_topk_q4kv(const fgq_kv_cache *kv, const void *q_f16, int32_t kv_len,
                                     int32_t top_k, float softmax_scale, void *out, int32_t out_dtype,
                                     int32_t *sel, void *stream);

/*
 * fgq_prefill_attn_f16 - attention of the prefill step over the prompt's own
 * fp16 q, k, v, before its K and V are compressed (then one bulk
 * fgq_kv_append with n_new = seq): the prefill step runs every prompt token
 * at once and leaves each layer's KV cache behind (paper-graph-ui FlexGen
 * summary, section 3.4, token 0 of the Figure-2 grid; FlexGen review on
 * blog.gzher.com, section 1).  Causal: per (sequence, head, token i)
 *   o_i = sum_{j<=i} softmax_j(softmax_scale * q_i . k_j) v_j
 *   q, k, v fp16 [batch][seq][heads*head_dim] (token-major, as the QKV
 *   projection emits them); out [batch][seq][heads*head_dim] in out_dtype.
 *   softmax_scale <= 0 selects 1/sqrt(head_dim).  head_dim 64 or 128;
 *   batch, heads <= 65535 and batch*heads*ceil(seq/128) < 2^31
 *   (FGQ_ERR_SHAPE).  Fp16 matrix cores with fp32
 *   accumulation; the probabilities enter P.V rounded to fp16.  No workspace.
 */
fgq_status fgq_prefill_attn_f16(const void *q_f16, const void *k_f16, const void *v_f16, int32_t batch,
                                int32_t seq, int32_t heads, int32_t head_dim, float softmax_scale, void *out,
                                int32_t out_dtype, void *stream);

/*
 * fgq_dequant_gemm - Y = X * W^ for one block of m GPU batches of g rows that
 * share one read of the compressed weight (paper-graph-ui FlexGen summary,
 * section 3.4 "Compute Schedule"; FlexGen review on jaehun.me, "A block is
 * the unit of weight reuse": B = g*m), straight from the weight's codes and
 * metadata as fgq_quantize_g64 writes them for W [K = in][N = out] (groups
 * of 64 output channels: FlexGen review on jaehun.me, "Is 4-bit compression
 * the same as integer-arithmetic acceleration?").
 *   x       fp16 [g*m][K], GPU batch j in rows j*g .. j*g+g-1;
 *   w_codes uint8 [K][N/2], w_meta uint32 [K][N/64] (half2 {min, step});
 *   y       [g*m][N] in y_dtype.
 * W^ = fp16(min + q*step) (one rounding) is multiplied on the fp16 matrix
 * cores with fp32 accumulation.  Requires K % 64 == 0, N % 64 == 0,
 * K <= 2^23 and N <= 2^27 (FGQ_ERR_SHAPE otherwise); g*m == 0 is a no-op.
 *   ws / ws_bytes: at least fgq_dequant_gemm_ws_bytes(g*m, K, N) bytes of
 *   workspace (split-K partial sums; may be NULL when that is 0).
 * stream is a hipStream_t.
 */
size_t fgq_dequant_gemm_ws_bytes(int64_t M, int64_t K, int64_t N);
fgq_status fgq_dequant_gemm(const void *x_f16, int32_t g, int32_t m, int64_t K, int64_t N,
                            const uint8_t *w_codes, const void *w_meta, void *y, int32_t y_dtype,
                            void *ws, size_t ws_bytes, void *stream);

/*
 * fgq_pack_weight_g64 - part of the offline weight compression: a one-time
 * re-layout of a compressed weight (codes and meta as fgq_quantize_g64
 * writes them for W [K][N]) into the tile order of fgq_dequant_gemm_packed.
 * The codes are only moved; the metadata are rescaled by powers of two (and
 * rounded to fp16 again, which changes a value only when it falls below the
 * fp16 normal range).
 *   packed_codes uint32 [K/32][N/64][64][4]: word (kc, g, lane, j) holds the
 *     codes of W[k][n], n = 64g + 16j + lane%16, k = 32kc + 8(lane/16) + i for
 *     i = 0..7, code i in nibble [0,4,1,5,2,6,3,7][i] of the word (same byte
 *     size as codes).
 *   packed_meta uint32, fgq_pack_weight_meta_words(K, N) = K*N/64 + N/64
 *     words: first [K/32][N/64][4][8], entry (kc, g, kq, t) the half2
 *     {step[k] * 2^s, step[k+1] * 2^s} for t < 4 (s = 24 - e_g for even t,
 *     20 - e_g for odd t) and {min[k] * 2^-e_g, min[k+1] * 2^-e_g} for
 *     t >= 4, with k = 32kc + 8kq + 2(t%4), each rounded to fp16 (exact
 *     unless it falls below the fp16 normal range); then int32 e_g for every
 *     column group g: the smallest e >= 0 with max_k step[k][g] * 2^(24-e)
 *     <= 65504.  (The GEMM multiplies codes placed as q * 2^-24 or q * 2^-20
 *     by these steps, and its result by 2^e_g.)
 * Requires K % 32 == 0, N % 64 == 0, K <= 2^23 and N <= 2^28 (FGQ_ERR_SHAPE
 * otherwise; the word count query returns 0 for such sizes).
 */
size_t fgq_pack_weight_meta_words(int64_t K, int64_t N);
fgq_status fgq_pack_weight_g64(const uint8_t *codes, const uint32_t *meta, int64_t K, int64_t N,
                               uint32_t *packed_codes, uint32_t *packed_meta, void *stream);

/*
 * fgq_dequant_gemm_packed - fgq_dequant_gemm over the packed layout that
 * fgq_pack_weight_g64 makes offline (same block semantics and workspace
 * query).  The restored weight is 2^e_g * fp16(2^-e_g * min + q * 2^-e_g *
 * step), which equals fp16(min + q*step) unless 2^-e_g * W^ falls below the
 * fp16 normal range (then within 2^(e_g - 25)).  Requires K % 32 == 0,
 * N % 64 == 0, K <= 2^23 and N <= 2^28 (FGQ_ERR_SHAPE otherwise).
 */
fgq_status fgq_dequant_gemm_packed(const void *x_f16, int32_t g, int32_t m, int64_t K, int64_t N,
                                   const uint32_t *packed_codes, const uint32_t *packed_meta,
                                   void *y, int32_t y_dtype, void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FGQ_H */
