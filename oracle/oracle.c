/*
 * CPU ORACLE for 4-bit asymmetric group-wise (group = 64) compression of
 * weights and KV cache, decode attention over the compressed cache, and the
 * dequantize-then-multiply weight GEMM of a block of GPU batches.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The GPU library never
 * links, calls or includes anything from here, and this file includes nothing
 * from the GPU library.
 *
 * Plain and slow on purpose: per-element loops in the order of the method's
 * definition, IEEE fp32 for the quantiser (its decisions are integers and are
 * taken in fp32, as the GPU takes them), fp64 for attention and the GEMM.
 * OpenMP only splits independent output units; every output is summed in the
 * same order for any thread count.
 *
 * Sources (pages on FlexGen, arXiv 2303.06865):
 *  [jaehun] FlexGen review on jaehun.me, section "Is 4-bit compression the
 *           same as integer-arithmetic acceleration?" (paper section 5):
 *           weights and KV are stored as 4-bit integers and restored to FP16
 *           before compute; groups of 64 elements, weights grouped along the
 *           output channel, KV along the hidden dimension; asymmetric, using
 *           the group's minimum a and maximum b when a != b; constant groups
 *           need separate handling; reconstruction is not exact.
 *  [gzher]  FlexGen review on blog.gzher.com, section 3.4 (4-bit compression
 *           of weights and KV cache): fine-grained group-wise asymmetric
 *           quantisation, dequantised back to FP16 before computation.
 *  [pgui]   paper-graph-ui FlexGen summary, section 3.4, "Compute Schedule":
 *           block = GPU batch size x number of GPU batches; one load of a
 *           layer's weights serves every GPU batch of the block.
 *
 * The pages drop the quantisation formula itself.  The reading taken here is
 * the plain min-max one:  q = roundTiesToEven(((x - a) / (b - a)) * 15),
 * stored with min a and step (b - a)/15 as fp16, each operation a separate
 * IEEE fp32 operation in exactly this order (no reciprocal, no fused
 * multiply-add).  A constant group (a == b) stores codes 0 and step +0, so it
 * reconstructs exactly.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

#define ORACLE_OK 0
#define ORACLE_ERR_SHAPE -2
#define ORACLE_ERR_NONFINITE -9

/* ---------------------------------------------------------------------------
 * IEEE-754 binary16 <-> binary32, written from the format's definition:
 * sign bit, 5-bit biased exponent (bias 15), 10-bit fraction; exponent field 0
 * encodes subnormals (fraction * 2^-24), 31 encodes inf/NaN.
 * ------------------------------------------------------------------------- */
float oracle_f16_to_f32(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f + 1024), e - 25);
    return (float)(sign ? -v : v);
}

/* Round-to-nearest, ties-to-even conversion of a float to binary16. */
uint16_t oracle_f32_to_f16(float x) {
    if (isnan(x)) return 0x7e00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs((double)x);
    if (a == 0.0) return sign;
    /* quantum (spacing of binary16 numbers) at the magnitude of a */
    int e;
    frexp(a, &e);               /* a = m * 2^e, m in [0.5, 1) -> leading bit at 2^(e-1) */
    int lead = e - 1;
    if (lead < -14) lead = -14; /* subnormal range shares the quantum 2^-24 */
    double quantum = ldexp(1.0, lead - 10);
    double n = rint(a / quantum);   /* exact division by a power of two; RNE in default mode */
    double r = n * quantum;
    if (r >= 65536.0) return sign | 0x7c00;  /* overflow to infinity */
    if (r < ldexp(1.0, -14)) {                /* subnormal (or rounded up to min normal below) */
        return sign | (uint16_t)(r / ldexp(1.0, -24));
    }
    int re;
    double rm = frexp(r, &re);  /* r = rm * 2^re, rm in [0.5, 1) */
    int biased = re - 1 + 15;
    uint16_t frac = (uint16_t)((rm * 2.0 - 1.0) * 1024.0);
    return sign | (uint16_t)(biased << 10) | frac;
}

static int f16_finite(uint16_t h) { return ((h >> 10) & 0x1f) != 31; }

/* ---------------------------------------------------------------------------
 * One group of 64 fp16 values -> 32 code bytes + one meta word.
 * codes: byte j holds element 2j in its low nibble and 2j+1 in its high nibble.
 * meta:  low 16 bits = fp16 min a, high 16 bits = fp16 step (b - a) / 15.
 * ------------------------------------------------------------------------- */
static void quantize_group(const uint16_t *xh, uint8_t *codes, uint32_t *meta) {
    float x[64];
    for (int i = 0; i < 64; ++i) x[i] = oracle_f16_to_f32(xh[i]);

    float a = x[0], b = x[0];
    for (int i = 1; i < 64; ++i) {
        if (x[i] < a) a = x[i];
        if (x[i] > b) b = x[i];
    }
    a = a + 0.0f;   /* -0 becomes +0 */
    b = b + 0.0f;
    uint16_t min_h = oracle_f32_to_f16(a);  /* exact: a is an fp16 value */

    if (a == b) {   /* constant group: all codes 0, step +0 */
        memset(codes, 0, 32);
        *meta = (uint32_t)min_h;
        return;
    }

    float d = b - a;
    uint8_t q[64];
    for (int i = 0; i < 64; ++i) {
        float t = x[i] - a;
        float u = t / d;
        float v = u * 15.0f;
        float r = rintf(v);             /* ties to even */
        if (r < 0.0f) r = 0.0f;
        if (r > 15.0f) r = 15.0f;
        q[i] = (uint8_t)r;
    }
    for (int j = 0; j < 32; ++j) codes[j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));

    float step = d / 15.0f;
    uint16_t step_h = oracle_f32_to_f16(step);
    *meta = (uint32_t)min_h | ((uint32_t)step_h << 16);
}

/* Reconstruction of one code: fp32(min + q * step), one rounding. */
static inline float dequant_one(uint32_t meta, int q) {
    double mn = (double)oracle_f16_to_f32((uint16_t)(meta & 0xffff));
    double st = (double)oracle_f16_to_f32((uint16_t)(meta >> 16));
    return (float)(mn + (double)q * st);
}

static inline int code_at(const uint8_t *codes_row, int64_t i) {
    uint8_t byte = codes_row[i >> 1];
    return (i & 1) ? (byte >> 4) : (byte & 0xf);
}

/* x: fp16 [rows][ld_x] (cols used), groups of 64 consecutive columns.
 * codes: [rows][cols/2], meta: [rows][cols/64]. */
int oracle_quantize_g64(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                        uint8_t *codes, uint32_t *meta) {
    if (rows < 0 || cols < 0 || cols % 64 != 0 || ld_x < cols) return ORACLE_ERR_SHAPE;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            if (!f16_finite(x[r * ld_x + c])) return ORACLE_ERR_NONFINITE;
    int64_t ng = cols / 64;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t gi = 0; gi < ng; ++gi)
            quantize_group(x + r * ld_x + gi * 64, codes + r * (cols / 2) + gi * 32, meta + r * ng + gi);
    return ORACLE_OK;
}

/* out: fp32 [rows][cols] = reconstruction of every code. */
int oracle_dequant_g64(const uint8_t *codes, const uint32_t *meta, int64_t rows, int64_t cols, float *out) {
    if (rows < 0 || cols < 0 || cols % 64 != 0) return ORACLE_ERR_SHAPE;
    int64_t ng = cols / 64;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = dequant_one(meta[r * ng + c / 64], code_at(codes + r * (cols / 2), c));
    return ORACLE_OK;
}

/* KV append: k_new, v_new fp16 [batch][n_new][heads*head_dim] (token-major);
 * cache K/V codes [batch][heads][cap][head_dim/2], meta [batch][heads][cap][head_dim/64].
 * Each new token's K (and V) row is grouped along the hidden dimension, 64
 * consecutive hidden elements per group; groups never straddle heads because
 * head_dim is a multiple of 64.  Writes positions [pos, pos + n_new). */
int oracle_kv_append(const uint16_t *k_new, const uint16_t *v_new,
                     int32_t batch, int32_t heads, int32_t head_dim, int32_t cap,
                     int32_t pos, int32_t n_new,
                     uint8_t *k_codes, uint32_t *k_meta, uint8_t *v_codes, uint32_t *v_meta) {
    if (head_dim % 64 != 0 || pos < 0 || n_new < 0 || (int64_t)pos + n_new > cap) return ORACLE_ERR_SHAPE;
    int64_t h = (int64_t)heads * head_dim;
    int64_t gph = head_dim / 64;
    for (int64_t i = 0; i < (int64_t)batch * n_new * h; ++i)
        if (!f16_finite(k_new[i]) || !f16_finite(v_new[i])) return ORACLE_ERR_NONFINITE;
    #pragma omp parallel for collapse(2) schedule(static)
    for (int32_t b = 0; b < batch; ++b)
        for (int32_t hd = 0; hd < heads; ++hd)
            for (int32_t i = 0; i < n_new; ++i)
                for (int64_t gi = 0; gi < gph; ++gi) {
                    int64_t src = ((int64_t)b * n_new + i) * h + (int64_t)hd * head_dim + gi * 64;
                    int64_t slot = ((int64_t)b * heads + hd) * cap + pos + i;
                    quantize_group(k_new + src, k_codes + slot * (head_dim / 2) + gi * 32, k_meta + slot * gph + gi);
                    quantize_group(v_new + src, v_codes + slot * (head_dim / 2) + gi * 32, v_meta + slot * gph + gi);
                }
    return ORACLE_OK;
}

/* Decode attention for one new query per sequence over the compressed cache.
 * q fp16 [batch][heads*head_dim]; attends positions [0, kv_len) of every
 * sequence; out fp32 [batch][heads*head_dim].
 *   s_j = scale * sum_d q_d * K^_{j,d}          (fp64, d ascending)
 *   p_j = exp(s_j - max_j s_j) / sum_j exp(...)  (fp64)
 *   o_d = sum_j p_j * V^_{j,d}                   (fp64, j ascending)
 * where K^, V^ are the fp32 reconstructions of the stored codes. */
int oracle_decode_attn(const uint16_t *q, int32_t batch, int32_t heads, int32_t head_dim, int32_t cap,
                       const uint8_t *k_codes, const uint32_t *k_meta,
                       const uint8_t *v_codes, const uint32_t *v_meta,
                       int32_t kv_len, double scale, float *out) {
    if (head_dim % 64 != 0 || kv_len < 1 || kv_len > cap) return ORACLE_ERR_SHAPE;
    int64_t h = (int64_t)heads * head_dim;
    int64_t gph = head_dim / 64;
    #pragma omp parallel for collapse(2) schedule(static)
    for (int32_t b = 0; b < batch; ++b)
        for (int32_t hd = 0; hd < heads; ++hd) {
            double *s = (double *)malloc(sizeof(double) * (size_t)kv_len);
            double *o = (double *)calloc((size_t)head_dim, sizeof(double));
            const uint16_t *qv = q + (int64_t)b * h + (int64_t)hd * head_dim;
            int64_t base = ((int64_t)b * heads + hd) * cap;
            for (int32_t j = 0; j < kv_len; ++j) {
                const uint8_t *kc = k_codes + (base + j) * (head_dim / 2);
                const uint32_t *km = k_meta + (base + j) * gph;
                double acc = 0.0;
                for (int32_t d = 0; d < head_dim; ++d)
                    acc += (double)oracle_f16_to_f32(qv[d]) * (double)dequant_one(km[d / 64], code_at(kc, d));
                s[j] = acc * scale;
            }
            double mx = s[0];
            for (int32_t j = 1; j < kv_len; ++j) if (s[j] > mx) mx = s[j];
            double den = 0.0;
            for (int32_t j = 0; j < kv_len; ++j) { s[j] = exp(s[j] - mx); den += s[j]; }
            for (int32_t j = 0; j < kv_len; ++j) {
                const uint8_t *vc = v_codes + (base + j) * (head_dim / 2);
                const uint32_t *vm = v_meta + (base + j) * gph;
                for (int32_t d = 0; d < head_dim; ++d)
                    o[d] += s[j] * (double)dequant_one(vm[d / 64], code_at(vc, d));
            }
            float *ov = out + (int64_t)b * h + (int64_t)hd * head_dim;
            for (int32_t d = 0; d < head_dim; ++d) ov[d] = (float)(o[d] / den);
            free(s);
            free(o);
        }
    return ORACLE_OK;
}

/* Top-K sparse decode attention: the paper's optional approximation that
 * reads only the top 10% of the value cache (FlexGen review on
 * blog.gzher.com, section 3.4; paper-graph-ui FlexGen summary, section 3.3
 * "Roadmap for the Deep Dive": with 4-bit group-wise compression, one of the
 * two section-5 approximations, both meant to cut I/O volume).  The pages
 * give no formula.  Reading taken: every position is scored
 * over the compressed K exactly as in dense decode attention; the top_k
 * positions with the largest scores are kept, the scores compared as fp32
 * values (the GPU's precision: fp64 score rounded once to fp32, -0 taken as
 * +0), equal scores going to the lower position; softmax over the kept
 * positions only, and V rows of kept positions only:
 *   T   = top_k positions by (fp32(s_j) descending, j ascending)
 *   o_d = sum_{j in T} exp(s_j - m) V^_{j,d} / sum_{j in T} exp(s_j - m),
 *         m = max_j s_j                      (fp64, j ascending)
 * top_k >= kv_len keeps every position, and then the result is the dense one
 * bit for bit (the same loops in the same order).  sel (may be NULL) receives
 * the kept positions of every (b, head) in ascending order, int32
 * [batch][heads][min(top_k, kv_len)]. */
typedef struct { float s32; int32_t j; } oracle_rank;

static int rank_cmp(const void *pa, const void *pb) {
    const oracle_rank *a = (const oracle_rank *)pa, *b = (const oracle_rank *)pb;
    if (a->s32 > b->s32) return -1;
    if (a->s32 < b->s32) return 1;
    return (a->j > b->j) - (a->j < b->j);
}

int oracle_decode_attn_topk(const uint16_t *q, int32_t batch, int32_t heads, int32_t head_dim, int32_t cap,
                            const uint8_t *k_codes, const uint32_t *k_meta,
                            const uint8_t *v_codes, const uint32_t *v_meta,
                            int32_t kv_len, int32_t top_k, double scale, float *out, int32_t *sel) {
    if (head_dim % 64 != 0 || kv_len < 1 || kv_len > cap || top_k < 1) return ORACLE_ERR_SHAPE;
    const int32_t kk = top_k < kv_len ? top_k : kv_len;
    int64_t h = (int64_t)heads * head_dim;
    int64_t gph = head_dim / 64;
    #pragma omp parallel for collapse(2) schedule(static)
    for (int32_t b = 0; b < batch; ++b)
        for (int32_t hd = 0; hd < heads; ++hd) {
            double *s = (double *)malloc(sizeof(double) * (size_t)kv_len);
            unsigned char *keep = (unsigned char *)calloc((size_t)kv_len, 1);
            oracle_rank *rk = (oracle_rank *)malloc(sizeof(oracle_rank) * (size_t)kv_len);
            double *o = (double *)calloc((size_t)head_dim, sizeof(double));
            const uint16_t *qv = q + (int64_t)b * h + (int64_t)hd * head_dim;
            int64_t base = ((int64_t)b * heads + hd) * cap;
            for (int32_t j = 0; j < kv_len; ++j) {
                const uint8_t *kc = k_codes + (base + j) * (head_dim / 2);
                const uint32_t *km = k_meta + (base + j) * gph;
                double acc = 0.0;
                for (int32_t d = 0; d < head_dim; ++d)
                    acc += (double)oracle_f16_to_f32(qv[d]) * (double)dequant_one(km[d / 64], code_at(kc, d));
                s[j] = acc * scale;
                rk[j].s32 = (float)s[j] + 0.0f;
                rk[j].j = j;
            }
            qsort(rk, (size_t)kv_len, sizeof(oracle_rank), rank_cmp);
            for (int32_t i = 0; i < kk; ++i) keep[rk[i].j] = 1;
            double mx = s[0];
            for (int32_t j = 1; j < kv_len; ++j) if (s[j] > mx) mx = s[j];
            double den = 0.0;
            for (int32_t j = 0; j < kv_len; ++j)
                if (keep[j]) { s[j] = exp(s[j] - mx); den += s[j]; }
            int32_t n = 0;
            for (int32_t j = 0; j < kv_len; ++j) {
                if (!keep[j]) continue;
                if (sel) sel[((int64_t)b * heads + hd) * kk + n] = j;
                ++n;
                const uint8_t *vc = v_codes + (base + j) * (head_dim / 2);
                const uint32_t *vm = v_meta + (base + j) * gph;
                for (int32_t d = 0; d < head_dim; ++d)
                    o[d] += s[j] * (double)dequant_one(vm[d / 64], code_at(vc, d));
            }
            float *ov = out + (int64_t)b * h + (int64_t)hd * head_dim;
            for (int32_t d = 0; d < head_dim; ++d) ov[d] = (float)(o[d] / den);
            free(s);
            free(keep);
            free(rk);
            free(o);
        }
    return ORACLE_OK;
}

/* Prefill attention over the prompt's fp16 K and V, before they are
 * compressed: the prefill step runs every prompt token at once and leaves
 * each layer's KV cache behind (paper-graph-ui FlexGen summary, section 3.4,
 * the problem formulation around Figure 2, where token 0 of the grid is the
 * prefill step; FlexGen review on blog.gzher.com, section 1, the prefill /
 * decode split).  OPT models are decoder-only, so each prompt token attends
 * to itself and the tokens before it (the plainest reading; the pages do not
 * spell out the mask).  q, k, v fp16 [batch][seq][heads*head_dim]
 * (token-major, as the QKV projection emits them); rows [row0, row1) of
 * every sequence and head are computed:
 *   s_ij = scale * sum_d q_{i,d} k_{j,d}               j <= i   (fp64)
 *   o_i  = sum_{j<=i} exp(s_ij - m_i) v_j / sum_{j<=i} exp(s_ij - m_i)
 * out fp32 [batch][seq][heads*head_dim]; rows outside [row0, row1) are
 * left untouched. */
int oracle_prefill_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v, int32_t batch, int32_t seq,
                        int32_t heads, int32_t head_dim, int32_t row0, int32_t row1, double scale, float *out) {
    if (batch < 0 || seq < 0 || heads < 0 || head_dim <= 0 || row0 < 0 || row1 > seq || row0 > row1)
        return ORACLE_ERR_SHAPE;
    const int64_t h = (int64_t)heads * head_dim;
    #pragma omp parallel for collapse(3) schedule(dynamic, 1)
    for (int32_t b = 0; b < batch; ++b)
        for (int32_t hd = 0; hd < heads; ++hd)
            for (int32_t i = row0; i < row1; ++i) {
                double *s = (double *)malloc(sizeof(double) * (size_t)(i + 1));
                double *o = (double *)calloc((size_t)head_dim, sizeof(double));
                const uint16_t *qi = q + ((int64_t)b * seq + i) * h + (int64_t)hd * head_dim;
                double mx = -INFINITY;
                for (int32_t j = 0; j <= i; ++j) {
                    const uint16_t *kj = k + ((int64_t)b * seq + j) * h + (int64_t)hd * head_dim;
                    double acc = 0.0;
                    for (int32_t d = 0; d < head_dim; ++d)
                        acc += (double)oracle_f16_to_f32(qi[d]) * (double)oracle_f16_to_f32(kj[d]);
                    s[j] = acc * scale;
                    if (s[j] > mx) mx = s[j];
                }
                double den = 0.0;
                for (int32_t j = 0; j <= i; ++j) {
                    s[j] = exp(s[j] - mx);
                    den += s[j];
                }
                for (int32_t j = 0; j <= i; ++j) {
                    const uint16_t *vj = v + ((int64_t)b * seq + j) * h + (int64_t)hd * head_dim;
                    for (int32_t d = 0; d < head_dim; ++d) o[d] += s[j] * (double)oracle_f16_to_f32(vj[d]);
                }
                float *oi = out + ((int64_t)b * seq + i) * h + (int64_t)hd * head_dim;
                for (int32_t d = 0; d < head_dim; ++d) oi[d] = (float)(o[d] / den);
                free(s);
                free(o);
            }
    return ORACLE_OK;
}

/* Weight GEMM of one block of g*m rows (m GPU batches of g rows each, batch j
 * occupying rows j*g .. j*g+g-1) against the compressed weight W [K][N]
 * (codes [K][N/2], meta [K][N/64]: groups along the output channel n):
 *   Y[r][n] = sum_k X[r][k] * W^[k][n]   (fp64, k ascending) -> fp32.
 * The weight is reconstructed once per k-row and used for every row of the
 * block; each Y[r][n] is still a plain k-ascending sum. */
int oracle_dequant_gemm(const uint16_t *x, int32_t g, int32_t m, int64_t K, int64_t N,
                        const uint8_t *w_codes, const uint32_t *w_meta, float *y) {
    if (g < 0 || m < 0 || K < 0 || N % 64 != 0) return ORACLE_ERR_SHAPE;
    int64_t M = (int64_t)g * m;
    int64_t ng = N / 64;
    const int64_t CB = 256;   /* independent column blocks for the threads */
    int64_t nblk = (N + CB - 1) / CB;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t blk = 0; blk < nblk; ++blk) {
        int64_t n0 = blk * CB, n1 = n0 + CB < N ? n0 + CB : N, nw = n1 - n0;
        double *acc = (double *)calloc((size_t)(M * nw), sizeof(double));
        double *wrow = (double *)malloc(sizeof(double) * (size_t)nw);
        double *xcol = (double *)malloc(sizeof(double) * (size_t)(M ? M : 1));
        for (int64_t k = 0; k < K; ++k) {
            const uint8_t *cr = w_codes + k * (N / 2);
            const uint32_t *mr = w_meta + k * ng;
            for (int64_t n = n0; n < n1; ++n) wrow[n - n0] = (double)dequant_one(mr[n / 64], code_at(cr, n));
            for (int64_t r = 0; r < M; ++r) xcol[r] = (double)oracle_f16_to_f32(x[r * K + k]);
            for (int64_t r = 0; r < M; ++r) {
                double xv = xcol[r];
                double *ar = acc + r * nw;
                for (int64_t n = 0; n < nw; ++n) ar[n] += xv * wrow[n];
            }
        }
        for (int64_t r = 0; r < M; ++r)
            for (int64_t n = 0; n < nw; ++n) y[r * N + n0 + n] = (float)acc[r * nw + n];
        free(acc);
        free(wrow);
        free(xcol);
    }
    return ORACLE_OK;
}

/* Decode attention with grouped K/V heads (GQA) or one shared K/V head (MQA)
 * over the compressed cache (vTensor page on papercache.org, background
 * section "GQA and MQA optimisation": with MQA every query head shares one
 * key head and one value head; with GQA the query heads are divided into
 * groups and each group shares one key head and one value head; section
 * "Roofline comparison" and Figure 3: fewer shared heads raise the
 * arithmetic intensity of decode attention).  The pages do not say which
 * query heads form a group; the reading taken is consecutive heads:
 * with R = q_heads / kv_heads, query head hq reads cache head kh = hq / R.
 * q fp16 [batch][q_heads*head_dim]; the cache holds kv_heads heads; out fp32
 * [batch][q_heads*head_dim].  Per (b, hq):
 *   s_j = scale * sum_d q_{hq,d} * K^_{kh,j,d}        (fp64, d ascending)
 *   o_d = sum_j exp(s_j - max s) * V^_{kh,j,d} / sum_j exp(s_j - max s)
 * kv_heads == q_heads is plain multi-head attention (R = 1). */
int oracle_decode_attn_gqa(const uint16_t *q, int32_t batch, int32_t q_heads, int32_t kv_heads,
                           int32_t head_dim, int32_t cap, const uint8_t *k_codes, const uint32_t *k_meta,
                           const uint8_t *v_codes, const uint32_t *v_meta, int32_t kv_len, double scale,
                           float *out) {
    if (head_dim % 64 != 0 || kv_len < 1 || kv_len > cap || kv_heads < 1 || q_heads < kv_heads ||
        q_heads % kv_heads != 0)
        return ORACLE_ERR_SHAPE;
    const int32_t R = q_heads / kv_heads;
    const int64_t hq_stride = (int64_t)q_heads * head_dim;
    const int64_t gph = head_dim / 64;
    #pragma omp parallel for collapse(2) schedule(static)
    for (int32_t b = 0; b < batch; ++b)
        for (int32_t hq = 0; hq < q_heads; ++hq) {
            const int32_t kh = hq / R;
            double *s = (double *)malloc(sizeof(double) * (size_t)kv_len);
            double *o = (double *)calloc((size_t)head_dim, sizeof(double));
            const uint16_t *qv = q + (int64_t)b * hq_stride + (int64_t)hq * head_dim;
            const int64_t base = ((int64_t)b * kv_heads + kh) * cap;
            double mx = -INFINITY;
            for (int32_t j = 0; j < kv_len; ++j) {
                const uint8_t *kc = k_codes + (base + j) * (head_dim / 2);
                const uint32_t *km = k_meta + (base + j) * gph;
                double acc = 0.0;
                for (int32_t d = 0; d < head_dim; ++d)
                    acc += (double)oracle_f16_to_f32(qv[d]) * (double)dequant_one(km[d / 64], code_at(kc, d));
                s[j] = acc * scale;
                if (s[j] > mx) mx = s[j];
            }
            double den = 0.0;
            for (int32_t j = 0; j < kv_len; ++j) {
                s[j] = exp(s[j] - mx);
                den += s[j];
            }
            for (int32_t j = 0; j < kv_len; ++j) {
                const uint8_t *vc = v_codes + (base + j) * (head_dim / 2);
                const uint32_t *vm = v_meta + (base + j) * gph;
                for (int32_t d = 0; d < head_dim; ++d)
                    o[d] += s[j] * (double)dequant_one(vm[d / 64], code_at(vc, d));
            }
            float *ov = out + (int64_t)b * hq_stride + (int64_t)hq * head_dim;
            for (int32_t d = 0; d < head_dim; ++d) ov[d] = (float)(o[d] / den);
            free(s);
            free(o);
        }
    return ORACLE_OK;
}
