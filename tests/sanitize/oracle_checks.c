/* The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.
 * Every function runs on small ragged shapes with heap buffers of exactly
 * the documented size (so a read or write one element past an array is
 * reported), on the edge cases (kv_len == capacity, kv_len == 1, top_k above
 * kv_len, partial prefill row ranges, K == 0), and with arguments it must
 * reject, including sizes whose sums overflow 32 bits.  Outputs must be
 * finite.  Built from oracle.c itself; links nothing else. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#define ORACLE_OK 0
#define ORACLE_ERR_SHAPE -2
#define ORACLE_ERR_NONFINITE -9

float oracle_f16_to_f32(uint16_t h);
uint16_t oracle_f32_to_f16(float x);
int oracle_quantize_g64(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t *codes,
                        uint32_t *meta);
int oracle_dequant_g64(const uint8_t *codes, const uint32_t *meta, int64_t rows, int64_t cols, float *out);
int oracle_kv_append(const uint16_t *k_new, const uint16_t *v_new, int32_t batch, int32_t heads, int32_t head_dim,
                     int32_t cap, int32_t pos, int32_t n_new, uint8_t *k_codes, uint32_t *k_meta, uint8_t *v_codes,
                     uint32_t *v_meta);
int oracle_decode_attn(const uint16_t *q, int32_t batch, int32_t heads, int32_t head_dim, int32_t cap,
                       const uint8_t *k_codes, const uint32_t *k_meta, const uint8_t *v_codes,
                       const uint32_t *v_meta, int32_t kv_len, double scale, float *out);
int oracle_decode_attn_topk(const uint16_t *q, int32_t batch, int32_t heads, int32_t head_dim, int32_t cap,
                            const uint8_t *k_codes, const uint32_t *k_meta, const uint8_t *v_codes,
                            const uint32_t *v_meta, int32_t kv_len, int32_t top_k, double scale, float *out,
                            int32_t *sel);
int oracle_prefill_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v, int32_t batch, int32_t seq,
                        int32_t heads, int32_t head_dim, int32_t row0, int32_t row1, double scale, float *out);
int oracle_dequant_gemm(const uint16_t *x, int32_t g, int32_t m, int64_t K, int64_t N, const uint8_t *w_codes,
                        const uint32_t *w_meta, float *y);
int oracle_decode_attn_gqa(const uint16_t *q, int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                           int32_t cap, const uint8_t *k_codes, const uint32_t *k_meta, const uint8_t *v_codes,
                           const uint32_t *v_meta, int32_t kv_len, double scale, float *out);

static int failures = 0;
static uint64_t rng_state = 0x9e3779b97f4a7c15ULL;

static void check(const char *what, int got, int want) {
    if (got != want) {
        fprintf(stderr, "FAIL %s: %d, expected %d\n", what, got, want);
        ++failures;
    }
}

static void finite(const char *what, const float *a, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(a[i])) {
            fprintf(stderr, "FAIL %s: non-finite output at %lld\n", what, (long long)i);
            ++failures;
            return;
        }
}

/* fp16 values in about [-2, 2] (a small test pattern, not a distribution) */
static uint16_t *halves(int64_t n) {
    uint16_t *a = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) {
        rng_state = rng_state * 6364136223846793005ULL + 1442695040888963407ULL;
        const double u = (double)(rng_state >> 11) / 9007199254740992.0;
        a[i] = oracle_f32_to_f16((float)(4.0 * u - 2.0));
    }
    return a;
}

static void conversions(void) {
    for (uint32_t h = 0; h < 65536; ++h) {
        const float f = oracle_f16_to_f32((uint16_t)h);
        if (isnan(f)) continue;
        if (oracle_f32_to_f16(f) != (uint16_t)h) {
            fprintf(stderr, "FAIL fp16 round trip of 0x%04x\n", h);
            ++failures;
            return;
        }
    }
}

static void weights(void) {
    const int64_t rows = 3, cols = 128, ld = 136;
    uint16_t *x = halves((rows - 1) * ld + cols);   /* the last row ends at its last used column */
    uint8_t *codes = (uint8_t *)malloc((size_t)(rows * cols / 2));
    uint32_t *meta = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(rows * cols / 64));
    float *back = (float *)malloc(sizeof(float) * (size_t)(rows * cols));
    check("quantize", oracle_quantize_g64(x, rows, cols, ld, codes, meta), ORACLE_OK);
    check("dequant", oracle_dequant_g64(codes, meta, rows, cols, back), ORACLE_OK);
    finite("dequant", back, rows * cols);
    check("quantize ragged cols", oracle_quantize_g64(x, rows, 96, ld, codes, meta), ORACLE_ERR_SHAPE);
    check("quantize ld < cols", oracle_quantize_g64(x, rows, cols, 64, codes, meta), ORACLE_ERR_SHAPE);
    check("quantize negative", oracle_quantize_g64(x, -1, cols, ld, codes, meta), ORACLE_ERR_SHAPE);
    const uint16_t inf = 0x7c00;
    uint16_t *y = halves(64);
    y[17] = inf;
    check("quantize non-finite", oracle_quantize_g64(y, 1, 64, 64, codes, meta), ORACLE_ERR_NONFINITE);
    free(y);
    free(back);

    /* block GEMM: M = 3 rows, K = 96, N = 128, and K == 0 */
    const int32_t g = 3, m = 1;
    const int64_t K = 96, N = 128, M = (int64_t)g * m;
    uint16_t *w = halves(K * N);
    uint8_t *wc = (uint8_t *)malloc((size_t)(K * N / 2));
    uint32_t *wm = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(K * N / 64));
    check("quantize weight", oracle_quantize_g64(w, K, N, N, wc, wm), ORACLE_OK);
    uint16_t *xx = halves(M * K);
    float *out = (float *)malloc(sizeof(float) * (size_t)(M * N));
    check("gemm", oracle_dequant_gemm(xx, g, m, K, N, wc, wm, out), ORACLE_OK);
    finite("gemm", out, M * N);
    check("gemm K = 0", oracle_dequant_gemm(xx, g, m, 0, N, wc, wm, out), ORACLE_OK);
    for (int64_t i = 0; i < M * N; ++i)
        if (out[i] != 0.0f) { fprintf(stderr, "FAIL gemm K = 0 not zero\n"); ++failures; break; }
    check("gemm ragged N", oracle_dequant_gemm(xx, g, m, K, 96, wc, wm, out), ORACLE_ERR_SHAPE);
    check("gemm negative", oracle_dequant_gemm(xx, -1, m, K, N, wc, wm, out), ORACLE_ERR_SHAPE);
    free(x); free(codes); free(meta); free(w); free(wc); free(wm); free(xx); free(out);
}

struct cache {
    int32_t batch, heads, head_dim, cap;
    uint8_t *kc, *vc;
    uint32_t *km, *vm;
};

static struct cache cache_new(int32_t batch, int32_t heads, int32_t head_dim, int32_t cap) {
    struct cache c = {batch, heads, head_dim, cap, NULL, NULL, NULL, NULL};
    const int64_t slots = (int64_t)batch * heads * cap;
    c.kc = (uint8_t *)calloc((size_t)(slots * head_dim / 2), 1);
    c.vc = (uint8_t *)calloc((size_t)(slots * head_dim / 2), 1);
    c.km = (uint32_t *)calloc((size_t)(slots * head_dim / 64), sizeof(uint32_t));
    c.vm = (uint32_t *)calloc((size_t)(slots * head_dim / 64), sizeof(uint32_t));
    return c;
}

static void cache_free(struct cache *c) {
    free(c->kc); free(c->vc); free(c->km); free(c->vm);
}

static int fill(struct cache *c, int32_t pos, int32_t n_new) {
    const int64_t n = (int64_t)c->batch * n_new * c->heads * c->head_dim;
    uint16_t *k = halves(n), *v = halves(n);
    const int r = oracle_kv_append(k, v, c->batch, c->heads, c->head_dim, c->cap, pos, n_new, c->kc, c->km, c->vc,
                                   c->vm);
    free(k);
    free(v);
    return r;
}

static void attention(void) {
    for (int hd = 64; hd <= 128; hd += 64) {
        struct cache c = cache_new(2, 3, hd, 5);
        check("append prompt", fill(&c, 0, 3), ORACLE_OK);
        check("append to capacity", fill(&c, 3, 2), ORACLE_OK);
        check("append past capacity", fill(&c, 4, 2), ORACLE_ERR_SHAPE);
        check("append pos + n_new overflows int32",
              oracle_kv_append(NULL, NULL, 2, 3, hd, 5, INT32_MAX, INT32_MAX, c.kc, c.km, c.vc, c.vm),
              ORACLE_ERR_SHAPE);
        check("append no-op", fill(&c, 5, 0), ORACLE_OK);
        const int64_t qn = (int64_t)c.batch * c.heads * hd;
        uint16_t *q = halves(qn);
        float *out = (float *)malloc(sizeof(float) * (size_t)qn);
        for (int32_t L = 1; L <= c.cap; L += c.cap - 1) {
            check("attention", oracle_decode_attn(q, c.batch, c.heads, hd, c.cap, c.kc, c.km, c.vc, c.vm, L,
                                                  1.0 / sqrt((double)hd), out), ORACLE_OK);
            finite("attention", out, qn);
            for (int32_t tk = 1; tk <= 9; tk += 4) {
                const int32_t kk = tk < L ? tk : L;
                int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)(c.batch * c.heads * kk));
                check("top-k", oracle_decode_attn_topk(q, c.batch, c.heads, hd, c.cap, c.kc, c.km, c.vc, c.vm, L,
                                                       tk, 0.125, out, sel), ORACLE_OK);
                finite("top-k", out, qn);
                for (int64_t i = 0; i < (int64_t)c.batch * c.heads * kk; ++i)
                    if (sel[i] < 0 || sel[i] >= L) { fprintf(stderr, "FAIL top-k index\n"); ++failures; break; }
                free(sel);
            }
        }
        check("attention kv_len 0", oracle_decode_attn(q, c.batch, c.heads, hd, c.cap, c.kc, c.km, c.vc, c.vm, 0,
                                                       0.1, out), ORACLE_ERR_SHAPE);
        check("attention kv_len > cap", oracle_decode_attn(q, c.batch, c.heads, hd, c.cap, c.kc, c.km, c.vc, c.vm,
                                                           6, 0.1, out), ORACLE_ERR_SHAPE);
        check("top-k k 0", oracle_decode_attn_topk(q, c.batch, c.heads, hd, c.cap, c.kc, c.km, c.vc, c.vm, 3, 0,
                                                   0.1, out, NULL), ORACLE_ERR_SHAPE);
        free(q);
        free(out);
        cache_free(&c);

        /* grouped-query: 4 query heads over 2 K/V heads */
        struct cache g = cache_new(2, 2, hd, 6);
        check("append gqa", fill(&g, 0, 6), ORACLE_OK);
        const int64_t gn = (int64_t)g.batch * 4 * hd;
        uint16_t *gq = halves(gn);
        float *gout = (float *)malloc(sizeof(float) * (size_t)gn);
        check("gqa", oracle_decode_attn_gqa(gq, g.batch, 4, 2, hd, g.cap, g.kc, g.km, g.vc, g.vm, 6, 0.1, gout),
              ORACLE_OK);
        finite("gqa", gout, gn);
        check("gqa ragged group", oracle_decode_attn_gqa(gq, g.batch, 3, 2, hd, g.cap, g.kc, g.km, g.vc, g.vm, 6,
                                                         0.1, gout), ORACLE_ERR_SHAPE);
        free(gq);
        free(gout);
        cache_free(&g);
    }
}

static void prefill(void) {
    const int32_t batch = 2, seq = 7, heads = 2, hd = 64;
    const int64_t n = (int64_t)batch * seq * heads * hd;
    uint16_t *q = halves(n), *k = halves(n), *v = halves(n);
    float *out = (float *)malloc(sizeof(float) * (size_t)n);
    check("prefill", oracle_prefill_attn(q, k, v, batch, seq, heads, hd, 0, seq, 0.125, out), ORACLE_OK);
    finite("prefill", out, n);
    check("prefill rows 3..5", oracle_prefill_attn(q, k, v, batch, seq, heads, hd, 3, 5, 0.125, out), ORACLE_OK);
    check("prefill empty rows", oracle_prefill_attn(q, k, v, batch, seq, heads, hd, 4, 4, 0.125, out), ORACLE_OK);
    check("prefill row1 > seq", oracle_prefill_attn(q, k, v, batch, seq, heads, hd, 0, 8, 0.125, out),
          ORACLE_ERR_SHAPE);
    free(q); free(k); free(v); free(out);
}

int main(void) {
    conversions();
    weights();
    attention();
    prefill();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle checks ok\n");
    return 0;
}
