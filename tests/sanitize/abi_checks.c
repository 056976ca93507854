/* Host-side argument validation of libfgq under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every entry point and size query is called
 * with arguments that must be rejected before any HIP call (null, misaligned,
 * negative, ragged, out-of-range and overflow-sized shapes), and the size
 * queries with extreme values.  Pointers handed to the library are never
 * dereferenced on these paths; a sanitizer report or an unexpected status
 * fails the run.  No GPU is needed. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fgq.h"

#define A16 ((void *)(uintptr_t)0x7f0000000000ULL) /* aligned, never dereferenced */
#define MIS ((void *)(uintptr_t)0x7f0000000001ULL) /* misaligned, never dereferenced */

static int failures = 0;

static void expect(const char *what, fgq_status got, fgq_status want) {
    if (got != want) {
        fprintf(stderr, "FAIL %s: status %d (%s), expected %d; last error: %s\n", what, got,
                fgq_status_string(got), want, fgq_last_error());
        ++failures;
    }
}

static void expect_size(const char *what, size_t got, size_t want) {
    if (got != want) {
        fprintf(stderr, "FAIL %s: %zu, expected %zu\n", what, got, want);
        ++failures;
    }
}

static fgq_kv_cache kv_of(int32_t batch, int32_t heads, int32_t head_dim, int32_t cap) {
    fgq_kv_cache kv;
    kv.k_codes = (uint8_t *)A16;
    kv.v_codes = (uint8_t *)A16;
    kv.k_meta = (uint32_t *)A16;
    kv.v_meta = (uint32_t *)A16;
    kv.batch = batch;
    kv.heads = heads;
    kv.head_dim = head_dim;
    kv.capacity = cap;
    return kv;
}

static void strings(void) {
    for (int s = -12; s <= 2; ++s) {
        const char *t = fgq_status_string(s);
        if (!t || !t[0]) { fprintf(stderr, "FAIL status string %d\n", s); ++failures; }
    }
    if (fgq_abi_version() <= 0) { fprintf(stderr, "FAIL abi version\n"); ++failures; }
    (void)strlen(fgq_last_error());
}

static void quantize(void) {
    expect("quantize negative rows", fgq_quantize_g64(A16, -1, 64, 64, A16, A16, NULL), FGQ_ERR_INVALID_ARG);
    expect("quantize ragged cols", fgq_quantize_g64(A16, 4, 96, 96, A16, A16, NULL), FGQ_ERR_SHAPE);
    expect("quantize ld < cols", fgq_quantize_g64(A16, 4, 128, 64, A16, A16, NULL), FGQ_ERR_SHAPE);
    expect("quantize null x", fgq_quantize_g64(NULL, 4, 64, 64, A16, A16, NULL), FGQ_ERR_INVALID_ARG);
    expect("quantize misaligned", fgq_quantize_g64(MIS, 4, 64, 64, A16, A16, NULL), FGQ_ERR_ALIGN);
    expect("quantize ld % 8", fgq_quantize_g64(A16, 4, 64, 68, A16, A16, NULL), FGQ_ERR_ALIGN);
    expect("quantize empty", fgq_quantize_g64(NULL, 0, 64, 64, NULL, NULL, NULL), FGQ_OK);
    expect("quantize huge rows", fgq_quantize_g64(A16, INT64_MAX, 64, 64, A16, A16, NULL), FGQ_ERR_SHAPE);
    expect("quantize huge cols", fgq_quantize_g64(A16, 2, INT64_MAX - 63, INT64_MAX - 63, A16, A16, NULL),
           FGQ_ERR_SHAPE);
    expect("quantize huge ld", fgq_quantize_g64(A16, 2, 64, INT64_MAX - 7, A16, A16, NULL), FGQ_ERR_SHAPE);
}

static void append(void) {
    fgq_kv_cache kv = kv_of(2, 4, 128, 100);
    expect("append null kv", fgq_kv_append(NULL, A16, A16, 0, 1, NULL), FGQ_ERR_INVALID_ARG);
    expect("append negative pos", fgq_kv_append(&kv, A16, A16, -1, 1, NULL), FGQ_ERR_INVALID_ARG);
    expect("append over capacity", fgq_kv_append(&kv, A16, A16, 99, 2, NULL), FGQ_ERR_CAPACITY);
    expect("append pos+n overflow", fgq_kv_append(&kv, A16, A16, INT32_MAX, INT32_MAX, NULL), FGQ_ERR_CAPACITY);
    expect("append null k", fgq_kv_append(&kv, NULL, A16, 0, 1, NULL), FGQ_ERR_INVALID_ARG);
    expect("append misaligned", fgq_kv_append(&kv, MIS, A16, 0, 1, NULL), FGQ_ERR_ALIGN);
    expect("append_ld short ld", fgq_kv_append_ld(&kv, A16, A16, 511, 0, 1, NULL), FGQ_ERR_SHAPE);
    expect("append_ld ld % 8", fgq_kv_append_ld(&kv, A16, A16, 516, 0, 1, NULL), FGQ_ERR_ALIGN);
    expect("append_ld huge ld", fgq_kv_append_ld(&kv, A16, A16, INT64_MAX - 7, 0, 1, NULL), FGQ_ERR_SHAPE);
    expect("append no-op", fgq_kv_append(&kv, NULL, NULL, 5, 0, NULL), FGQ_OK);
    fgq_kv_cache bad = kv_of(2, 4, 96, 100);
    expect("append head_dim 96", fgq_kv_append(&bad, A16, A16, 0, 1, NULL), FGQ_ERR_SHAPE);
    bad = kv_of(2, 4, 256, 100);
    expect("append head_dim 256", fgq_kv_append(&bad, A16, A16, 0, 1, NULL), FGQ_ERR_UNSUPPORTED);
    bad = kv_of(-1, 4, 128, 100);
    expect("append negative batch", fgq_kv_append(&bad, A16, A16, 0, 1, NULL), FGQ_ERR_INVALID_ARG);
    bad = kv_of(2, 4, 128, 100);
    bad.v_meta = (uint32_t *)MIS;
    expect("append misaligned cache", fgq_kv_append(&bad, A16, A16, 0, 1, NULL), FGQ_ERR_ALIGN);
    bad = kv_of(INT32_MAX, INT32_MAX, 128, INT32_MAX);
    expect("append capacity beyond 2^30", fgq_kv_append(&bad, A16, A16, 0, 1, NULL), FGQ_ERR_SHAPE);
    bad = kv_of(1 << 20, 1 << 10, 128, 1 << 20);
    expect("append cache beyond 2^48 elements", fgq_kv_append(&bad, A16, A16, 0, 1, NULL), FGQ_ERR_SHAPE);
}

static void attention(void) {
    fgq_kv_cache kv = kv_of(2, 4, 128, 100);
    char ws[64];
    void *w = (void *)(((uintptr_t)ws + 15) & ~(uintptr_t)15);
    expect("attn null kv", fgq_decode_attn_q4kv(NULL, A16, 10, 0.f, A16, FGQ_DTYPE_F32, NULL, 0, NULL),
           FGQ_ERR_INVALID_ARG);
    expect("attn dtype", fgq_decode_attn_q4kv(&kv, A16, 10, 0.f, A16, 7, NULL, 0, NULL), FGQ_ERR_DTYPE);
    expect("attn kv_len 0", fgq_decode_attn_q4kv(&kv, A16, 0, 0.f, A16, FGQ_DTYPE_F32, NULL, 0, NULL),
           FGQ_ERR_SHAPE);
    expect("attn kv_len > cap", fgq_decode_attn_q4kv(&kv, A16, 101, 0.f, A16, FGQ_DTYPE_F32, NULL, 0, NULL),
           FGQ_ERR_CAPACITY);
    expect("attn nan scale", fgq_decode_attn_q4kv(&kv, A16, 10, 0.f / 0.f, A16, FGQ_DTYPE_F32, NULL, 0, NULL),
           FGQ_ERR_INVALID_ARG);
    expect("attn null q", fgq_decode_attn_q4kv(&kv, NULL, 10, 0.f, A16, FGQ_DTYPE_F32, NULL, 0, NULL),
           FGQ_ERR_INVALID_ARG);
    expect("attn misaligned out", fgq_decode_attn_q4kv(&kv, A16, 10, 0.f, MIS, FGQ_DTYPE_F32, NULL, 0, NULL),
           FGQ_ERR_ALIGN);
    expect("attn_ld short ld", fgq_decode_attn_q4kv_ld(&kv, A16, 8, 10, 0.f, A16, FGQ_DTYPE_F32, NULL, 0, NULL),
           FGQ_ERR_SHAPE);
    expect("attn_ld ld % 8", fgq_decode_attn_q4kv_ld(&kv, A16, 514, 10, 0.f, A16, FGQ_DTYPE_F32, NULL, 0, NULL),
           FGQ_ERR_ALIGN);
    /* 2 x 4 pairs split a 100-token context: a workspace is needed */
    expect("attn missing ws", fgq_decode_attn_q4kv(&kv, A16, 100, 0.f, A16, FGQ_DTYPE_F32, NULL, 0, NULL),
           fgq_decode_attn_ws_bytes(2, 4, 128, 100) > 0 ? FGQ_ERR_WORKSPACE : FGQ_ERR_DEVICE);
    expect("attn misaligned ws",
           fgq_decode_attn_q4kv(&kv, A16, 100, 0.f, A16, FGQ_DTYPE_F32, MIS, (size_t)1 << 40, NULL),
           fgq_decode_attn_ws_bytes(2, 4, 128, 100) > 0 ? FGQ_ERR_ALIGN : FGQ_ERR_DEVICE);
    (void)w;
    fgq_kv_cache big = kv_of(INT32_MAX, INT32_MAX, 128, INT32_MAX);
    expect("attn huge cache", fgq_decode_attn_q4kv(&big, A16, INT32_MAX, 0.f, A16, FGQ_DTYPE_F32, NULL, 0, NULL),
           FGQ_ERR_SHAPE);
    fgq_kv_cache wide = kv_of(1 << 20, 2, 64, 1 << 10);   /* 2^37 elements: valid; q rows huge */
    expect("attn_ld q beyond 2^48 elements",
           fgq_decode_attn_q4kv_ld(&wide, A16, (int64_t)1 << 40, 10, 0.f, A16, FGQ_DTYPE_F32, NULL, 0, NULL),
           FGQ_ERR_SHAPE);
    expect("noalloc null kv", fgq_decode_attn_q4kv_noalloc(NULL, A16, 10, 0.f, A16, FGQ_DTYPE_F32, NULL),
           FGQ_ERR_INVALID_ARG);
    expect("noalloc dtype", fgq_decode_attn_q4kv_noalloc(&kv, A16, 10, 0.f, A16, 3, NULL), FGQ_ERR_DTYPE);
    expect("noalloc kv_len > cap", fgq_decode_attn_q4kv_noalloc(&kv, A16, 101, 0.f, A16, FGQ_DTYPE_F32, NULL),
           FGQ_ERR_CAPACITY);

    /* grouped-query */
    expect("gqa negative q_heads", fgq_decode_attn_gqa_q4kv(&kv, A16, -4, 10, 0.f, A16, FGQ_DTYPE_F32, NULL, 0,
                                                            NULL), FGQ_ERR_INVALID_ARG);
    expect("gqa q_heads not a multiple", fgq_decode_attn_gqa_q4kv(&kv, A16, 6, 10, 0.f, A16, FGQ_DTYPE_F32, NULL, 0,
                                                                  NULL), FGQ_ERR_SHAPE);
    expect("gqa group too wide", fgq_decode_attn_gqa_q4kv(&kv, A16, 4 * 64, 10, 0.f, A16, FGQ_DTYPE_F32, NULL, 0,
                                                          NULL), FGQ_ERR_UNSUPPORTED);
    expect("gqa dtype", fgq_decode_attn_gqa_q4kv(&kv, A16, 8, 10, 0.f, A16, 9, NULL, 0, NULL), FGQ_ERR_DTYPE);
    expect("gqa kv_len > cap", fgq_decode_attn_gqa_q4kv(&kv, A16, 8, 101, 0.f, A16, FGQ_DTYPE_F32, NULL, 0, NULL),
           FGQ_ERR_CAPACITY);
    expect("gqa null q", fgq_decode_attn_gqa_q4kv(&kv, NULL, 8, 10, 0.f, A16, FGQ_DTYPE_F32, NULL, 0, NULL),
           FGQ_ERR_INVALID_ARG);
    expect("gqa huge cache", fgq_decode_attn_gqa_q4kv(&big, A16, INT32_MAX, INT32_MAX, 0.f, A16, FGQ_DTYPE_F32,
                                                      NULL, 0, NULL), FGQ_ERR_SHAPE);
    fgq_kv_cache zero_heads = kv_of(2, 0, 128, 100);
    expect("gqa zero kv heads", fgq_decode_attn_gqa_q4kv(&zero_heads, A16, 8, 10, 0.f, A16, FGQ_DTYPE_F32, NULL, 0,
                                                         NULL), FGQ_ERR_SHAPE);

    /* top-K */
    expect("topk top_k 0", fgq_decode_attn_topk_q4kv(&kv, A16, 10, 0, 0.f, A16, FGQ_DTYPE_F32, NULL, NULL),
           FGQ_ERR_INVALID_ARG);
    expect("topk dtype", fgq_decode_attn_topk_q4kv(&kv, A16, 10, 3, 0.f, A16, 5, NULL, NULL), FGQ_ERR_DTYPE);
    expect("topk misaligned sel", fgq_decode_attn_topk_q4kv(&kv, A16, 10, 3, 0.f, A16, FGQ_DTYPE_F32,
                                                            (int32_t *)MIS, NULL), FGQ_ERR_ALIGN);
    expect("topk huge cache", fgq_decode_attn_topk_q4kv(&big, A16, INT32_MAX, INT32_MAX, 0.f, A16, FGQ_DTYPE_F32,
                                                        NULL, NULL), FGQ_ERR_SHAPE);

    /* prefill */
    expect("prefill negative", fgq_prefill_attn_f16(A16, A16, A16, -1, 4, 4, 128, 0.f, A16, FGQ_DTYPE_F32, NULL),
           FGQ_ERR_INVALID_ARG);
    expect("prefill head_dim", fgq_prefill_attn_f16(A16, A16, A16, 1, 4, 4, 96, 0.f, A16, FGQ_DTYPE_F32, NULL),
           FGQ_ERR_SHAPE);
    expect("prefill dtype", fgq_prefill_attn_f16(A16, A16, A16, 1, 4, 4, 64, 0.f, A16, 2, NULL), FGQ_ERR_DTYPE);
    expect("prefill huge", fgq_prefill_attn_f16(A16, A16, A16, 65535, INT32_MAX, 65535, 128, 0.f, A16,
                                                FGQ_DTYPE_F32, NULL), FGQ_ERR_SHAPE);
    expect("prefill misaligned", fgq_prefill_attn_f16(A16, MIS, A16, 1, 4, 4, 128, 0.f, A16, FGQ_DTYPE_F32, NULL),
           FGQ_ERR_ALIGN);
    expect("prefill empty", fgq_prefill_attn_f16(NULL, NULL, NULL, 0, 4, 4, 128, 0.f, NULL, FGQ_DTYPE_F32, NULL),
           FGQ_OK);
}

static void gemm(void) {
    expect("gemm negative", fgq_dequant_gemm(A16, -1, 4, 64, 64, A16, A16, A16, 0, NULL, 0, NULL),
           FGQ_ERR_INVALID_ARG);
    expect("gemm K % 64", fgq_dequant_gemm(A16, 1, 4, 32, 64, A16, A16, A16, 0, NULL, 0, NULL), FGQ_ERR_SHAPE);
    expect("gemm N % 64", fgq_dequant_gemm(A16, 1, 4, 64, 96, A16, A16, A16, 0, NULL, 0, NULL), FGQ_ERR_SHAPE);
    expect("gemm dtype", fgq_dequant_gemm(A16, 1, 4, 64, 64, A16, A16, A16, 4, NULL, 0, NULL), FGQ_ERR_DTYPE);
    expect("gemm huge M", fgq_dequant_gemm(A16, INT32_MAX, INT32_MAX, 64, 64, A16, A16, A16, 0, NULL, 0, NULL),
           FGQ_ERR_SHAPE);
    expect("gemm huge K", fgq_dequant_gemm(A16, 1, 4, INT64_MAX - 63, 64, A16, A16, A16, 0, NULL, 0, NULL),
           FGQ_ERR_SHAPE);
    expect("gemm huge N", fgq_dequant_gemm(A16, 1, 4, 64, INT64_MAX - 63, A16, A16, A16, 0, NULL, 0, NULL),
           FGQ_ERR_SHAPE);
    expect("gemm null y", fgq_dequant_gemm(A16, 1, 4, 64, 64, A16, A16, NULL, 0, NULL, 0, NULL),
           FGQ_ERR_INVALID_ARG);
    expect("gemm misaligned", fgq_dequant_gemm(A16, 1, 4, 64, 64, MIS, A16, A16, 0, NULL, 0, NULL), FGQ_ERR_ALIGN);
    expect("gemm empty", fgq_dequant_gemm(NULL, 0, 4, 64, 64, NULL, NULL, NULL, 0, NULL, 0, NULL), FGQ_OK);
    /* a 144 x 12288 x 12288 product splits K: the workspace is checked */
    const size_t need = fgq_dequant_gemm_ws_bytes(144, 12288, 12288);
    expect("gemm missing ws", fgq_dequant_gemm(A16, 36, 4, 12288, 12288, A16, A16, A16, 0, NULL, 0, NULL),
           need > 0 ? FGQ_ERR_WORKSPACE : FGQ_ERR_DEVICE);
    expect("gemm small ws", fgq_dequant_gemm(A16, 36, 4, 12288, 12288, A16, A16, A16, 0, A16, need - 1, NULL),
           need > 0 ? FGQ_ERR_WORKSPACE : FGQ_ERR_DEVICE);
    expect("packed K % 32", fgq_dequant_gemm_packed(A16, 1, 4, 48, 64, A16, A16, A16, 0, NULL, 0, NULL),
           FGQ_ERR_SHAPE);
    expect("packed huge N", fgq_dequant_gemm_packed(A16, 1, 4, 64, ((int64_t)1 << 28) + 64, A16, A16, A16, 0,
                                                    NULL, 0, NULL), FGQ_ERR_SHAPE);
    expect("packed misaligned ws", fgq_dequant_gemm_packed(A16, 36, 4, 12288, 12288, A16, A16, A16, 0, MIS,
                                                           (size_t)1 << 40, NULL),
           need > 0 ? FGQ_ERR_ALIGN : FGQ_ERR_DEVICE);
    expect("pack negative", fgq_pack_weight_g64(A16, A16, -32, 64, A16, A16, NULL), FGQ_ERR_INVALID_ARG);
    expect("pack K % 32", fgq_pack_weight_g64(A16, A16, 48, 64, A16, A16, NULL), FGQ_ERR_SHAPE);
    expect("pack null", fgq_pack_weight_g64(NULL, A16, 64, 64, A16, A16, NULL), FGQ_ERR_INVALID_ARG);
    expect("pack misaligned", fgq_pack_weight_g64(A16, MIS, 64, 64, A16, A16, NULL), FGQ_ERR_ALIGN);
    expect("pack huge", fgq_pack_weight_g64(A16, A16, INT64_MAX - 31, INT64_MAX - 63, A16, A16, NULL),
           FGQ_ERR_SHAPE);
}

static void sizes(void) {
    const int32_t i32[] = {INT32_MIN, -1, 0, 1, 2, 63, 64, 127, 128, 4096, 65535, 1 << 20, INT32_MAX - 1, INT32_MAX};
    const int n32 = (int)(sizeof(i32) / sizeof(i32[0]));
    for (int a = 0; a < n32; ++a)
        for (int b = 0; b < n32; ++b)
            for (int c = 0; c < n32; ++c) {
                (void)fgq_decode_attn_ws_bytes(i32[a], i32[b], 128, i32[c]);
                (void)fgq_decode_attn_ws_bytes(i32[a], i32[b], 64, i32[c]);
                (void)fgq_decode_attn_gqa_ws_bytes(i32[a], 8 * (i32[b] / 8 > 0 ? i32[b] / 8 : 1), i32[b] / 8,
                                                   128, i32[c]);
                (void)fgq_decode_attn_gqa_ws_bytes(i32[a], i32[b], i32[b], 64, i32[c]);
            }
    const int64_t i64[] = {INT64_MIN, -64, 0, 32, 64, 144, 4096, 12288, 49152, (int64_t)1 << 23,
                           (int64_t)1 << 28, (int64_t)1 << 30, (int64_t)1 << 40, INT64_MAX - 63, INT64_MAX};
    const int n64 = (int)(sizeof(i64) / sizeof(i64[0]));
    for (int a = 0; a < n64; ++a)
        for (int b = 0; b < n64; ++b) {
            (void)fgq_pack_weight_meta_words(i64[a], i64[b]);
            for (int c = 0; c < n64; ++c) (void)fgq_dequant_gemm_ws_bytes(i64[a], i64[b], i64[c]);
        }
    expect_size("attn ws of invalid head_dim", fgq_decode_attn_ws_bytes(1, 1, 96, 100), 0);
    expect_size("gemm ws of ragged K", fgq_dequant_gemm_ws_bytes(144, 48, 64), 0);
    expect_size("gemm ws beyond the entry points' limits", fgq_dequant_gemm_ws_bytes((int64_t)1 << 40, 64, 64), 0);
    expect_size("pack meta words beyond the limits", fgq_pack_weight_meta_words((int64_t)1 << 40, 64), 0);
    expect_size("pack meta words", fgq_pack_weight_meta_words(64, 128), 64 * 2 + 2);
}

int main(void) {
    strings();
    quantize();
    append();
    attention();
    gemm();
    sizes();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("abi checks ok\n");
    return 0;
}
