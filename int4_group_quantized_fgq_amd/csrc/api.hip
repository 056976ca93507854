// extern "C" entry points of libfgq: argument validation on the host (nothing
// is enqueued when a check fails), then the launches.
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "common.h"

namespace fgq {

fgq_status launch_quantize(const void *x, int64_t rows, int64_t cols, int64_t ld, uint8_t *codes,
                           uint32_t *meta, hipStream_t stream);
fgq_status launch_kv_append(const fgq_kv_cache *kv, const void *k_new, const void *v_new, int64_t ld, int32_t pos,
                            int32_t n_new, hipStream_t stream);
fgq_status launch_pack_weight(const uint8_t *codes, const uint32_t *meta, int64_t K, int64_t N,
                              uint32_t *packed_codes, uint32_t *packed_meta, hipStream_t stream);
size_t attn_ws_bytes(int32_t batch, int32_t heads, int32_t head_dim, int32_t kv_len);
size_t attn_scratch_bytes();
fgq_status attn_scratch_ptr(void **ptr);
fgq_status launch_decode_attn(const fgq_kv_cache *kv, const void *q, int64_t ld_q, int32_t kv_len, float scale,
                              void *out, int32_t out_dtype, void *ws, hipStream_t stream);
size_t gqa_ws_bytes(int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t head_dim, int32_t kv_len);
fgq_status launch_decode_attn_gqa(const fgq_kv_cache *kv, const void *q, int32_t q_heads, int32_t kv_len,
                                  float scale, void *out, int32_t out_dtype, void *ws, hipStream_t stream);
fgq_status launch_decode_attn_topk(const fgq_kv_cache *kv, const void *q, int32_t kv_len, int32_t kept,
                                   float scale, void *out, int32_t out_dtype, int32_t *sel, hipStream_t stream);
fgq_status launch_prefill_attn(const void *q, const void *k, const void *v, int32_t batch, int32_t seq,
                               int32_t heads, int32_t head_dim, float scale, void *out, int32_t out_dtype,
                               hipStream_t stream);
size_t gemm_ws_bytes(int64_t M, int64_t K, int64_t N);
fgq_status launch_dequant_gemm(const void *x, int64_t M, int64_t K, int64_t N, const void *wc, const uint32_t *wm,
                               bool canonical, void *y, int32_t y_dtype, void *ws, hipStream_t stream);

static thread_local char g_err[512];

// Size limits that keep every host and device offset computation inside
// 64-bit (host) and the kernels' index types: at most 2^48 elements in any
// one array, 2^30 cache positions per sequence.
constexpr double kMaxElems = 281474976710656.0;   // 2^48
constexpr int32_t kMaxCapacity = 1 << 30;
// GEMM limits: rows of the block, K, N (packed layout; the canonical layout
// takes half that N).
constexpr int64_t kMaxM = (int64_t)1 << 30;
constexpr int64_t kMaxK = (int64_t)1 << 23;
constexpr int64_t kMaxNPacked = (int64_t)1 << 28;

fgq_status fail(fgq_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

fgq_status check_launch(const char *what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(FGQ_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
    return FGQ_OK;
}

static fgq_status check_kv(const fgq_kv_cache *kv) {
    if (!kv) return fail(FGQ_ERR_INVALID_ARG, "kv is NULL");
    if (kv->batch < 0 || kv->heads < 0 || kv->capacity < 0 || kv->head_dim <= 0)
        return fail(FGQ_ERR_INVALID_ARG, "negative kv dimension");
    if (kv->head_dim != 64 && kv->head_dim != 128) {
        if (kv->head_dim % 64 != 0) return fail(FGQ_ERR_SHAPE, "head_dim %d is not a multiple of 64", kv->head_dim);
        return fail(FGQ_ERR_UNSUPPORTED, "head_dim %d (64 or 128 supported)", kv->head_dim);
    }
    if (kv->capacity > kMaxCapacity)
        return fail(FGQ_ERR_SHAPE, "capacity %d above 2^30 positions", kv->capacity);
    if ((double)kv->batch * kv->heads * kv->capacity * kv->head_dim > kMaxElems)
        return fail(FGQ_ERR_SHAPE, "cache of batch %d x heads %d x capacity %d x head_dim %d above 2^48 elements",
                    kv->batch, kv->heads, kv->capacity, kv->head_dim);
    if (!kv->k_codes || !kv->v_codes || !kv->k_meta || !kv->v_meta)
        return fail(FGQ_ERR_INVALID_ARG, "kv array is NULL");
    if (!aligned16(kv->k_codes) || !aligned16(kv->v_codes) || !aligned16(kv->k_meta) || !aligned16(kv->v_meta))
        return fail(FGQ_ERR_ALIGN, "kv arrays must be 16-byte aligned");
    return FGQ_OK;
}

}  // namespace fgq

using namespace fgq;

extern "C" {

int32_t fgq_abi_version(void) { return FGQ_ABI_VERSION; }

const char *fgq_status_string(fgq_status s) {
    switch (s) {
        case FGQ_OK: return "ok";
        case FGQ_ERR_INVALID_ARG: return "invalid argument";
        case FGQ_ERR_SHAPE: return "bad shape";
        case FGQ_ERR_ALIGN: return "misaligned array";
        case FGQ_ERR_CAPACITY: return "kv capacity exceeded";
        case FGQ_ERR_WORKSPACE: return "workspace too small";
        case FGQ_ERR_DTYPE: return "unsupported dtype";
        case FGQ_ERR_DEVICE: return "device error";
        case FGQ_ERR_UNSUPPORTED: return "unsupported configuration";
        default: return "unknown status";
    }
}

const char *fgq_last_error(void) { return g_err; }

fgq_status fgq_quantize_g64(const void *x_f16, int64_t rows, int64_t cols, int64_t ld_x, uint8_t *codes,
                            uint32_t *meta, void *stream) {
    g_err[0] = 0;
    if (rows < 0 || cols < 0) return fail(FGQ_ERR_INVALID_ARG, "negative size");
    if (cols % 64 != 0) return fail(FGQ_ERR_SHAPE, "cols %lld is not a multiple of 64", (long long)cols);
    if (ld_x < cols) return fail(FGQ_ERR_SHAPE, "ld_x %lld < cols %lld", (long long)ld_x, (long long)cols);
    if ((double)rows * ld_x > kMaxElems || cols / 64 > INT32_MAX)
        return fail(FGQ_ERR_SHAPE, "x of %lld rows x ld %lld above 2^48 elements", (long long)rows, (long long)ld_x);
    if (rows == 0 || cols == 0) return FGQ_OK;
    if (!x_f16 || !codes || !meta) return fail(FGQ_ERR_INVALID_ARG, "NULL array");
    if (ld_x % 8 != 0 || !aligned16(x_f16) || !aligned16(codes) || !aligned16(meta))
        return fail(FGQ_ERR_ALIGN, "arrays and rows must be 16-byte aligned");
    return launch_quantize(x_f16, rows, cols, ld_x, codes, meta, static_cast<hipStream_t>(stream));
}

fgq_status fgq_kv_append_ld(const fgq_kv_cache *kv, const void *k_new_f16, const void *v_new_f16, int64_t ld_new,
                            int32_t pos, int32_t n_new, void *stream) {
    g_err[0] = 0;
    fgq_status s = check_kv(kv);
    if (s != FGQ_OK) return s;
    if (pos < 0 || n_new < 0) return fail(FGQ_ERR_INVALID_ARG, "negative pos or n_new");
    if ((int64_t)pos + n_new > kv->capacity)
        return fail(FGQ_ERR_CAPACITY, "pos %d + n_new %d > capacity %d", pos, n_new, kv->capacity);
    const int64_t hidden = (int64_t)kv->heads * kv->head_dim;
    if (ld_new < hidden) return fail(FGQ_ERR_SHAPE, "ld_new %lld < heads * head_dim %lld", (long long)ld_new,
                                     (long long)hidden);
    if ((double)kv->batch * n_new * ld_new > kMaxElems)
        return fail(FGQ_ERR_SHAPE, "k_new/v_new of batch %d x n_new %d x ld %lld above 2^48 elements", kv->batch,
                    n_new, (long long)ld_new);
    if (n_new == 0 || kv->batch == 0 || kv->heads == 0) return FGQ_OK;
    if (!k_new_f16 || !v_new_f16) return fail(FGQ_ERR_INVALID_ARG, "NULL k_new or v_new");
    if (!aligned16(k_new_f16) || !aligned16(v_new_f16) || ld_new % 8 != 0)
        return fail(FGQ_ERR_ALIGN, "k_new/v_new and their rows must be 16-byte aligned");
    return launch_kv_append(kv, k_new_f16, v_new_f16, ld_new, pos, n_new, static_cast<hipStream_t>(stream));
}

fgq_status fgq_kv_append(const fgq_kv_cache *kv, const void *k_new_f16, const void *v_new_f16, int32_t pos,
                         int32_t n_new, void *stream) {
    const int64_t hidden = kv ? (int64_t)kv->heads * kv->head_dim : 0;
    return fgq_kv_append_ld(kv, k_new_f16, v_new_f16, hidden, pos, n_new, stream);
}

size_t fgq_decode_attn_ws_bytes(int32_t batch, int32_t heads, int32_t head_dim, int32_t kv_len) {
    if (batch <= 0 || heads <= 0 || (head_dim != 64 && head_dim != 128) || kv_len <= 0 || kv_len > kMaxCapacity)
        return 0;
    return attn_ws_bytes(batch, heads, head_dim, kv_len);
}

// Host validation shared by the dense decode attention entry points (nothing
// about the workspace); *noop is set when there is nothing to compute.
static fgq_status check_attn(const fgq_kv_cache *kv, const void *q_f16, int64_t ld_q, int32_t kv_len,
                             float softmax_scale, const void *out, int32_t out_dtype, bool *noop) {
    *noop = false;
    fgq_status s = check_kv(kv);
    if (s != FGQ_OK) return s;
    if (out_dtype != FGQ_DTYPE_F32 && out_dtype != FGQ_DTYPE_F16)
        return fail(FGQ_ERR_DTYPE, "out_dtype %d", out_dtype);
    if (kv_len < 1) return fail(FGQ_ERR_SHAPE, "kv_len %d < 1", kv_len);
    if (kv_len > kv->capacity) return fail(FGQ_ERR_CAPACITY, "kv_len %d > capacity %d", kv_len, kv->capacity);
    if (!std::isfinite(softmax_scale)) return fail(FGQ_ERR_INVALID_ARG, "softmax_scale is not finite");
    const int64_t hidden = (int64_t)kv->heads * kv->head_dim;
    if (ld_q < hidden) return fail(FGQ_ERR_SHAPE, "ld_q %lld < heads * head_dim %lld", (long long)ld_q,
                                   (long long)hidden);
    if ((int64_t)kv->batch * kv->heads > INT32_MAX) return fail(FGQ_ERR_SHAPE, "batch * heads > 2^31 - 1");
    if ((double)kv->batch * ld_q > kMaxElems)
        return fail(FGQ_ERR_SHAPE, "q of batch %d x ld %lld above 2^48 elements", kv->batch, (long long)ld_q);
    if (kv->batch == 0 || kv->heads == 0) {
        *noop = true;
        return FGQ_OK;
    }
    if (!q_f16 || !out) return fail(FGQ_ERR_INVALID_ARG, "NULL q or out");
    if (!aligned16(q_f16) || !aligned16(out) || ld_q % 8 != 0)
        return fail(FGQ_ERR_ALIGN, "q (and its rows) and out must be 16-byte aligned");
    return FGQ_OK;
}

fgq_status fgq_decode_attn_q4kv_noalloc(const fgq_kv_cache *kv, const void *q_f16, int32_t kv_len,
                                        float softmax_scale, void *out, int32_t out_dtype, void *stream) {
    g_err[0] = 0;
    bool noop = false;
    const int64_t ld_q = kv ? (int64_t)kv->heads * kv->head_dim : 0;
    fgq_status s = check_attn(kv, q_f16, ld_q, kv_len, softmax_scale, out, out_dtype, &noop);
    if (s != FGQ_OK || noop) return s;
    const size_t need = attn_ws_bytes(kv->batch, kv->heads, kv->head_dim, kv_len);
    if (need > attn_scratch_bytes())
        return fail(FGQ_ERR_WORKSPACE, "split states need %zu bytes, more than the library's %zu-byte scratch",
                    need, attn_scratch_bytes());
    void *ws = nullptr;
    if (need > 0) {
        s = attn_scratch_ptr(&ws);
        if (s != FGQ_OK) return s;
    }
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)kv->head_dim);
    return launch_decode_attn(kv, q_f16, ld_q, kv_len, scale, out, out_dtype, ws, static_cast<hipStream_t>(stream));
}

fgq_status fgq_decode_attn_q4kv_ld(const fgq_kv_cache *kv, const void *q_f16, int64_t ld_q, int32_t kv_len,
                                   float softmax_scale, void *out, int32_t out_dtype, void *ws, size_t ws_bytes,
                                   void *stream) {
    g_err[0] = 0;
    bool noop = false;
    fgq_status s = check_attn(kv, q_f16, ld_q, kv_len, softmax_scale, out, out_dtype, &noop);
    if (s != FGQ_OK || noop) return s;
    const size_t need = attn_ws_bytes(kv->batch, kv->heads, kv->head_dim, kv_len);
    if (need > 0) {
        if (!ws || ws_bytes < need)
            return fail(FGQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : (size_t)0, need);
        if (!aligned16(ws)) return fail(FGQ_ERR_ALIGN, "workspace must be 16-byte aligned");
    }
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)kv->head_dim);
    return launch_decode_attn(kv, q_f16, ld_q, kv_len, scale, out, out_dtype, ws, static_cast<hipStream_t>(stream));
}

fgq_status fgq_decode_attn_q4kv(const fgq_kv_cache *kv, const void *q_f16, int32_t kv_len, float softmax_scale,
                                void *out, int32_t out_dtype, void *ws, size_t ws_bytes, void *stream) {
    const int64_t hidden = kv ? (int64_t)kv->heads * kv->head_dim : 0;
    return fgq_decode_attn_q4kv_ld(kv, q_f16, hidden, kv_len, softmax_scale, out, out_dtype, ws, ws_bytes, stream);
}

size_t fgq_decode_attn_gqa_ws_bytes(int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                                    int32_t kv_len) {
    if (batch <= 0 || kv_heads <= 0 || q_heads < kv_heads || q_heads % kv_heads != 0 ||
        q_heads / kv_heads > FGQ_GQA_MAX_GROUP || (head_dim != 64 && head_dim != 128) || kv_len <= 0 ||
        kv_len > kMaxCapacity)
        return 0;
    if (q_heads == kv_heads) return attn_ws_bytes(batch, q_heads, head_dim, kv_len);
    return gqa_ws_bytes(batch, q_heads, kv_heads, head_dim, kv_len);
}

fgq_status fgq_decode_attn_gqa_q4kv(const fgq_kv_cache *kv, const void *q_f16, int32_t q_heads, int32_t kv_len,
                                    float softmax_scale, void *out, int32_t out_dtype, void *ws, size_t ws_bytes,
                                    void *stream) {
    g_err[0] = 0;
    fgq_status s = check_kv(kv);
    if (s != FGQ_OK) return s;
    if (q_heads < 0) return fail(FGQ_ERR_INVALID_ARG, "negative q_heads");
    if (kv->heads == 0 || q_heads < kv->heads || q_heads % kv->heads != 0)
        return fail(FGQ_ERR_SHAPE, "q_heads %d is not a positive multiple of kv heads %d", q_heads, kv->heads);
    if (q_heads / kv->heads > FGQ_GQA_MAX_GROUP)
        return fail(FGQ_ERR_UNSUPPORTED, "%d query heads per K/V head (at most %d)", q_heads / kv->heads,
                    FGQ_GQA_MAX_GROUP);
    if (out_dtype != FGQ_DTYPE_F32 && out_dtype != FGQ_DTYPE_F16)
        return fail(FGQ_ERR_DTYPE, "out_dtype %d", out_dtype);
    if (kv_len < 1) return fail(FGQ_ERR_SHAPE, "kv_len %d < 1", kv_len);
    if (kv_len > kv->capacity) return fail(FGQ_ERR_CAPACITY, "kv_len %d > capacity %d", kv_len, kv->capacity);
    if (!std::isfinite(softmax_scale)) return fail(FGQ_ERR_INVALID_ARG, "softmax_scale is not finite");
    if ((int64_t)kv->batch * q_heads > INT32_MAX) return fail(FGQ_ERR_SHAPE, "batch * q_heads > 2^31 - 1");
    if (q_heads != kv->heads && (int64_t)kv->capacity * (kv->head_dim / 2) > UINT32_MAX)
        return fail(FGQ_ERR_UNSUPPORTED, "capacity %d: one head's code rows exceed 2^32 bytes", kv->capacity);
    if (kv->batch == 0) return FGQ_OK;
    if (!q_f16 || !out) return fail(FGQ_ERR_INVALID_ARG, "NULL q or out");
    if (!aligned16(q_f16) || !aligned16(out)) return fail(FGQ_ERR_ALIGN, "q/out must be 16-byte aligned");
    const bool mha = q_heads == kv->heads;
    const size_t need = mha ? attn_ws_bytes(kv->batch, kv->heads, kv->head_dim, kv_len)
                            : gqa_ws_bytes(kv->batch, q_heads, kv->heads, kv->head_dim, kv_len);
    if (need > 0) {
        if (!ws || ws_bytes < need)
            return fail(FGQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : (size_t)0, need);
        if (!aligned16(ws)) return fail(FGQ_ERR_ALIGN, "workspace must be 16-byte aligned");
    }
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)kv->head_dim);
    if (mha)
        return launch_decode_attn(kv, q_f16, (int64_t)kv->heads * kv->head_dim, kv_len, scale, out, out_dtype, ws,
                                  static_cast<hipStream_t>(stream));
    return launch_decode_attn_gqa(kv, q_f16, q_heads, kv_len, scale, out, out_dtype, ws,
                                  static_cast<hipStream_t>(stream));
}

fgq_status fgq_decode_attn_topk_q4kv(const fgq_kv_cache *kv, const void *q_f16, int32_t kv_len, int32_t top_k,
                                     float softmax_scale, void *out, int32_t out_dtype, int32_t *sel, void *stream) {
    g_err[0] = 0;
    fgq_status s = check_kv(kv);
    if (s != FGQ_OK) return s;
    if (out_dtype != FGQ_DTYPE_F32 && out_dtype != FGQ_DTYPE_F16)
        return fail(FGQ_ERR_DTYPE, "out_dtype %d", out_dtype);
    if (kv_len < 1) return fail(FGQ_ERR_SHAPE, "kv_len %d < 1", kv_len);
    if (kv_len > kv->capacity) return fail(FGQ_ERR_CAPACITY, "kv_len %d > capacity %d", kv_len, kv->capacity);
    if (top_k < 1) return fail(FGQ_ERR_INVALID_ARG, "top_k %d < 1", top_k);
    if (!std::isfinite(softmax_scale)) return fail(FGQ_ERR_INVALID_ARG, "softmax_scale is not finite");
    const int32_t kept = top_k < kv_len ? top_k : kv_len;
    if (kv_len > FGQ_TOPK_MAX_POSITIONS)
        return fail(FGQ_ERR_UNSUPPORTED, "kv_len %d > %d", kv_len, FGQ_TOPK_MAX_POSITIONS);
    if ((int64_t)kv->batch * kv->heads > INT32_MAX) return fail(FGQ_ERR_SHAPE, "batch * heads > 2^31 - 1");
    if (kv->batch == 0 || kv->heads == 0) return FGQ_OK;
    if (!q_f16 || !out) return fail(FGQ_ERR_INVALID_ARG, "NULL q or out");
    if (!aligned16(q_f16) || !aligned16(out) || (sel && !aligned16(sel)))
        return fail(FGQ_ERR_ALIGN, "q/out/sel must be 16-byte aligned");
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)kv->head_dim);
    return launch_decode_attn_topk(kv, q_f16, kv_len, kept, scale, out, out_dtype, sel,
                                   static_cast<hipStream_t>(stream));
}

fgq_status fgq_prefill_attn_f16(const void *q_f16, const void *k_f16, const void *v_f16, int32_t batch,
                                int32_t seq, int32_t heads, int32_t head_dim, float softmax_scale, void *out,
                                int32_t out_dtype, void *stream) {
    g_err[0] = 0;
    if (batch < 0 || seq < 0 || heads < 0 || head_dim <= 0) return fail(FGQ_ERR_INVALID_ARG, "negative size");
    if (head_dim != 64 && head_dim != 128) {
        if (head_dim % 64 != 0) return fail(FGQ_ERR_SHAPE, "head_dim %d is not a multiple of 64", head_dim);
        return fail(FGQ_ERR_UNSUPPORTED, "head_dim %d (64 or 128 supported)", head_dim);
    }
    if (out_dtype != FGQ_DTYPE_F32 && out_dtype != FGQ_DTYPE_F16)
        return fail(FGQ_ERR_DTYPE, "out_dtype %d", out_dtype);
    if (!std::isfinite(softmax_scale)) return fail(FGQ_ERR_INVALID_ARG, "softmax_scale is not finite");
    if (batch > 65535 || heads > 65535) return fail(FGQ_ERR_SHAPE, "batch and heads must be <= 65535");
    if ((double)batch * seq * heads * head_dim > (double)((int64_t)1 << 40))
        return fail(FGQ_ERR_SHAPE, "q/k/v larger than 2^40 elements");
    // the kernel numbers its workgroups (row blocks of at least 128 tokens x
    // heads x batch) in 32-bit ints
    if ((int64_t)batch * heads * ((seq + 127) / 128) > INT32_MAX)
        return fail(FGQ_ERR_SHAPE, "batch * heads * ceil(seq / 128) must be < 2^31");
    if (batch == 0 || seq == 0 || heads == 0) return FGQ_OK;
    if (!q_f16 || !k_f16 || !v_f16 || !out) return fail(FGQ_ERR_INVALID_ARG, "NULL array");
    if (!aligned16(q_f16) || !aligned16(k_f16) || !aligned16(v_f16) || !aligned16(out))
        return fail(FGQ_ERR_ALIGN, "q/k/v/out must be 16-byte aligned");
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
    return launch_prefill_attn(q_f16, k_f16, v_f16, batch, seq, heads, head_dim, scale, out, out_dtype,
                               static_cast<hipStream_t>(stream));
}

size_t fgq_pack_weight_meta_words(int64_t K, int64_t N) {
    if (K <= 0 || N <= 0 || K % 32 != 0 || N % 64 != 0 || K > kMaxK || N > kMaxNPacked) return 0;
    return (size_t)(K * (N / 64) + N / 64);
}

fgq_status fgq_pack_weight_g64(const uint8_t *codes, const uint32_t *meta, int64_t K, int64_t N,
                               uint32_t *packed_codes, uint32_t *packed_meta, void *stream) {
    g_err[0] = 0;
    if (K < 0 || N < 0) return fail(FGQ_ERR_INVALID_ARG, "negative size");
    if (K % 32 != 0 || N % 64 != 0) return fail(FGQ_ERR_SHAPE, "K %% 32 and N %% 64 must be 0");
    if (K > kMaxK || N > kMaxNPacked) return fail(FGQ_ERR_SHAPE, "K > 2^23 or N > 2^28");
    if (K == 0 || N == 0) return FGQ_OK;
    if (!codes || !meta || !packed_codes || !packed_meta) return fail(FGQ_ERR_INVALID_ARG, "NULL array");
    if (!aligned16(codes) || !aligned16(meta) || !aligned16(packed_codes) || !aligned16(packed_meta))
        return fail(FGQ_ERR_ALIGN, "arrays must be 16-byte aligned");
    return launch_pack_weight(codes, meta, K, N, packed_codes, packed_meta, static_cast<hipStream_t>(stream));
}

size_t fgq_dequant_gemm_ws_bytes(int64_t M, int64_t K, int64_t N) {
    if (M <= 0 || K < 0 || N <= 0 || K % 32 != 0 || N % 64 != 0 || M > kMaxM || K > kMaxK || N > kMaxNPacked)
        return 0;
    return gemm_ws_bytes(M, K, N);
}

// Shared validation of the two GEMM entry points; kmult is the K granule
// (64 for the canonical layout, 32 for the packed one), nmax the largest N.
static fgq_status check_gemm(const void *x_f16, int32_t g, int32_t m, int64_t K, int64_t N, const void *wc,
                             const void *wm, void *y, int32_t y_dtype, void *ws, size_t ws_bytes, int64_t kmult,
                             int64_t nmax, bool *noop) {
    *noop = false;
    if (g < 0 || m < 0 || K < 0 || N < 0) return fail(FGQ_ERR_INVALID_ARG, "negative size");
    if (K % kmult != 0 || N % 64 != 0)
        return fail(FGQ_ERR_SHAPE, "K %% %lld and N %% 64 must be 0 (K=%lld N=%lld)", (long long)kmult, (long long)K,
                    (long long)N);
    if (y_dtype != FGQ_DTYPE_F32 && y_dtype != FGQ_DTYPE_F16) return fail(FGQ_ERR_DTYPE, "y_dtype %d", y_dtype);
    const int64_t M = (int64_t)g * m;
    if (M > kMaxM) return fail(FGQ_ERR_SHAPE, "g*m too large");
    if (K > kMaxK || N > nmax)
        return fail(FGQ_ERR_SHAPE, "K > 2^23 or N > %lld", (long long)nmax);
    if (M == 0 || N == 0) {
        *noop = true;
        return FGQ_OK;
    }
    if (!y || (K > 0 && (!x_f16 || !wc || !wm))) return fail(FGQ_ERR_INVALID_ARG, "NULL array");
    if (!aligned16(y) || (K > 0 && (!aligned16(x_f16) || !aligned16(wc) || !aligned16(wm))))
        return fail(FGQ_ERR_ALIGN, "arrays must be 16-byte aligned");
    const size_t need = gemm_ws_bytes(M, K, N);
    if (need > 0) {
        if (!ws || ws_bytes < need)
            return fail(FGQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : (size_t)0, need);
        if (!aligned16(ws)) return fail(FGQ_ERR_ALIGN, "workspace must be 16-byte aligned");
    }
    return FGQ_OK;
}

fgq_status fgq_dequant_gemm(const void *x_f16, int32_t g, int32_t m, int64_t K, int64_t N, const uint8_t *w_codes,
                            const void *w_meta, void *y, int32_t y_dtype, void *ws, size_t ws_bytes, void *stream) {
    g_err[0] = 0;
    bool noop = false;
    const fgq_status s = check_gemm(x_f16, g, m, K, N, w_codes, w_meta, y, y_dtype, ws, ws_bytes, 64,
                                    kMaxNPacked / 2, &noop);
    if (s != FGQ_OK || noop) return s;
    return launch_dequant_gemm(x_f16, (int64_t)g * m, K, N, w_codes, static_cast<const uint32_t *>(w_meta), true, y,
                               y_dtype, ws, static_cast<hipStream_t>(stream));
}

fgq_status fgq_dequant_gemm_packed(const void *x_f16, int32_t g, int32_t m, int64_t K, int64_t N,
                                   const uint32_t *packed_codes, const uint32_t *packed_meta, void *y, int32_t y_dtype,
                                   void *ws, size_t ws_bytes, void *stream) {
    g_err[0] = 0;
    bool noop = false;
    const fgq_status s = check_gemm(x_f16, g, m, K, N, packed_codes, packed_meta, y, y_dtype, ws, ws_bytes, 32,
                                    kMaxNPacked, &noop);
    if (s != FGQ_OK || noop) return s;
    return launch_dequant_gemm(x_f16, (int64_t)g * m, K, N, packed_codes, packed_meta, false, y, y_dtype, ws,
                               static_cast<hipStream_t>(stream));
}

}  // extern "C"
