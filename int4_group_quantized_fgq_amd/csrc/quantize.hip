// Group-wise 4-bit quantiser (64 elements per group) for weights and KV
// rows, the KV-cache append, and the one-time weight re-layout for the GEMM.
//
// Encoding: FlexGen review on jaehun.me, section "Is 4-bit compression the
// same as integer-arithmetic acceleration?" (paper section 5) - asymmetric
// min/max groups of 64, weights along the output channel, KV along hidden,
// constant groups handled apart; FlexGen review on blog.gzher.com, section
// 3.4.  The formula itself is missing from the pages; the min-max reading
// q = RNE(((x - a) / (b - a)) * 15) is taken with each step an IEEE fp32
// operation in that order, so every code and meta word is reproducible bit
// for bit.
//
// Mapping: one group per 8 consecutive lanes, each lane owning 8 elements
// (one 16-byte load).  The group's min and max are combined with DPP lane
// moves inside the 8-lane segment; each lane then writes one 32-bit
// word of codes (8 nibbles) and the segment's first lane writes the meta
// word.  The division is the correctly rounded one (HIP default).
#include "common.h"
#include "fastdiv.h"

namespace fgq {
namespace {

struct GroupOut {
    uint32_t codes;   // 8 nibbles of this lane
    uint32_t meta;    // valid in every lane of the segment
};

template <int CTRL>
__device__ __forceinline__ float q_dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// x8: the lane's 8 fp16 values (as raw halves). All 8 lanes of the segment
// must call this together (lane exchanges).
__device__ __forceinline__ GroupOut quantize8(const uint4 raw) {
#pragma clang fp contract(off)
    float x[8];
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = h2f((uint16_t)(w[i] & 0xffffu));
        x[2 * i + 1] = h2f((uint16_t)(w[i] >> 16));
    }
    float a = x[0], b = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
        a = fminf(a, x[i]);
        b = fmaxf(b, x[i]);
    }
    // min and max over the 8 lanes of the segment with DPP lane moves (no LDS
    // round trip): swap neighbours, swap pairs, then mirror the half-row
    // (lane i <-> 7 - i) to combine the two quads.  Exact in any order.
    a = fminf(a, q_dpp<0xB1>(a));
    b = fmaxf(b, q_dpp<0xB1>(b));
    a = fminf(a, q_dpp<0x4E>(a));
    b = fmaxf(b, q_dpp<0x4E>(b));
    a = fminf(a, q_dpp<0x141>(a));
    b = fmaxf(b, q_dpp<0x141>(b));
    a = a + 0.0f;   // -0 -> +0
    b = b + 0.0f;
    GroupOut out;
    const uint32_t min_h = f2h_rne(a);   // exact: a is an fp16 value
    if (a == b) {
        out.codes = 0u;
        out.meta = min_h;
        return out;
    }
    const float d = __fsub_rn(b, a);
    // The code is rint(RN(RN(t / d) * 15)), t = x - a.  A cheaper estimate
    // t * RN(15 * rcp(d)) is within 2^-16 of that value (both are within a
    // few ulp of the exact 15t/d <= 15), so wherever the estimate is at least
    // 2^-15 away from a rounding boundary k + 1/2 it rounds to the same
    // integer; only elements closer than that (exact ties among them) take
    // the correctly rounded division.
    const float r15 = __fmul_rn(15.0f, __builtin_amdgcn_rcpf(d));
    uint32_t packed = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float t = __fsub_rn(x[i], a);
        const float va = __fmul_rn(t, r15);
        float r = rintf(va);
        // va - r is exact (|va - r| <= 1/2); near a boundary it is close to +-1/2
        if (__builtin_expect(fabsf(__fsub_rn(va, r)) > 0.5f - 3.0517578125e-05f, 0)) {
            const float u = __fdiv_rn(t, d);
            const float v = __fmul_rn(u, 15.0f);
            r = rintf(v);                   // v_rndne_f32: ties to even
        }
        // 0 <= t <= d, so 0 <= r <= 15 on both paths: no clamp is needed
        packed |= ((uint32_t)r) << (4 * i);
    }
    const float step = __fdiv_rn(d, 15.0f);
    out.codes = packed;
    out.meta = min_h | ((uint32_t)f2h_rne(step) << 16);
    return out;
}

// One launch covers fewer than 2^31 groups, so positions are 32-bit and the
// row of a group comes from a division by the launch-invariant group count
// per row (multiply-high + shifts) instead of a 64-bit division.
__global__ __launch_bounds__(256) void quantize_g64_kernel(const uint16_t *__restrict__ x, uint32_t total,
                                                           FastDiv div_ngr, int64_t cols, int64_t ld,
                                                           uint32_t *__restrict__ codes,
                                                           uint32_t *__restrict__ meta) {
    const uint32_t gid = blockIdx.x * 32u + (threadIdx.x >> 3);
    const int sub = threadIdx.x & 7;
    const bool valid = gid < total;
    const uint32_t g2 = valid ? gid : 0u;
    const uint32_t r = fastdiv(g2, div_ngr);
    const uint32_t gi = g2 - r * div_ngr.d;
    uint4 raw = make_uint4(0u, 0u, 0u, 0u);
    if (valid) raw = *reinterpret_cast<const uint4 *>(x + (int64_t)r * ld + gi * 64 + sub * 8);
    const GroupOut o = quantize8(raw);
    if (!valid) return;
    codes[((int64_t)r * (cols >> 1) + gi * 32 + sub * 4) >> 2] = o.codes;
    if (sub == 0) meta[gid] = o.meta;
}

// One group = 64 hidden elements of one token's K or V row of one head.
// gid enumerates (which in {K,V}, b, head, i, group-in-head), the group
// fastest and then the token: the groups of consecutive tokens of one head
// are consecutive in the head-major cache, so a wave's code and meta writes
// are contiguous runs (its reads are 128-byte slices of token rows).  The
// position is decoded with 32-bit divisions by the launch-invariant n_new and
// head count (multiply-high + shifts); a launch covers fewer than 2^31 groups.
// A workgroup takes 32 * GPT groups: each 8-lane segment loads its GPT groups
// first, so GPT 16-byte loads per lane are in flight at once.
struct AppendPos {
    const uint16_t *src;
    int64_t slot;
    uint32_t gi;
    int which;
};

__device__ __forceinline__ AppendPos append_pos(uint32_t g2, const fgq_kv_cache &kv, int lg, const FastDiv &div_n,
                                                const FastDiv &div_h, const uint16_t *k_new,
                                                const uint16_t *v_new, int64_t ld, int32_t pos, int sub) {
    const uint32_t gi = g2 & ((1u << lg) - 1u);
    const uint32_t r1 = g2 >> lg;                  // (which, b, head, i)
    const uint32_t r2 = fastdiv(r1, div_n);        // (which, b, head)
    const uint32_t i = r1 - r2 * div_n.d;
    const uint32_t r3 = fastdiv(r2, div_h);        // (which, b)
    const uint32_t hd = r2 - r3 * div_h.d;
    const int which = r3 >= (uint32_t)kv.batch ? 1 : 0;
    const uint32_t b = r3 - (which ? (uint32_t)kv.batch : 0u);
    AppendPos p;
    p.src = (which ? v_new : k_new) + ((int64_t)b * div_n.d + i) * ld + (int64_t)hd * kv.head_dim + gi * 64 +
            sub * 8;
    p.slot = ((int64_t)b * kv.heads + hd) * kv.capacity + pos + i;
    p.gi = gi;
    p.which = which;
    return p;
}

template <int GPT>
__global__ __launch_bounds__(256) void kv_append_kernel(const uint16_t *__restrict__ k_new,
                                                        const uint16_t *__restrict__ v_new,
                                                        fgq_kv_cache kv, int64_t ld, int32_t pos, uint32_t total,
                                                        FastDiv div_n, FastDiv div_h) {
    const int lg = kv.head_dim == 128 ? 1 : 0;              // log2(groups per head)
    const int sub = threadIdx.x & 7;
    AppendPos p[GPT];
    uint4 raw[GPT];
#pragma unroll
    for (int k = 0; k < GPT; ++k) {
        const uint32_t gid = blockIdx.x * (32u * GPT) + 32u * k + (threadIdx.x >> 3);
        p[k] = append_pos(gid < total ? gid : 0u, kv, lg, div_n, div_h, k_new, v_new, ld, pos, sub);
        raw[k] = make_uint4(0u, 0u, 0u, 0u);
        if (gid < total) raw[k] = *reinterpret_cast<const uint4 *>(p[k].src);
    }
#pragma unroll
    for (int k = 0; k < GPT; ++k) {
        const uint32_t gid = blockIdx.x * (32u * GPT) + 32u * k + (threadIdx.x >> 3);
        const GroupOut o = quantize8(raw[k]);   // every lane of the segment takes part
        if (gid >= total) continue;
        uint8_t *cbase = p[k].which ? kv.v_codes : kv.k_codes;
        uint32_t *mbase = p[k].which ? kv.v_meta : kv.k_meta;
        // nontemporal: nothing in this launch reads the rows again, and the
        // attention launch that follows ran ~3% faster than after plain stores
        __builtin_nontemporal_store(o.codes, reinterpret_cast<uint32_t *>(cbase + p[k].slot * (kv.head_dim >> 1) +
                                                                          p[k].gi * 32 + sub * 4));
        if (sub == 0) __builtin_nontemporal_store(o.meta, mbase + p[k].slot * (1 << lg) + p[k].gi);
    }
}

// Weight re-layout: one thread per packed code word (kc, g, lane, j).
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t *__restrict__ codes, int64_t K,
                                                         int64_t N, uint32_t *__restrict__ packed) {
    const int64_t words = K * N / 8;
    const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (w >= words) return;
    const int j = (int)(w & 3);
    const int lane = (int)((w >> 2) & 63);
    const int64_t tile = w >> 8;                 // kc * (N/64) + g
    const int64_t ng = N >> 6;
    const int64_t g = tile % ng, kc = tile / ng;
    const int64_t n = 64 * g + 16 * j + (lane & 15);
    const int64_t k0 = 32 * kc + 8 * (lane >> 4);
    const int slot_of[8] = {0, 4, 1, 5, 2, 6, 3, 7};
    uint32_t out = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint8_t byte = codes[(k0 + i) * (N >> 1) + (n >> 1)];
        const uint32_t q = (n & 1) ? (byte >> 4) : (byte & 15u);
        out |= q << (4 * slot_of[i]);
    }
    packed[w] = out;
}

// Column-group exponent e_g: the smallest e >= 0 with max_k step[k][g] *
// 2^(24 - e) <= 65504, so that every step scaled for the GEMM's subnormal
// code placement stays a finite fp16.  One workgroup per column group g.
__global__ __launch_bounds__(256) void pack_exponent_kernel(const uint32_t *__restrict__ meta, int64_t K,
                                                            int64_t N, int32_t *__restrict__ exps) {
    __shared__ uint32_t red[256];
    const int64_t ng = N >> 6;
    const int64_t g = blockIdx.x;
    uint32_t mx = 0u;   // steps are >= +0, so their fp16 bits order like their values
    for (int64_t k = threadIdx.x; k < K; k += 256) {
        const uint32_t st = meta[k * ng + g] >> 16;
        mx = st > mx ? st : mx;
    }
    red[threadIdx.x] = mx;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if ((int)threadIdx.x < off) red[threadIdx.x] = max(red[threadIdx.x], red[threadIdx.x + off]);
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const float ms = h2f((uint16_t)red[0]);
        int e = 0;
        while (e < 24 && ms * __builtin_amdgcn_ldexpf(1.0f, 24 - e) > 65504.0f) ++e;
        exps[g] = e;
    }
}

// fp16 value (bits) times 2^s, rounded to fp16 (exact unless the result is
// an fp16 subnormal).
__device__ __forceinline__ uint32_t scale_h(uint32_t hbits, int s) {
    return f2h_rne(h2f((uint16_t)hbits) * __builtin_amdgcn_ldexpf(1.0f, s));
}

// One thread per packed meta word (kc, g, kq, t).  The GEMM places codes
// 0, 1 (and 4, 5) of a word in fp16 subnormal mantissas as q * 2^-24, and
// codes 2, 3 (and 6, 7) as q * 2^-20, so their steps are stored times
// 2^(24 - e_g) (t = 0, 2) and 2^(20 - e_g) (t = 1, 3), and the minima
// times 2^-e_g; the GEMM multiplies its result by 2^e_g.
__global__ __launch_bounds__(256) void pack_meta_kernel(const uint32_t *__restrict__ meta, int64_t K,
                                                        int64_t N, const int32_t *__restrict__ exps,
                                                        uint32_t *__restrict__ packed) {
    const int64_t words = K * N / 64;
    const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (w >= words) return;
    const int t = (int)(w & 7);
    const int kq = (int)((w >> 3) & 3);
    const int64_t tile = w >> 5;
    const int64_t ng = N >> 6;
    const int64_t g = tile % ng, kc = tile / ng;
    const int64_t k = 32 * kc + 8 * kq + 2 * (t & 3);
    const uint32_t m0 = meta[k * ng + g], m1 = meta[(k + 1) * ng + g];
    const int e = exps[g];
    const int s = t >= 4 ? -e : ((t & 1) ? 20 - e : 24 - e);
    const uint32_t h0 = t < 4 ? (m0 >> 16) : (m0 & 0xffffu);
    const uint32_t h1 = t < 4 ? (m1 >> 16) : (m1 & 0xffffu);
    packed[w] = scale_h(h0, s) | (scale_h(h1, s) << 16);
}

}  // namespace

// Launches of fewer than 2^31 groups each: the rows in chunks for the
// quantiser, the sequences in chunks for the append.
constexpr int64_t kMaxGroupsPerLaunch = (int64_t)1 << 30;
// Bulk appends (a prompt) give each 8-lane segment FGQ_APPEND_GPT groups.
#ifndef FGQ_APPEND_GPT
#define FGQ_APPEND_GPT 2
#endif
constexpr int64_t kAppendManyGroups = (int64_t)1 << 18;

fgq_status launch_quantize(const void *x, int64_t rows, int64_t cols, int64_t ld, uint8_t *codes,
                           uint32_t *meta, hipStream_t stream) {
    const int64_t ngr = cols / 64;
    if (rows == 0 || ngr == 0) return FGQ_OK;
    const int64_t rows_per = kMaxGroupsPerLaunch / ngr > 0 ? kMaxGroupsPerLaunch / ngr : 1;
    const FastDiv div_ngr = make_fastdiv((uint32_t)ngr);
    for (int64_t r0 = 0; r0 < rows; r0 += rows_per) {
        const int64_t nr = rows - r0 < rows_per ? rows - r0 : rows_per;
        const int64_t groups = nr * ngr;
        quantize_g64_kernel<<<dim3((unsigned)((groups + 31) / 32)), dim3(256), 0, stream>>>(
            static_cast<const uint16_t *>(x) + r0 * ld, (uint32_t)groups, div_ngr, cols, ld,
            reinterpret_cast<uint32_t *>(codes + r0 * (cols / 2)), meta + r0 * ngr);
        fgq_status s = check_launch("quantize_g64_kernel");
        if (s != FGQ_OK) return s;
    }
    return FGQ_OK;
}

// k_new / v_new rows (one per sequence and new token) are ld elements apart.
fgq_status launch_kv_append(const fgq_kv_cache *kv, const void *k_new, const void *v_new, int64_t ld, int32_t pos,
                            int32_t n_new, hipStream_t stream) {
    const int64_t gph = kv->head_dim / 64;
    const int64_t per_seq = 2LL * n_new * kv->heads * gph;   // groups of one sequence (K and V)
    if (per_seq == 0 || kv->batch == 0) return FGQ_OK;
    const int64_t seq_per = kMaxGroupsPerLaunch / per_seq > 0 ? kMaxGroupsPerLaunch / per_seq : 1;
    const FastDiv div_n = make_fastdiv((uint32_t)n_new), div_h = make_fastdiv((uint32_t)kv->heads);
    const int64_t rows = (int64_t)kv->heads * kv->capacity;   // cache rows of one sequence
    for (int64_t b0 = 0; b0 < kv->batch; b0 += seq_per) {
        const int64_t nb = kv->batch - b0 < seq_per ? kv->batch - b0 : seq_per;
        fgq_kv_cache sub = *kv;
        sub.batch = (int32_t)nb;
        sub.k_codes = kv->k_codes + b0 * rows * (kv->head_dim / 2);
        sub.v_codes = kv->v_codes + b0 * rows * (kv->head_dim / 2);
        sub.k_meta = kv->k_meta + b0 * rows * gph;
        sub.v_meta = kv->v_meta + b0 * rows * gph;
        const int64_t groups = nb * per_seq;
        const uint16_t *kn = static_cast<const uint16_t *>(k_new) + b0 * n_new * ld;
        const uint16_t *vn = static_cast<const uint16_t *>(v_new) + b0 * n_new * ld;
        if (groups >= kAppendManyGroups) {
            constexpr int G2 = FGQ_APPEND_GPT;
            kv_append_kernel<G2><<<dim3((unsigned)((groups + 32 * G2 - 1) / (32 * G2))), dim3(256), 0, stream>>>(
                kn, vn, sub, ld, pos, (uint32_t)groups, div_n, div_h);
        } else {
            kv_append_kernel<1><<<dim3((unsigned)((groups + 31) / 32)), dim3(256), 0, stream>>>(
                kn, vn, sub, ld, pos, (uint32_t)groups, div_n, div_h);
        }
        fgq_status s = check_launch("kv_append_kernel");
        if (s != FGQ_OK) return s;
    }
    return FGQ_OK;
}

fgq_status launch_pack_weight(const uint8_t *codes, const uint32_t *meta, int64_t K, int64_t N,
                              uint32_t *packed_codes, uint32_t *packed_meta, hipStream_t stream) {
    const int64_t cw = K * N / 8, mw = K * N / 64;
    if (cw == 0) return FGQ_OK;
    pack_codes_kernel<<<dim3((unsigned)((cw + 255) / 256)), dim3(256), 0, stream>>>(codes, K, N, packed_codes);
    fgq_status s = check_launch("pack_codes_kernel");
    if (s != FGQ_OK) return s;
    int32_t *exps = reinterpret_cast<int32_t *>(packed_meta + mw);   // [N/64], after the meta words
    pack_exponent_kernel<<<dim3((unsigned)(N / 64)), dim3(256), 0, stream>>>(meta, K, N, exps);
    s = check_launch("pack_exponent_kernel");
    if (s != FGQ_OK) return s;
    pack_meta_kernel<<<dim3((unsigned)((mw + 255) / 256)), dim3(256), 0, stream>>>(meta, K, N, exps, packed_meta);
    return check_launch("pack_meta_kernel");
}

}  // namespace fgq
