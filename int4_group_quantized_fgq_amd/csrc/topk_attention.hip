// Top-K sparse decode attention over the 4-bit compressed KV cache.
//
// What is computed: the paper's optional approximation that reads only the
// top 10% of the value cache (FlexGen review on blog.gzher.com, section 3.4;
// paper-graph-ui FlexGen summary, section 3.3 "Roadmap for the Deep Dive",
// one of the two section-5 approximations that cut I/O volume).  Per
// (sequence b, head h), with K^, V^ the reconstructions of the stored codes:
//   s_j = scale * sum_d q_d K^_{j,d}                       j in [0, L)
//   T   = the kk = min(top_k, L) positions with the largest s_j, compared as
//         fp32 values (-0 as +0), equal scores going to the lower position
//   o_d = sum_{j in T} exp(s_j - m) V^_{j,d} / sum_{j in T} exp(s_j - m)
// where m = max_j s_j (always in T).  Only the kept V rows are read.
//
// Design: one 256-thread workgroup per (b, h), everything in LDS.
//  * Scores: a token's K row is read by D/32 lanes with one 16-byte
//    nontemporal load each (as in the dense kernel), four token groups of
//    loads in flight per wave; the reconstruction is folded out of the
//    element loop (sum_g min_g sum q + step_g sum q c, dot2 on codes placed
//    in fp16 subnormal mantissas, exact products).  Scores go to LDS.
//  * Selection: the cut at the kk-th largest score is found exactly by a
//    radix select (8-bit digits, LDS histogram, most significant first) over
//    order-preserving uint32 keys; it stops as soon as every candidate left
//    in the chosen bucket is kept (usually after two digits), else after four
//    with the exact kk-th largest key.  An ordered scan (wave ballots) then
//    keeps every key above the bucket and the first (lowest-position) ones in
//    it, compacting the kept positions in ascending order.
//  * P.V: the kept rows are gathered (16-byte loads per lane); fp32
//    accumulation of p_j*step_j*c plus p_j*min_j per group; slot sums by
//    lane shuffles, wave sums through LDS.
// Bytes: 0.5625*D per position of K, per kept position of V.
#include <algorithm>

#include "common.h"

namespace fgq {
namespace {

constexpr float kTkLog2e = 1.4426950408889634f;
constexpr int kTkThreads = 256;
constexpr int kTkUnroll = 4;   // token groups of K loads in flight per wave

__device__ __forceinline__ float tk_dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(as_f16x2(a), as_f16x2(b), c, false);
}

template <int CTRL>
__device__ __forceinline__ float tk_dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the PARTS consecutive lanes of one token (quad_perm xor 1, xor 2).
template <int PARTS>
__device__ __forceinline__ float tk_sum_parts(float v) {
    v += tk_dpp<0xB1>(v);
    if (PARTS == 4) v += tk_dpp<0x4E>(v);
    return v;
}

__device__ __forceinline__ uint4 tk_stream_load16(const uint8_t *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Order-preserving key of an fp32 score: a larger score gives a larger key;
// -0 is folded into +0 first, so equal scores give equal keys.
__device__ __forceinline__ uint32_t order_key(float s) {
    const uint32_t u = __float_as_uint(s + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The lane's 32 query values (elements part*32 .. part*32+31 of head bh) as
// dot2 pairs matching the code layout, and their sum.  Code word i holds
// elements 8i..8i+7, element 8i+2t in byte t's low nibble; the pairs are
// (q_{8i+0}, q_{8i+4}), (q_{8i+1}, q_{8i+5}), (q_{8i+2}, q_{8i+6}), (q_{8i+3}, q_{8i+7}).
template <int D>
__device__ __forceinline__ void tk_query(const uint16_t *__restrict__ q, int bh, int part, uint32_t (&QP)[4][4],
                                         float &qsum) {
    const uint4 *qp = reinterpret_cast<const uint4 *>(q + (size_t)bh * D + part * 32);
    qsum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 t = qp[i];
        QP[i][0] = __builtin_amdgcn_perm(t.z, t.x, 0x05040100u);
        QP[i][1] = __builtin_amdgcn_perm(t.z, t.x, 0x07060302u);
        QP[i][2] = __builtin_amdgcn_perm(t.w, t.y, 0x05040100u);
        QP[i][3] = __builtin_amdgcn_perm(t.w, t.y, 0x07060302u);
        const uint32_t w4[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int h2 = 0; h2 < 4; ++h2) {
            const f16x2 v = as_f16x2(w4[h2]);
            qsum += (float)v.x + (float)v.y;
        }
    }
}

// Score of one token from its 16-byte code slice and group meta: every lane
// of the token's PARTS returns the same fp32 value (the same operations in
// both kernels, so equal rows give bit-equal scores everywhere).
template <int PARTS>
__device__ __forceinline__ float tk_score(const uint4 kr, uint32_t kmeta, const uint32_t (&QP)[4][4], float qsum,
                                          float scale) {
    const uint32_t w[4] = {kr.x, kr.y, kr.z, kr.w};
    float lo = 0.f, hi = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w8 = w[i] >> 8;
        lo = tk_dot2(w[i] & 0x000F000Fu, QP[i][0], lo);
        hi = tk_dot2(w[i] & 0x00F000F0u, QP[i][1], hi);
        lo = tk_dot2(w8 & 0x000F000Fu, QP[i][2], lo);
        hi = tk_dot2(w8 & 0x00F000F0u, QP[i][3], hi);
    }
    const float csum = lo * 16777216.0f + hi * 1048576.0f;   // sum of q_d c_d over the lane's 32
    const float step = h2f((uint16_t)(kmeta >> 16));
    const float mn = h2f((uint16_t)(kmeta & 0xffffu));
    return tk_sum_parts<PARTS>(step * csum + mn * qsum) * scale;
}

// Sum of a P.V contribution: o[8i+e] += wgt * c, element 8i+e of the lane's
// 32 in nibble e of word i (byte e/2, the low nibble for even e).
__device__ __forceinline__ void tk_pv(float (&o)[32], const uint4 vr, float wgt) {
    const uint32_t w[4] = {vr.x, vr.y, vr.z, vr.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[8 * i + e] += wgt * (float)((w[i] >> (4 * e)) & 15u);
}

template <int D>
__global__ __launch_bounds__(kTkThreads) void attn_topk_kernel(
    const uint8_t *__restrict__ kc, const uint32_t *__restrict__ km, const uint8_t *__restrict__ vc,
    const uint32_t *__restrict__ vm, const uint16_t *__restrict__ q, int H, int cap, int L, int kk, float scale,
    void *__restrict__ out, int out_f16, int32_t *__restrict__ sel) {
    constexpr int PARTS = D / 32;    // lanes per token row
    constexpr int TPI = 64 / PARTS;  // tokens per wave per load
    constexpr int G = D / 64;        // groups per token row
    constexpr int NW = kTkThreads / 64;
    extern __shared__ float tk_smem[];           // scores [L], then kept positions [kk]
    __shared__ uint32_t hist[256];
    __shared__ uint32_t wtot[2][NW];
    __shared__ float wmax[NW];
    __shared__ uint32_t sh_digit, sh_rem, sh_cnt;
    __shared__ float red_o[NW][D];
    __shared__ float red_m[NW][PARTS];
    __shared__ float red_l[NW];

    float *sc = tk_smem;
    int32_t *kept = reinterpret_cast<int32_t *>(tk_smem + L);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int bh = blockIdx.x;
    const int slot = lane / PARTS, part = lane % PARTS, grp = part >> 1;

    uint32_t QP[4][4];
    float qsum;
    tk_query<D>(q, bh, part, QP, qsum);

    const size_t rowbase = (size_t)bh * cap;
    const uint8_t *kbase = kc + rowbase * (D / 2) + part * 16;
    const uint32_t *kmb = km + rowbase * G + grp;

    // ---- scores of every position into LDS
    float lmax = -INFINITY;
    constexpr int BLOCK_TOK = kTkUnroll * NW * TPI;
    for (int base = 0; base < L; base += BLOCK_TOK) {
        uint4 Kr[kTkUnroll];
        uint32_t Km[kTkUnroll];
#pragma unroll
        for (int u = 0; u < kTkUnroll; ++u) {
            const int j = base + (u * NW + wv) * TPI + slot;
            const size_t jc = (size_t)(j < L ? j : L - 1);   // past the end: re-read the last row
            Kr[u] = tk_stream_load16(kbase + jc * (D / 2));
            Km[u] = __builtin_nontemporal_load(kmb + jc * G);
        }
#pragma unroll
        for (int u = 0; u < kTkUnroll; ++u) {
            const int j = base + (u * NW + wv) * TPI + slot;
            const float s = tk_score<PARTS>(Kr[u], Km[u], QP, qsum, scale);
            if (j < L) {
                if (part == 0) sc[j] = s;
                lmax = fmaxf(lmax, s);
            }
        }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, off, 64));
    if (lane == 0) wmax[wv] = lmax;
    __syncthreads();
    float m = wmax[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) m = fmaxf(m, wmax[w]);

    // ---- radix select of the kk-th largest key (8-bit digits, most significant first)
    uint32_t prefix = 0, pmask = 0, rem = (uint32_t)kk;
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        hist[tid] = 0;
        __syncthreads();
        // four scores per iteration: their LDS reads are in flight together
        for (int j0 = tid; j0 < L; j0 += 4 * kTkThreads) {
            uint32_t key[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = j0 + u * kTkThreads;
                key[u] = order_key(sc[j < L ? j : 0]);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (j0 + u * kTkThreads < L && (key[u] & pmask) == prefix)
                    atomicAdd(&hist[(key[u] >> shift) & 255u], 1u);
        }
        __syncthreads();
        // S(t) = number of candidate keys whose digit is >= t (suffix sum over bins)
        const uint32_t hv = hist[tid];
        uint32_t x = hv;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_down(x, off, 64);
            if (lane + off < 64) x += y;
        }
        if (lane == 0) wtot[0][wv] = x;
        __syncthreads();
        uint32_t S = x;
        for (int w = wv + 1; w < NW; ++w) S += wtot[0][w];
        const uint32_t S_above = S - hv;   // digit > t
        if (S >= rem && S_above < rem) {   // exactly one bin satisfies this
            sh_digit = (uint32_t)tid;
            sh_rem = rem - S_above;
            sh_cnt = hv;
        }
        __syncthreads();
        prefix |= sh_digit << shift;
        pmask |= 255u << shift;
        rem = sh_rem;
        if (rem == sh_cnt) break;          // every candidate left is kept: the cut is found
    }
    // keys whose leading bits (pmask) exceed prefix are kept, and the first
    // `rem` by position of those equal to it (all of them after an early exit;
    // after four passes they are the keys equal to the kk-th largest)

    // ---- ordered compaction
    const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    uint32_t carry_eq = 0, carry_keep = 0;
    for (int base = 0; base < L; base += kTkThreads) {
        const int j = base + tid;
        const uint32_t key = j < L ? (order_key(sc[j]) & pmask) : 0u;
        const bool eq = j < L && key == prefix;
        const bool gt = j < L && key > prefix;
        const uint64_t be = __ballot(eq);
        if (lane == 0) wtot[0][wv] = (uint32_t)__popcll(be);
        __syncthreads();
        uint32_t off_eq = carry_eq, tile_eq = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const uint32_t c = wtot[0][w];
            off_eq += w < wv ? c : 0u;
            tile_eq += c;
        }
        const bool keep = gt || (eq && off_eq + (uint32_t)__popcll(be & lt_mask) < rem);
        carry_eq += tile_eq;
        const uint64_t bk = __ballot(keep);
        if (lane == 0) wtot[1][wv] = (uint32_t)__popcll(bk);
        __syncthreads();
        uint32_t off_k = carry_keep, tile_k = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const uint32_t c = wtot[1][w];
            off_k += w < wv ? c : 0u;
            tile_k += c;
        }
        const uint32_t pos = off_k + (uint32_t)__popcll(bk & lt_mask);   // < kk by construction
        if (keep && pos < (uint32_t)kk) {
            kept[pos] = j;
            if (sel) sel[(size_t)bh * kk + pos] = j;
        }
        carry_keep += tile_k;
    }
    __syncthreads();

    // ---- P.V over the kept rows
    const uint8_t *vbase = vc + rowbase * (D / 2) + part * 16;
    const uint32_t *vmb = vm + rowbase * G + grp;
    float o[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) o[e] = 0.f;
    float l_acc = 0.f, m_acc = 0.f;
    const float ml2 = m * kTkLog2e;
    constexpr int PV_U = 2;
    for (int i0 = 0; i0 < kk; i0 += PV_U * NW * TPI) {
        uint4 Vr[PV_U];
        uint32_t Vm[PV_U];
        int jj[PV_U];
#pragma unroll
        for (int u = 0; u < PV_U; ++u) {
            const int i = i0 + (u * NW + wv) * TPI + slot;
            jj[u] = i < kk ? min(max(kept[i], 0), L - 1) : -1;
            if (jj[u] >= 0) {
                Vr[u] = tk_stream_load16(vbase + (size_t)jj[u] * (D / 2));
                Vm[u] = __builtin_nontemporal_load(vmb + (size_t)jj[u] * G);
            }
        }
#pragma unroll
        for (int u = 0; u < PV_U; ++u) {
            if (jj[u] < 0) continue;
            const float p = __builtin_amdgcn_exp2f(sc[jj[u]] * kTkLog2e - ml2);
            const float wgt = p * h2f((uint16_t)(Vm[u] >> 16));
            l_acc += p;
            m_acc += p * h2f((uint16_t)(Vm[u] & 0xffffu));
            tk_pv(o, Vr[u], wgt);
        }
    }
    // sum over the token slots of the wave (lanes with the same part)
#pragma unroll
    for (int off = PARTS; off < 64; off <<= 1) {
#pragma unroll
        for (int e = 0; e < 32; ++e) o[e] += __shfl_xor(o[e], off, 64);
        l_acc += __shfl_xor(l_acc, off, 64);
        m_acc += __shfl_xor(m_acc, off, 64);
    }
    if (slot == 0) {
#pragma unroll
        for (int e = 0; e < 32; ++e) red_o[wv][part * 32 + e] = o[e];
        red_m[wv][part] = m_acc;
        if (part == 0) red_l[wv] = l_acc;
    }
    __syncthreads();
    if (tid < D) {
        float num = 0.f, mins = 0.f, den = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            num += red_o[w][tid];
            mins += red_m[w][tid / 32];
            den += red_l[w];
        }
        const float v = (num + mins) / den;
        if (out_f16)
            static_cast<_Float16 *>(out)[(size_t)bh * D + tid] = (_Float16)v;
        else
            static_cast<float *>(out)[(size_t)bh * D + tid] = v;
    }
}

// Make the wave's earlier LDS writes visible to its later LDS reads (the
// wave's LDS operations complete in order; this keeps the compiler from
// moving them across).
__device__ __forceinline__ void tk_wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The same computation with one wavefront per (b, h) and no workgroup
// barrier: for short contexts, where a whole workgroup per (b, h) has too
// little to stream.  The K rows stream through two register buffers (the
// next chunk's loads in flight while the current one is scored); selection
// and compaction use wave-wide ballots and shuffles only, on the keys held
// in registers (key r of lane l is position 64r + l; KR * 64 >= L).  Each wave owns
// wave_words 32-bit words of LDS: a 256-bin histogram, scores [L], kept
// positions [kk].
template <int D, int KR>
__global__ __launch_bounds__(256) void attn_topk_wave_kernel(
    const uint8_t *__restrict__ kc, const uint32_t *__restrict__ km, const uint8_t *__restrict__ vc,
    const uint32_t *__restrict__ vm, const uint16_t *__restrict__ q, int H, int cap, int L, int kk, float scale,
    void *__restrict__ out, int out_f16, int32_t *__restrict__ sel, int total_items, int wave_words) {
    constexpr int PARTS = D / 32;
    constexpr int TPI = 64 / PARTS;
    constexpr int G = D / 64;
    constexpr int CH = 4;                // token iterations per chunk
    constexpr int STEP = CH * TPI;
    extern __shared__ float tk_smem[];

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int bh = blockIdx.x * (blockDim.x >> 6) + wv;
    if (bh >= total_items) return;       // wave-uniform; no workgroup barrier below
    // the wave's words: histogram [256] (16-byte aligned: wave_words % 4 == 0),
    // scores [L], kept positions [kk]
    uint32_t *hist = reinterpret_cast<uint32_t *>(tk_smem + (size_t)wv * wave_words);
    float *sc = reinterpret_cast<float *>(hist + 256);
    int32_t *kept = reinterpret_cast<int32_t *>(sc + L);
    const int slot = lane / PARTS, part = lane % PARTS, grp = part >> 1;

    uint32_t QP[4][4];
    float qsum;
    tk_query<D>(q, bh, part, QP, qsum);

    const size_t rowbase = (size_t)bh * cap;
    const uint8_t *kbase = kc + rowbase * (D / 2) + part * 16;
    const uint32_t *kmb = km + rowbase * G + grp;

    // ---- scores, double-buffered
    struct Chunk {
        uint4 K[CH];
        uint32_t KM[CH];
    };
    auto load = [&](int c0, Chunk &d) {
#pragma unroll
        for (int it = 0; it < CH; ++it) {
            const int j = c0 + it * TPI + slot;
            const size_t jc = (size_t)(j < L ? j : L - 1);
            d.K[it] = tk_stream_load16(kbase + jc * (D / 2));
            d.KM[it] = __builtin_nontemporal_load(kmb + jc * G);
        }
    };
    float lmax = -INFINITY;
    auto score = [&](int c0, const Chunk &d) {
#pragma unroll
        for (int it = 0; it < CH; ++it) {
            const int j = c0 + it * TPI + slot;
            const float sv = tk_score<PARTS>(d.K[it], d.KM[it], QP, qsum, scale);
            if (j < L) {
                if (part == 0) sc[j] = sv;
                lmax = fmaxf(lmax, sv);
            }
        }
    };
    Chunk bufA, bufB;
    load(0, bufA);
    for (int c0 = 0; c0 < L; c0 += 2 * STEP) {
        if (c0 + STEP < L) load(c0 + STEP, bufB);
        score(c0, bufA);
        if (c0 + STEP >= L) break;
        if (c0 + 2 * STEP < L) load(c0 + 2 * STEP, bufA);
        score(c0 + STEP, bufB);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, off, 64));
    const float m = lmax;
    tk_wave_sync();

    uint32_t keys[KR];
#pragma unroll
    for (int r = 0; r < KR; ++r) {
        const int j = 64 * r + lane;
        keys[r] = j < L ? order_key(sc[j]) : 0u;
    }

    // ---- radix select of the kk-th largest key; lane l owns bins 4l .. 4l+3
    uint32_t prefix = 0, pmask = 0, rem = (uint32_t)kk;
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        *reinterpret_cast<uint4 *>(hist + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
        tk_wave_sync();
#pragma unroll
        for (int r = 0; r < KR; ++r)
            if (64 * r + lane < L && (keys[r] & pmask) == prefix) atomicAdd(&hist[(keys[r] >> shift) & 255u], 1u);
        tk_wave_sync();
        const uint4 hb = *reinterpret_cast<const uint4 *>(hist + 4 * lane);
        const uint32_t h[4] = {hb.x, hb.y, hb.z, hb.w};
        uint32_t loc[4];                 // suffix sums inside the lane's four bins
        loc[3] = h[3];
        loc[2] = h[2] + loc[3];
        loc[1] = h[1] + loc[2];
        loc[0] = h[0] + loc[1];
        uint32_t x = loc[0];             // suffix sum over lanes >= this one
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_down(x, off, 64);
            if (lane + off < 64) x += y;
        }
        const uint32_t above = x - loc[0];
        int found = -1;
        uint32_t nrem = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t S = above + loc[r];   // candidates with digit >= 4*lane + r
            if (S >= rem && S - h[r] < rem) {    // exactly one bin of the wave
                found = r;
                nrem = rem - (S - h[r]);
            }
        }
        const uint64_t who = __ballot(found >= 0);
        const int src = who ? (int)__builtin_ctzll(who) : 0;
        const uint32_t dsel = (uint32_t)__shfl(4 * lane + (found < 0 ? 0 : found), src, 64);
        const uint32_t cnt = (uint32_t)__shfl((int)(found < 0 ? 0u : h[found]), src, 64);
        rem = (uint32_t)__shfl((int)nrem, src, 64);
        prefix |= dsel << shift;
        pmask |= 255u << shift;
        tk_wave_sync();                  // histogram reads done before the next clear
        if (rem == cnt) break;           // every candidate left is kept: the cut is found
    }

    // ---- ordered compaction: keys whose leading bits (pmask) exceed prefix,
    // then the first `rem` by position of those equal to it (all of them after
    // an early exit; after four passes, the keys equal to the kk-th largest)
    const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    uint32_t carry_eq = 0, carry_keep = 0;
#pragma unroll
    for (int r = 0; r < KR; ++r) {
        const int j = 64 * r + lane;
        const uint32_t key = keys[r] & pmask;
        const bool eq = j < L && key == prefix;
        const bool gt = j < L && key > prefix;
        const uint64_t be = __ballot(eq);
        const bool keep = gt || (eq && carry_eq + (uint32_t)__popcll(be & lt_mask) < rem);
        carry_eq += (uint32_t)__popcll(be);
        const uint64_t bk = __ballot(keep);
        const uint32_t pos = carry_keep + (uint32_t)__popcll(bk & lt_mask);
        if (keep && pos < (uint32_t)kk) {
            kept[pos] = j;
            if (sel) sel[(size_t)bh * kk + pos] = j;
        }
        carry_keep += (uint32_t)__popcll(bk);
    }
    tk_wave_sync();

    // ---- P.V over the kept rows
    const uint8_t *vbase = vc + rowbase * (D / 2) + part * 16;
    const uint32_t *vmb = vm + rowbase * G + grp;
    float o[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) o[e] = 0.f;
    float l_acc = 0.f, m_acc = 0.f;
    const float ml2 = m * kTkLog2e;
    constexpr int PV_U = 4;
    for (int i0 = 0; i0 < kk; i0 += PV_U * TPI) {
        uint4 Vr[PV_U];
        uint32_t Vm[PV_U];
        int jj[PV_U];
#pragma unroll
        for (int u = 0; u < PV_U; ++u) {
            const int i = i0 + u * TPI + slot;
            jj[u] = i < kk ? min(max(kept[i], 0), L - 1) : -1;
            if (jj[u] >= 0) {
                Vr[u] = tk_stream_load16(vbase + (size_t)jj[u] * (D / 2));
                Vm[u] = __builtin_nontemporal_load(vmb + (size_t)jj[u] * G);
            }
        }
#pragma unroll
        for (int u = 0; u < PV_U; ++u) {
            if (jj[u] < 0) continue;
            const float p = __builtin_amdgcn_exp2f(sc[jj[u]] * kTkLog2e - ml2);
            l_acc += p;
            m_acc += p * h2f((uint16_t)(Vm[u] & 0xffffu));
            tk_pv(o, Vr[u], p * h2f((uint16_t)(Vm[u] >> 16)));
        }
    }
    // sum over the token slots (lanes with the same part)
#pragma unroll
    for (int off = PARTS; off < 64; off <<= 1) {
#pragma unroll
        for (int e = 0; e < 32; ++e) o[e] += __shfl_xor(o[e], off, 64);
        l_acc += __shfl_xor(l_acc, off, 64);
        m_acc += __shfl_xor(m_acc, off, 64);
    }
    if (slot == 0) {
        const float inv = 1.0f / l_acc;
        const size_t ob = (size_t)bh * D + part * 32;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            const float v = (o[e] + m_acc) * inv;
            if (out_f16)
                static_cast<_Float16 *>(out)[ob + e] = (_Float16)v;
            else
                static_cast<float *>(out)[ob + e] = v;
        }
    }
}


// Long contexts, where the fp32 scores of one (b, h) no longer fit in LDS.
// The same selection and output, with a 16-bit key per position in LDS:
//  * the K stream stores the upper 16 bits of each position's order key
//    and keeps the exact fp32 maximum;
//  * a radix select over those 16 bits finds the bucket holding the
//    kk-th largest key; when every candidate left in it is kept, the cut is
//    found;
//  * otherwise the candidates (the positions of that one bucket, usually a
//    few hundred) get their scores recomputed from their K rows, their low
//    16 key bits replace the stored ones (a bitmap marks them), and two more
//    radix passes over those bits find the exact cut;
//  * the ordered compaction (four tiles of positions per barrier round) fills
//    an LDS buffer of kept positions, and each time it is half full the P.V
//    pass runs over it, recomputing each kept position's score from its K row
//    (the same operations as the stream, so the same fp32 value) and reading
//    its V row.
// Bytes: every K row once, the kept K and V rows once more (plus the
// candidates' K rows when the bucket does not settle the cut).
constexpr int kTkLongThreads = 512;  // 8 waves per (b, h): more K rows in flight
constexpr int kTkLongUnroll = 8;     // token groups of K loads in flight per wave
constexpr int kTkLongSub = 4;        // tiles of kTkLongThreads positions per compaction round
constexpr int kTkLongRound = kTkLongSub * kTkLongThreads;
constexpr int kTkLongKept = 2 * kTkLongRound;   // kept positions buffered between P.V passes

// Histograms of the long kernel: four copies (lane % 4 picks one) at a
// stride of 257 words, so the lanes of a wave that share a digit (the first
// digit of nearby scores is often the same) spread over four addresses in
// four banks.
constexpr int kTkHistCopies = 4;
constexpr int kTkHistStride = 257;
constexpr int kTkHistWords = kTkHistCopies * kTkHistStride;

__device__ __forceinline__ void tk_hist_clear(uint32_t *hist) {
    for (int i = threadIdx.x; i < kTkHistWords; i += blockDim.x) hist[i] = 0u;
}

__device__ __forceinline__ void tk_hist_add(uint32_t *hist, uint32_t bin) {
    atomicAdd(&hist[(threadIdx.x & (kTkHistCopies - 1)) * kTkHistStride + bin], 1u);
}

// The bin of the rem-th largest candidate once the histogram is complete:
// S(t) = candidates with digit >= t; the bin t with S(t) >= rem and
// S(t + 1) < rem.  Leaves the digit, the rank inside the bin and the bin's
// count in sh[0..2]; every thread reads them after the barrier at the end.
template <int NW>
__device__ __forceinline__ void tk_pick_bin(const uint32_t *hist, uint32_t *wsum, uint32_t *sh, uint32_t rem) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    uint32_t hv = 0;
    if (tid < 256) {
#pragma unroll
        for (int c = 0; c < kTkHistCopies; ++c) hv += hist[c * kTkHistStride + tid];
    }
    uint32_t x = hv;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_down(x, off, 64);
        if (lane + off < 64) x += y;
    }
    if (lane == 0) wsum[wv] = x;
    __syncthreads();
    uint32_t S = x;
    for (int w = wv + 1; w < NW; ++w) S += wsum[w];
    const uint32_t S_above = S - hv;
    if (S >= rem && S_above < rem) {   // exactly one bin satisfies this
        sh[0] = (uint32_t)tid;
        sh[1] = rem - S_above;
        sh[2] = hv;
    }
    __syncthreads();
}

// The eight waves' counts of one tile (16-byte aligned): the sum over the
// waves before this one, and the total.
__device__ __forceinline__ void tk_wave_counts(const uint32_t *c8, uint32_t &before, uint32_t &total) {
    const int wv = threadIdx.x >> 6;
    const uint4 a = *reinterpret_cast<const uint4 *>(c8);
    const uint4 b = *reinterpret_cast<const uint4 *>(c8 + 4);
    const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        before += w < wv ? v[w] : 0u;
        total += v[w];
    }
}

template <int D>
__global__ __launch_bounds__(kTkLongThreads) void attn_topk_long_kernel(
    const uint8_t *__restrict__ kc, const uint32_t *__restrict__ km, const uint8_t *__restrict__ vc,
    const uint32_t *__restrict__ vm, const uint16_t *__restrict__ q, int H, int cap, int L, int kk, float scale,
    void *__restrict__ out, int out_f16, int32_t *__restrict__ sel) {
    constexpr int PARTS = D / 32;    // lanes per token row
    constexpr int TPI = 64 / PARTS;  // tokens per wave per load
    constexpr int G = D / 64;        // groups per token row
    constexpr int NW = kTkLongThreads / 64;
    constexpr int TH = kTkLongThreads;
    constexpr int SUB = kTkLongSub;
    static_assert(NW == 8, "tk_wave_counts reads eight wave counts");
    extern __shared__ uint32_t tk_long_smem[];   // key16 [L] as (L+1)/2 words, then the candidate bitmap
    __shared__ __align__(16) int32_t kept[kTkLongKept];
    __shared__ uint32_t hist[kTkHistWords];
    __shared__ __align__(16) uint32_t cnt[2][SUB][NW];
    __shared__ float wmax[NW];
    __shared__ uint32_t sh[3];
    // the final reduction reuses the kept buffer (no P.V pass reads it then)
    static_assert((NW * D + NW * PARTS + NW) * 4 <= kTkLongKept * 4, "reduction fits the kept buffer");
    float(*red_o)[D] = reinterpret_cast<float(*)[D]>(kept);
    float(*red_m)[PARTS] = reinterpret_cast<float(*)[PARTS]>(reinterpret_cast<float *>(kept) + NW * D);
    float *red_l = reinterpret_cast<float *>(kept) + NW * D + NW * PARTS;

    uint16_t *key16 = reinterpret_cast<uint16_t *>(tk_long_smem);
    uint32_t *cbits = tk_long_smem + (L + 1) / 2;
    const int nwords = (L + 31) / 32;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int bh = blockIdx.x;
    const int slot = lane / PARTS, part = lane % PARTS, grp = part >> 1;
    const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));

    uint32_t QP[4][4];
    float qsum;
    tk_query<D>(q, bh, part, QP, qsum);

    const size_t rowbase = (size_t)bh * cap;
    const uint8_t *kbase = kc + rowbase * (D / 2) + part * 16;
    const uint32_t *kmb = km + rowbase * G + grp;
    const uint8_t *vbase = vc + rowbase * (D / 2) + part * 16;
    const uint32_t *vmb = vm + rowbase * G + grp;

    tk_hist_clear(hist);
    for (int w = tid; w < nwords; w += TH) cbits[w] = 0u;
    __syncthreads();

    // ---- scores of every position: the upper key bits into LDS, the maximum
    float lmax = -INFINITY;
    constexpr int BLOCK_TOK = kTkLongUnroll * NW * TPI;
    for (int base = 0; base < L; base += BLOCK_TOK) {
        uint4 Kr[kTkLongUnroll];
        uint32_t Km[kTkLongUnroll];
#pragma unroll
        for (int u = 0; u < kTkLongUnroll; ++u) {
            const int j = base + (u * NW + wv) * TPI + slot;
            const size_t jc = (size_t)(j < L ? j : L - 1);   // past the end: re-read the last row
            Kr[u] = tk_stream_load16(kbase + jc * (D / 2));
            Km[u] = __builtin_nontemporal_load(kmb + jc * G);
        }
#pragma unroll
        for (int u = 0; u < kTkLongUnroll; ++u) {
            const int j = base + (u * NW + wv) * TPI + slot;
            const float s = tk_score<PARTS>(Kr[u], Km[u], QP, qsum, scale);
            if (j < L) {
                if (part == 0) key16[j] = (uint16_t)(order_key(s) >> 16);
                lmax = fmaxf(lmax, s);
            }
        }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, off, 64));
    if (lane == 0) wmax[wv] = lmax;
    __syncthreads();
    float m = wmax[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) m = fmaxf(m, wmax[w]);

    // ---- radix select over the upper 16 key bits (two 8-bit digits)
    uint32_t prefix = 0, pmask = 0, rem = (uint32_t)kk;
    bool settled = false;
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
        const int shift = 8 - 8 * pass;
        if (pass > 0) {
            tk_hist_clear(hist);
            __syncthreads();
        }
        for (int j0 = tid; j0 < L; j0 += 4 * TH) {
            uint32_t key[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = j0 + u * TH;
                key[u] = key16[j < L ? j : 0];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (j0 + u * TH < L && (key[u] & pmask) == prefix) tk_hist_add(hist, (key[u] >> shift) & 255u);
        }
        __syncthreads();
        tk_pick_bin<NW>(hist, cnt[0][0], sh, rem);
        prefix |= sh[0] << shift;
        pmask |= 255u << shift;
        rem = sh[1];
        if (rem == sh[2]) {   // every candidate left is kept: the cut is found
            settled = true;
            break;
        }
    }

    // ---- otherwise refine inside the one 16-bit bucket `prefix`: recompute
    // its positions' scores, store their low 16 key bits, mark them
    uint32_t lo_prefix = 0, lo_mask = 0;
    if (!settled) {
        uint32_t nbuf = 0;
        for (int base = 0;; base += kTkLongRound) {
            const bool more = base < L;
            if (more) {
                uint64_t bc[SUB];
#pragma unroll
                for (int u = 0; u < SUB; ++u) {
                    const int j = base + u * TH + tid;
                    bc[u] = __ballot(j < L && key16[j] == prefix);
                    if (lane == 0) cnt[0][u][wv] = (uint32_t)__popcll(bc[u]);
                }
                __syncthreads();
                uint32_t run = nbuf;
#pragma unroll
                for (int u = 0; u < SUB; ++u) {
                    const int j = base + u * TH + tid;
                    uint32_t before, total;
                    tk_wave_counts(cnt[0][u], before, total);
                    if ((bc[u] >> lane) & 1ull) kept[run + before + (uint32_t)__popcll(bc[u] & lt_mask)] = j;
                    run += total;
                }
                nbuf = run;
                __syncthreads();
            }
            // recompute the buffered candidates once the buffer is half full, and at the end
            if (nbuf > 0 && (!more || nbuf + kTkLongRound > (uint32_t)kTkLongKept)) {
                for (uint32_t i0 = 0; i0 < nbuf; i0 += NW * TPI) {
                    const uint32_t i = i0 + wv * TPI + slot;
                    const int j = kept[i < nbuf ? i : nbuf - 1];
                    const uint4 kr = tk_stream_load16(kbase + (size_t)j * (D / 2));
                    const uint32_t kmeta = __builtin_nontemporal_load(kmb + (size_t)j * G);
                    const float s = tk_score<PARTS>(kr, kmeta, QP, qsum, scale);
                    if (i < nbuf && part == 0) {
                        key16[j] = (uint16_t)(order_key(s) & 0xffffu);
                        atomicOr(&cbits[j >> 5], 1u << (j & 31));
                    }
                }
                nbuf = 0;
                __syncthreads();
            }
            if (!more) break;
        }
        // two radix passes over the candidates' low 16 bits
#pragma unroll 1
        for (int pass = 0; pass < 2; ++pass) {
            const int shift = 8 - 8 * pass;
            tk_hist_clear(hist);
            __syncthreads();
            for (int j = tid; j < L; j += TH) {
                if (!((cbits[j >> 5] >> (j & 31)) & 1u)) continue;
                const uint32_t key = key16[j];
                if ((key & lo_mask) == lo_prefix) tk_hist_add(hist, (key >> shift) & 255u);
            }
            __syncthreads();
            tk_pick_bin<NW>(hist, cnt[0][0], sh, rem);
            lo_prefix |= sh[0] << shift;
            lo_mask |= 255u << shift;
            rem = sh[1];
            if (rem == sh[2]) break;
        }
    }
    // Kept: positions whose upper key bits (masked by pmask) exceed prefix;
    // when settled, every one equal to it; otherwise the candidates whose low
    // bits (masked by lo_mask) exceed lo_prefix, and the first `rem` by
    // position of those equal to it.

    // ---- ordered compaction into the LDS buffer, P.V each time it is half full
    float o[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) o[e] = 0.f;
    float l_acc = 0.f, m_acc = 0.f;
    const float ml2 = m * kTkLog2e;
    uint32_t carry_eq = 0, nbuf = 0, flushed = 0;
    for (int base = 0;; base += kTkLongRound) {
        const bool more = base < L;
        if (more) {
            bool gt[SUB];
            uint64_t be[SUB];
#pragma unroll
            for (int u = 0; u < SUB; ++u) {
                const int j = base + u * TH + tid;
                bool g = false, e = false;
                if (j < L) {
                    const uint32_t key = key16[j];
                    if (!settled && ((cbits[j >> 5] >> (j & 31)) & 1u)) {
                        g = (key & lo_mask) > lo_prefix;
                        e = (key & lo_mask) == lo_prefix;
                    } else {
                        g = (key & pmask) > prefix;
                        e = settled && (key & pmask) == prefix;
                    }
                }
                gt[u] = g;
                be[u] = __ballot(e);
                if (lane == 0) cnt[0][u][wv] = (uint32_t)__popcll(be[u]);
            }
            __syncthreads();
            uint64_t bk[SUB];
            uint32_t run = carry_eq;
#pragma unroll
            for (int u = 0; u < SUB; ++u) {
                uint32_t before, total;
                tk_wave_counts(cnt[0][u], before, total);
                const bool e = (be[u] >> lane) & 1ull;
                const bool keep = gt[u] || (e && run + before + (uint32_t)__popcll(be[u] & lt_mask) < rem);
                run += total;
                bk[u] = __ballot(keep);
                if (lane == 0) cnt[1][u][wv] = (uint32_t)__popcll(bk[u]);
            }
            carry_eq = run;
            __syncthreads();
            uint32_t runk = nbuf;
#pragma unroll
            for (int u = 0; u < SUB; ++u) {
                const int j = base + u * TH + tid;
                uint32_t before, total;
                tk_wave_counts(cnt[1][u], before, total);
                const uint32_t pos = runk + before + (uint32_t)__popcll(bk[u] & lt_mask);
                if (((bk[u] >> lane) & 1ull) && flushed + pos < (uint32_t)kk) {
                    kept[pos] = j;
                    if (sel) sel[(size_t)bh * kk + flushed + pos] = j;
                }
                runk += total;
            }
            nbuf = runk;
            if (flushed + nbuf > (uint32_t)kk) nbuf = (uint32_t)kk - flushed;   // never more than kk in all
            __syncthreads();
        }
        if (nbuf > 0 && (!more || nbuf + kTkLongRound > (uint32_t)kTkLongKept)) {
            constexpr int PV_U = 4;
            for (uint32_t i0 = 0; i0 < nbuf; i0 += PV_U * NW * TPI) {
                uint4 Kr[PV_U], Vr[PV_U];
                uint32_t Kmeta[PV_U], Vmeta[PV_U];
                bool ok[PV_U];
#pragma unroll
                for (int u = 0; u < PV_U; ++u) {
                    const uint32_t i = i0 + (u * NW + wv) * TPI + slot;
                    ok[u] = i < nbuf;
                    const size_t j = (size_t)min(max(kept[ok[u] ? i : nbuf - 1], 0), L - 1);
                    Kr[u] = tk_stream_load16(kbase + j * (D / 2));
                    Kmeta[u] = __builtin_nontemporal_load(kmb + j * G);
                    Vr[u] = tk_stream_load16(vbase + j * (D / 2));
                    Vmeta[u] = __builtin_nontemporal_load(vmb + j * G);
                }
#pragma unroll
                for (int u = 0; u < PV_U; ++u) {
                    const float s = tk_score<PARTS>(Kr[u], Kmeta[u], QP, qsum, scale);
                    if (!ok[u]) continue;
                    const float p = __builtin_amdgcn_exp2f(s * kTkLog2e - ml2);
                    l_acc += p;
                    m_acc += p * h2f((uint16_t)(Vmeta[u] & 0xffffu));
                    tk_pv(o, Vr[u], p * h2f((uint16_t)(Vmeta[u] >> 16)));
                }
            }
            flushed += nbuf;
            nbuf = 0;
            __syncthreads();
        }
        if (!more) break;
    }

    // sum over the token slots of the wave (lanes with the same part), then over waves
#pragma unroll
    for (int off = PARTS; off < 64; off <<= 1) {
#pragma unroll
        for (int e = 0; e < 32; ++e) o[e] += __shfl_xor(o[e], off, 64);
        l_acc += __shfl_xor(l_acc, off, 64);
        m_acc += __shfl_xor(m_acc, off, 64);
    }
    if (slot == 0) {
#pragma unroll
        for (int e = 0; e < 32; ++e) red_o[wv][part * 32 + e] = o[e];
        red_m[wv][part] = m_acc;
        if (part == 0) red_l[wv] = l_acc;
    }
    __syncthreads();
    if (tid < D) {
        float num = 0.f, mins = 0.f, den = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            num += red_o[w][tid];
            mins += red_m[w][tid / 32];
            den += red_l[w];
        }
        const float v = (num + mins) / den;
        if (out_f16)
            static_cast<_Float16 *>(out)[(size_t)bh * D + tid] = (_Float16)v;
        else
            static_cast<float *>(out)[(size_t)bh * D + tid] = v;
    }
}

}  // namespace

size_t attn_topk_lds_bytes(int32_t kv_len, int32_t kept) {
    return ((size_t)kv_len + (size_t)kept) * 4;
}

// Dynamic LDS of the long-context kernel: 16-bit keys and the candidate bitmap.
size_t attn_topk_long_lds_bytes(int32_t kv_len) {
    return (((size_t)kv_len + 1) / 2 + ((size_t)kv_len + 31) / 32) * 4;
}

// Scores and kept list in fp32 up to this many bytes of LDS: with the
// kernel's ~2.1 KB of static LDS, two workgroups still share a CU's 160 KB
// (kv_len + kk <= 19840 positions); longer contexts take the 16-bit-key
// kernel.  At 16416 positions the fp32 kernel took 6-7% less time than the
// 16-bit-key kernel for kk from 16 to 3200 (it re-reads no K rows and needs
// no refinement).
constexpr size_t kTopkF32Lds = 19840 * 4;

// Contexts up to this length run one wavefront per (sequence, head); longer
// ones one workgroup per (sequence, head).
constexpr int kTopkWaveMaxLen = 2048;

fgq_status launch_decode_attn_topk(const fgq_kv_cache *kv, const void *q, int32_t kv_len, int32_t kept,
                                   float scale, void *out, int32_t out_dtype, int32_t *sel, hipStream_t stream) {
    if (kv->batch == 0 || kv->heads == 0) return FGQ_OK;
    const int64_t items = (int64_t)kv->batch * kv->heads;
    const int f16 = out_dtype == FGQ_DTYPE_F16;
    const uint16_t *qh = static_cast<const uint16_t *>(q);
    if (kv_len <= kTopkWaveMaxLen) {
        const int words = (256 + kv_len + kept + 3) & ~3;
        // waves per workgroup: as many as fit 64 KB of LDS (>= 3 here: words <= 4352)
        const int wpb = std::min(4, (int)(65536 / ((size_t)words * 4)));
        const size_t lds = (size_t)wpb * words * 4;
        const dim3 grid((unsigned)((items + wpb - 1) / wpb)), block(64 * wpb);
        const int kr = kv_len <= 128 ? 2 : kv_len <= 256 ? 4 : kv_len <= 512 ? 8 : kv_len <= 1024 ? 16 : 32;
#define FGQ_TOPK_WAVE(DD, KRR)                                                                                   \
    attn_topk_wave_kernel<DD, KRR><<<grid, block, lds, stream>>>(kv->k_codes, kv->k_meta, kv->v_codes, kv->v_meta, \
                                                                 qh, kv->heads, kv->capacity, kv_len, kept, scale,  \
                                                                 out, f16, sel, (int)items, words)
        if (kv->head_dim == 128) {
            switch (kr) {
                case 2: FGQ_TOPK_WAVE(128, 2); break;
                case 4: FGQ_TOPK_WAVE(128, 4); break;
                case 8: FGQ_TOPK_WAVE(128, 8); break;
                case 16: FGQ_TOPK_WAVE(128, 16); break;
                default: FGQ_TOPK_WAVE(128, 32); break;
            }
        } else {
            switch (kr) {
                case 2: FGQ_TOPK_WAVE(64, 2); break;
                case 4: FGQ_TOPK_WAVE(64, 4); break;
                case 8: FGQ_TOPK_WAVE(64, 8); break;
                case 16: FGQ_TOPK_WAVE(64, 16); break;
                default: FGQ_TOPK_WAVE(64, 32); break;
            }
        }
#undef FGQ_TOPK_WAVE
        return check_launch("attn_topk_wave_kernel");
    }
    const size_t lds = attn_topk_lds_bytes(kv_len, kept);
    if (lds <= kTopkF32Lds) {
        if (kv->head_dim == 128)
            attn_topk_kernel<128><<<dim3((unsigned)items), dim3(kTkThreads), lds, stream>>>(
                kv->k_codes, kv->k_meta, kv->v_codes, kv->v_meta, qh, kv->heads, kv->capacity, kv_len, kept, scale,
                out, f16, sel);
        else
            attn_topk_kernel<64><<<dim3((unsigned)items), dim3(kTkThreads), lds, stream>>>(
                kv->k_codes, kv->k_meta, kv->v_codes, kv->v_meta, qh, kv->heads, kv->capacity, kv_len, kept, scale,
                out, f16, sel);
        return check_launch("attn_topk_kernel");
    }
    // long contexts: 16-bit keys and a candidate bitmap in LDS
    const void *fn = kv->head_dim == 128 ? reinterpret_cast<const void *>(&attn_topk_long_kernel<128>)
                                         : reinterpret_cast<const void *>(&attn_topk_long_kernel<64>);
    const size_t lds_long = attn_topk_long_lds_bytes(kv_len);
    int dev = 0, max_lds = 0;
    hipFuncAttributes fa{};
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e == hipSuccess) e = hipFuncGetAttributes(&fa, fn);
    if (e != hipSuccess) return fail(FGQ_ERR_DEVICE, "top-k attention: %s", hipGetErrorString(e));
    if (lds_long + fa.sharedSizeBytes > (size_t)max_lds)
        return fail(FGQ_ERR_UNSUPPORTED, "kv_len %d needs %zu bytes of LDS per workgroup (device: %d)", kv_len,
                    lds_long + fa.sharedSizeBytes, max_lds);
    if (kv->head_dim == 128)
        attn_topk_long_kernel<128><<<dim3((unsigned)items), dim3(kTkLongThreads), lds_long, stream>>>(
            kv->k_codes, kv->k_meta, kv->v_codes, kv->v_meta, qh, kv->heads, kv->capacity, kv_len, kept, scale, out,
            f16, sel);
    else
        attn_topk_long_kernel<64><<<dim3((unsigned)items), dim3(kTkLongThreads), lds_long, stream>>>(
            kv->k_codes, kv->k_meta, kv->v_codes, kv->v_meta, qh, kv->heads, kv->capacity, kv_len, kept, scale, out,
            f16, sel);
    return check_launch("attn_topk_long_kernel");
}

}  // namespace fgq
