// Grouped-query (GQA) and multi-query (MQA) decode attention over the 4-bit
// compressed KV cache.
//
// What is computed: the vTensor page on papercache.org, background section
// "GQA and MQA optimisation" (query heads are divided into groups and each
// group shares one key head and one value head; MQA is a single shared head),
// with the compressed cache of the FlexGen pages (codes restored before
// compute: FlexGen review on blog.gzher.com, section 3.4).  With
// R = q_heads / kv_heads, query head hq reads cache head kh = hq / R:
//   s_j = scale * sum_d q_{hq,d} * (min_{kh,j,g(d)} + c_{kh,j,d} * step_{kh,j,g(d)})
//   o_d = sum_j softmax(s)_j * (min + c * step)  of the V cache
//
// Why the matrix cores: the R query heads of a group read the same K and V
// rows, so per cached element the work is R multiply-adds for q.k and R for
// p.v (the vTensor page, "Roofline comparison", Figure 3: fewer shared heads
// raise the arithmetic intensity).  At R >= ~4 that outgrows the vector ALUs
// while the cache is still streamed from HBM, so both products run on
// v_mfma_f32_16x16x32_f16 with the codes as the fp16 operand:
//  * a code c enters the matrix core as the fp16 subnormal c * 2^-24 (one AND
//    of the packed word), so products and sums are exact in the fp32
//    accumulator; the scale 2^24 and the group's step and minimum are applied
//    per (token, group) afterwards:
//      q.k^ = sum_g [ step_g * 2^24 * (sum_{d in g} q_d (c_d 2^-24)) + min_g * sum_{d in g} q_d ]
//  * S^T = K Q^T: A = 16 tokens x 32 codes of one group, B = the group's
//    query fragments (up to 16 heads per MFMA column tile, held in registers
//    for the whole sequence), one accumulator per group;
//  * O^T = V^T (P*step)^T: the k index of the MFMA is the token, so the B
//    operand is fp16(p_j * step_{j,g}) straight from the score accumulators
//    (a lane's accumulator rows are the tokens of its k-slots), and the A
//    operand is each token's V codes of 4 consecutive d (one 16-bit load per
//    token and group, two tokens packed per register, one shift and AND per
//    d); every MFMA's 16 output rows lie in one group; the minimum term
//    sum_j p_j min_{j,g} is a per-(head, group) scalar;
//  * online softmax in the log2 domain on the transposed scores: every
//    accumulator of a lane belongs to one query head, so the max, the
//    exponentials and the rescale stay in the lane except for a two-step
//    max across the four lane groups;
//  * a workgroup of 4 waves takes one (sequence, kv head, split); the waves
//    take interleaved 32-token blocks and merge their softmax states in LDS,
//    so one partial state per split goes to the workspace (a second kernel
//    merges the splits when there are several).
#include <type_traits>

#include "common.h"

namespace fgq {
namespace {

constexpr float kGqLog2e = 1.4426950408889634f;
constexpr int kGqWaves = 4;    // waves per workgroup
constexpr int kGqBlock = 32;   // tokens per wave iteration: two 16-token MFMA tiles
#ifndef FGQ_GQA_RING
#define FGQ_GQA_RING 3         // blocks per wave in the load ring (RING - 1 in flight)
#endif
#ifndef FGQ_GQA_WAVE_ITEMS
#define FGQ_GQA_WAVE_ITEMS 2048 // (sequence, K/V head) pairs from which each pair gets one wave
#endif
#ifndef FGQ_GQA_WAVES_PER_EU
#define FGQ_GQA_WAVES_PER_EU 2 // occupancy the register budget is fitted to
#endif
constexpr int kGqRing = FGQ_GQA_RING;
constexpr uint32_t kLow4 = 0x000F000Fu;    // nibbles 0 and 4 of a word: codes * 2^-24 as fp16
constexpr uint32_t kHigh4 = 0x00F000F0u;   // nibbles 1 and 5: codes * 2^-20

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f16x8 pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const u32x4 v = {a, b, c, d};
    return __builtin_bit_cast(f16x8, v);
}

// The 8 codes of a packed word as fp16 subnormals, in the k-slot order
// [n0, n4, n1, n5, n2, n6, n3, n7] (nibble i = element i of the word):
// nibbles 0, 4 (and 2, 6 after one shift) land in the low mantissa bits as
// c * 2^-24, nibbles 1, 5 (3, 7) four bits up as c * 2^-20.  The matching
// query slots carry q / 16, so every product is c * q * 2^-24.
__device__ __forceinline__ f16x8 codes_as_f16(uint32_t w) {
    const uint32_t w8 = w >> 8;
    return pack4(w & kLow4, w & kHigh4, w8 & kLow4, w8 & kHigh4);
}

__device__ __forceinline__ float lo_f(uint32_t m) { return (float)as_f16x2(m).x; }
__device__ __forceinline__ float hi_f(uint32_t m) { return (float)as_f16x2(m).y; }

// Cache rows of one 32-token block as they arrive (coalesced loads; lane
// (c, g) = (lane % 16, lane / 16)):
//  kw[t][grp]  K codes of token 16t + c, bytes 32grp + 8g .. +7: the q.k A
//              operand, used straight from registers;
//  vr[i]       16 bytes of V codes: token (8/G)i + lane/(4G)... i.e. whole
//              rows, 4G lanes per row of D/2 bytes;
//  mt          one token's K meta (lanes 0-31) or V meta (lanes 32-63).
// The V codes and the meta pass through a per-wave LDS stage to reach the
// lanes that need them (a lane's score rows are tokens 16t + 4g + r).
template <int G>
struct GqBlock {
    u32x2 kw[2][G];
    u32x4 vr[G];
    uint32_t mt[G];
};

// WPI = waves per work item (sequence, K/V head, split): 4 (the workgroup's
// waves share the item and merge in LDS) when there are few items, 1 (four
// independent items per workgroup) when there are enough to fill the chip.
template <int D, int NT, int WPI>
__global__ __launch_bounds__(64 * kGqWaves)
__attribute__((amdgpu_waves_per_eu(NT == 1 ? FGQ_GQA_WAVES_PER_EU : 1))) void attn_gqa_kernel(
    const uint8_t *__restrict__ kc, const uint32_t *__restrict__ km, const uint8_t *__restrict__ vc,
    const uint32_t *__restrict__ vm, const uint16_t *__restrict__ q, int Hkv, int R, int cap, int L, int n_split,
    int tok_per_split, int total_items, float sl2, float *__restrict__ ws, void *__restrict__ out, int out_f16) {
    static_assert(WPI == 1 || WPI == kGqWaves, "a work item takes one wave or the whole workgroup");
    constexpr int G = D / 64;       // groups per token row
    constexpr int KS = 2 * G;       // q.k MFMA k-steps (32 d each)
    constexpr int NDT = 4 * G;      // p.v output tiles of 16 d
    constexpr int RB = D / 2;       // code bytes per token row
    constexpr int VS = RB + 8;      // LDS row stride of the V stage (bank-conflict-free 16-bit reads)
    constexpr int LPR = RB / 16;    // lanes per V row (16 bytes each)
    __shared__ float s_o[kGqWaves * NDT * NT * 4][64];
    __shared__ float s_m[kGqWaves][NT][16], s_l[kGqWaves][NT][16], s_mc[kGqWaves][G][NT][16];
    __shared__ __attribute__((aligned(16))) uint8_t s_v[kGqWaves][kGqBlock * VS];
    // the block's metadata converted once, as fp32 pairs: K {step * c2, min}, V {step, min}
    __shared__ __attribute__((aligned(16))) float2 s_meta[kGqWaves][2][kGqBlock * G];

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int c = lane & 15, g = lane >> 4;
    const int item = WPI == 1 ? (int)blockIdx.x * kGqWaves + wv : (int)blockIdx.x;
    if (WPI == 1 && item >= total_items) return;   // wave-uniform; no workgroup barrier on this path
    const int wi = WPI == 1 ? 0 : wv;               // the wave's place within its item
    const int split = item % n_split;
    const int bk = item / n_split;           // b * Hkv + kv head
    const int b = bk / Hkv, kh = bk - b * Hkv;
    const int Hq = Hkv * R;
    const int j0 = split * tok_per_split;
    const int j1 = min(L, j0 + tok_per_split);

    // ---- query fragments (B operands) and per-group query sums of the
    // lane's head column(s): k-step s = 2 grp + hh covers
    // d = 64 grp + 16 g + 8 hh + [0, 4, 1, 5, 2, 6, 3, 7]
    f16x8 qf[KS][NT];
    float qs[G][NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int col = 16 * nt + c;
        const bool valid = col < R;
        const uint16_t *qrow = q + ((size_t)b * Hq + (size_t)kh * R + (valid ? col : 0)) * D;
#pragma unroll
        for (int grp = 0; grp < G; ++grp) {
            float part = 0.f;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                uint4 w = *reinterpret_cast<const uint4 *>(qrow + 64 * grp + 16 * g + 8 * hh);
                if (!valid) w = make_uint4(0u, 0u, 0u, 0u);
                // slots (d1, d5) and (d3, d7) meet codes scaled by 2^-20: q / 16
                // there (exact unless |q| < 2^-10, then within 2^-25)
                const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
                qf[2 * grp + hh][nt] = pack4(__builtin_amdgcn_perm(w.z, w.x, 0x05040100u),
                                             as_u32(as_f16x2(__builtin_amdgcn_perm(w.z, w.x, 0x07060302u)) * sixteenth),
                                             __builtin_amdgcn_perm(w.w, w.y, 0x05040100u),
                                             as_u32(as_f16x2(__builtin_amdgcn_perm(w.w, w.y, 0x07060302u)) * sixteenth));
                const uint32_t ws4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) part += lo_f(ws4[i]) + hi_f(ws4[i]);
            }
            part += __shfl_xor(part, 16, 64);
            part += __shfl_xor(part, 32, 64);
            qs[grp][nt] = part * 5.9604644775390625e-08f;   // * 2^-24, matching the code scale
        }
    }
    const float c2 = sl2 * 16777216.0f;   // log2-domain scale times 2^24
    float qsc[G][NT];                     // the query sums in the scores' scale
#pragma unroll
    for (int grp = 0; grp < G; ++grp)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) qsc[grp][nt] = qs[grp][nt] * c2;

    // (sequence, kv head) bases; offsets inside one head's rows fit in 32 bits
    const size_t rowbase = (size_t)bk * cap;
    const uint8_t *kcb = kc + rowbase * RB;
    const uint8_t *vcb = vc + rowbase * RB;
    const uint32_t *mb = (lane < 32 ? km : vm) + rowbase * G;
    const int vrow_lane = lane / LPR, vcol = 16 * (lane % LPR);   // V rows: 64/LPR per load
    constexpr int VROWS = 64 / LPR;

    auto load = [&](int jb, GqBlock<G> &d) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t jk = (uint32_t)min(jb + 16 * t + c, j1 - 1);
#pragma unroll
            for (int grp = 0; grp < G; ++grp)
                d.kw[t][grp] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x2 *>(kcb + (jk * RB + 32 * grp + 8 * g)));
        }
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const uint32_t jv = (uint32_t)min(jb + VROWS * i + vrow_lane, j1 - 1);
            d.vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vcb + (jv * RB + vcol)));
        }
        const uint32_t jm = (uint32_t)min(jb + (lane & 31), j1 - 1);
#pragma unroll
        for (int grp = 0; grp < G; ++grp) d.mt[grp] = __builtin_nontemporal_load(mb + (jm * G + grp));
    };

    float m_run[NT], l_run[NT], mc[G][NT];
    f32x4 o[NDT][NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        m_run[nt] = -INFINITY;
        l_run[nt] = 0.f;
#pragma unroll
        for (int grp = 0; grp < G; ++grp) mc[grp][nt] = 0.f;
#pragma unroll
        for (int n = 0; n < NDT; ++n) o[n][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    uint8_t *sv = s_v[wv];
    const float2 *smk = s_meta[wv][0], *smv = s_meta[wv][1];

    // TAIL: the block reaches past the end of the split (the last one)
    auto process = [&](int jb, const GqBlock<G> &d, auto tail) {
        constexpr bool TAIL = decltype(tail)::value;
        // ---- stage the V codes and the meta of the block in LDS (the wave's
        // own region; the previous block's reads are complete: every LDS read
        // result was consumed before this point)
#pragma unroll
        for (int i = 0; i < G; ++i) {
            uint8_t *dst = sv + (VROWS * i + vrow_lane) * VS + vcol;
            *reinterpret_cast<u32x2 *>(dst) = u32x2{d.vr[i][0], d.vr[i][1]};
            *reinterpret_cast<u32x2 *>(dst + 8) = u32x2{d.vr[i][2], d.vr[i][3]};
        }
#pragma unroll
        for (int grp = 0; grp < G; ++grp) {
            const float step = hi_f(d.mt[grp]);
            s_meta[wv][lane >> 5][(lane & 31) * G + grp] = make_float2(lane < 32 ? step * c2 : step, lo_f(d.mt[grp]));
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- S^T = K Q^T per group: acc[t][grp][nt][r] = token 16t + 4g + r, head column c
        f32x4 acc[2][G][NT];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int grp = 0; grp < G; ++grp) {
                const f16x8 a0 = codes_as_f16(d.kw[t][grp][0]);
                const f16x8 a1 = codes_as_f16(d.kw[t][grp][1]);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    z = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, qf[2 * grp][nt], z, 0, 0, 0);
                    acc[t][grp][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, qf[2 * grp + 1][nt], z, 0, 0, 0);
                }
            }
        // ---- the lane's meta (tokens 16t + 4g + r) and V codes from the stage
        float2 kmw[2][4][G], vmw[2][4][G];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const float2 *pk = smk + (16 * t + 4 * g) * G;
            const float2 *pv = smv + (16 * t + 4 * g) * G;
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int grp = 0; grp < G; ++grp) {
                    kmw[t][r][grp] = pk[r * G + grp];
                    vmw[t][r][grp] = pv[r * G + grp];
                }
        }
        uint32_t vv[2][2][G];   // tokens 16t + 4g + 2p (low half) and +1 (high half), d = 64grp + 4c .. +3
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int grp = 0; grp < G; ++grp) {
                    const uint8_t *src = sv + (16 * t + 4 * g + 2 * p) * VS + 32 * grp + 2 * c;
                    u16x2 v;
                    v.x = *reinterpret_cast<const uint16_t *>(src);
                    v.y = *reinterpret_cast<const uint16_t *>(src + VS);
                    vv[t][p][grp] = __builtin_bit_cast(uint32_t, v);
                }

        // ---- scores in the log2 domain; positions past the end of the split are -inf
        float s[NT][2][4];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = 0.f;
#pragma unroll
                    for (int grp = 0; grp < G; ++grp) {
                        const float2 mw = kmw[t][r][grp];
                        v = __builtin_fmaf(mw.x, acc[t][grp][nt][r], v);
                        v = __builtin_fmaf(mw.y, qsc[grp][nt], v);
                    }
                    s[nt][t][r] = v;
                    if (TAIL && jb + 16 * t + 4 * g + r >= j1) s[nt][t][r] = -INFINITY;
                }
        // ---- running max per head column: the block max over the lane's 8
        // rows, then over the four lane groups of the column
        bool moved = false;
        float corr[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            float mx = fmaxf(fmaxf(fmaxf(s[nt][0][0], s[nt][0][1]), fmaxf(s[nt][0][2], s[nt][0][3])),
                             fmaxf(fmaxf(s[nt][1][0], s[nt][1][1]), fmaxf(s[nt][1][2], s[nt][1][3])));
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_new = fmaxf(m_run[nt], mx);
            corr[nt] = __builtin_amdgcn_exp2f(m_run[nt] - m_new);
            moved |= m_new != m_run[nt];
            m_run[nt] = m_new;
        }
        if (__ballot(moved)) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                l_run[nt] *= corr[nt];
#pragma unroll
                for (int grp = 0; grp < G; ++grp) mc[grp][nt] *= corr[nt];
#pragma unroll
                for (int n = 0; n < NDT; ++n) o[n][nt] *= corr[nt];
            }
        }
        // ---- probabilities; the p.v B operands fp16(p * step) per group, in
        // the k-slot order of the score rows (slot e = token 16(e/4) + 4g + e%4)
        f16x8 wb[G][NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = __builtin_amdgcn_exp2f(s[nt][t][r] - m_run[nt]);
                    l_run[nt] += p;
#pragma unroll
                    for (int grp = 0; grp < G; ++grp) {
                        const float2 mw = vmw[t][r][grp];
                        mc[grp][nt] = __builtin_fmaf(p, mw.y, mc[grp][nt]);
                        wb[grp][nt][4 * t + r] = (_Float16)(p * mw.x);
                    }
                }
        // ---- O^T += V^T W^T: tile n = 4 grp + qn holds d = 64 grp + 4 row + qn;
        // its codes are c * 2^-24 (qn even) or c * 2^-20 (qn odd)
#pragma unroll
        for (int n = 0; n < NDT; ++n) {
            const int grp = n / 4, sh = (n % 4) >= 2 ? 8 : 0;
            const uint32_t msk = (n % 2) ? kHigh4 : kLow4;
            const f16x8 a = pack4((vv[0][0][grp] >> sh) & msk, (vv[0][1][grp] >> sh) & msk,
                                  (vv[1][0][grp] >> sh) & msk, (vv[1][1][grp] >> sh) & msk);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                o[n][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, wb[grp][nt], o[n][nt], 0, 0, 0);
        }
    };

    // ---- the wave's blocks: j0 + 32 (wv + 4 i), a ring of kGqRing blocks:
    // the loads of the next kGqRing - 1 are in flight while one is
    // multiplied.  Loads past the end of the split re-read its last row (in
    // bounds, unused), so every iteration issues the same loads and the waits
    // are static.
    constexpr int STRIDE = kGqBlock * WPI;
    int jb = j0 + kGqBlock * wi;
    if (jb < j1) {
        GqBlock<G> buf[kGqRing];
        const std::true_type tail;
        const std::false_type body;
#pragma unroll
        for (int i = 0; i + 1 < kGqRing; ++i) load(jb + i * STRIDE, buf[i]);
        bool more = true;
        while (more) {
#pragma unroll
            for (int i = 0; i < kGqRing; ++i) {
                if (more) {
                    load(jb + (kGqRing - 1) * STRIDE, buf[(i + kGqRing - 1) % kGqRing]);
                    if (jb + kGqBlock <= j1) process(jb, buf[i], body); else process(jb, buf[i], tail);
                    jb += STRIDE;
                    more = jb < j1;
                }
            }
        }
    }

    // ---- the wave's softmax state: l and the minimum terms summed over the
    // four lane groups; o and m are already per column
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        l_run[nt] += __shfl_xor(l_run[nt], 16, 64);
        l_run[nt] += __shfl_xor(l_run[nt], 32, 64);
#pragma unroll
        for (int grp = 0; grp < G; ++grp) {
            mc[grp][nt] += __shfl_xor(mc[grp][nt], 16, 64);
            mc[grp][nt] += __shfl_xor(mc[grp][nt], 32, 64);
        }
    }

    if constexpr (WPI == 1) {
        // ---- one wave holds the whole item: lane (c, g) finishes
        // d = 64 grp + 16 g + 4 r + qn, qn = 0..3 (16-byte stores)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int col = 16 * nt + c;
            if (col >= R) continue;
            const size_t orow = (size_t)b * Hq + (size_t)kh * R + col;
            const float inv = 1.0f / l_run[nt];
#pragma unroll
            for (int grp = 0; grp < G; ++grp)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    f32x4 val;
#pragma unroll
                    for (int qn = 0; qn < 4; ++qn)
                        val[qn] = __builtin_fmaf(o[4 * grp + qn][nt][r], (qn & 1) ? 1048576.0f : 16777216.0f,
                                                 mc[grp][nt]);
                    const int d0 = 64 * grp + 16 * g + 4 * r;
                    if (n_split == 1) {
                        val *= inv;
                        if (out_f16) {
                            _Float16 *op = static_cast<_Float16 *>(out) + orow * D + d0;
                            op[0] = (_Float16)val[0]; op[1] = (_Float16)val[1];
                            op[2] = (_Float16)val[2]; op[3] = (_Float16)val[3];
                        } else {
                            *reinterpret_cast<f32x4 *>(static_cast<float *>(out) + orow * D + d0) = val;
                        }
                    } else {
                        float *wrow = ws + (orow * n_split + split) * (D + 4);
                        *reinterpret_cast<f32x4 *>(wrow + d0) = val;
                        if (grp == 0 && r == 0 && g == 0) {
                            wrow[D] = m_run[nt];
                            wrow[D + 1] = l_run[nt];
                        }
                    }
                }
        }
        return;
    } else {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        if (g == 0) {
            s_m[wv][nt][c] = m_run[nt];
            s_l[wv][nt][c] = l_run[nt];
#pragma unroll
            for (int grp = 0; grp < G; ++grp) s_mc[wv][grp][nt][c] = mc[grp][nt];
        }
#pragma unroll
        for (int n = 0; n < NDT; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) s_o[((wv * NDT + n) * NT + nt) * 4 + r][lane] = o[n][nt][r];
    }
    __syncthreads();
    // ---- merge the 4 waves: wave wv finishes (group, row) pairs wv*G .. wv*G + G-1,
    // i.e. d = 64 grp + 16 g + 4 r + qn for qn = 0..3 (one 16-byte store)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int col = 16 * nt + c;
        float mw[kGqWaves], M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kGqWaves; ++w) {
            mw[w] = s_m[w][nt][c];
            M = fmaxf(M, mw[w]);
        }
        float f[kGqWaves], den = 0.f;
#pragma unroll
        for (int w = 0; w < kGqWaves; ++w) {
            f[w] = __builtin_amdgcn_exp2f(mw[w] - M);   // a wave with no tokens has m = -inf: f = 0
            den = __builtin_fmaf(f[w], s_l[w][nt][c], den);
        }
        const size_t orow = (size_t)b * Hq + (size_t)kh * R + col;
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int pi = wv * G + i, grp = pi / 4, r = pi % 4;
            f32x4 val = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < kGqWaves; ++w) {
                const float base = s_mc[w][grp][nt][c];
#pragma unroll
                for (int qn = 0; qn < 4; ++qn)
                    val[qn] = __builtin_fmaf(
                        f[w],
                        __builtin_fmaf(s_o[((w * NDT + 4 * grp + qn) * NT + nt) * 4 + r][lane],
                                       (qn & 1) ? 1048576.0f : 16777216.0f, base),
                        val[qn]);
            }
            if (col >= R) continue;
            const int d0 = 64 * grp + 16 * g + 4 * r;
            if (n_split == 1) {
                const float inv = 1.0f / den;
                val *= inv;
                if (out_f16) {
                    _Float16 *op = static_cast<_Float16 *>(out) + orow * D + d0;
                    op[0] = (_Float16)val[0]; op[1] = (_Float16)val[1]; op[2] = (_Float16)val[2]; op[3] = (_Float16)val[3];
                } else {
                    *reinterpret_cast<f32x4 *>(static_cast<float *>(out) + orow * D + d0) = val;
                }
            } else {
                float *wrow = ws + (orow * n_split + split) * (D + 4);
                *reinterpret_cast<f32x4 *>(wrow + d0) = val;
                if (wv == 0 && i == 0 && g == 0) {
                    wrow[D] = M;
                    wrow[D + 1] = den;
                }
            }
        }
    }
    }
}

// Merge the n_split partial states (o unnormalised, m in the log2 domain, l)
// of each (sequence, query head): one block of D threads per row.
template <int D>
__global__ __launch_bounds__(128) void attn_gqa_merge_kernel(const float *__restrict__ ws, int n_split,
                                                             void *__restrict__ out, int out_f16) {
    const size_t row = blockIdx.x;
    const int d = threadIdx.x;
    const float *base = ws + row * n_split * (D + 4);
    // unrolled so that the loads of several splits are in flight at once
    float mx = -INFINITY;
#pragma unroll 8
    for (int i = 0; i < n_split; ++i) mx = fmaxf(mx, base[i * (D + 4) + D]);
    float num = 0.f, den = 0.f;
#pragma unroll 8
    for (int i = 0; i < n_split; ++i) {
        const float w = exp2f(base[i * (D + 4) + D] - mx);
        num += w * base[i * (D + 4) + d];
        den += w * base[i * (D + 4) + D + 1];
    }
    const float v = num / den;
    if (out_f16)
        static_cast<_Float16 *>(out)[row * D + d] = (_Float16)v;
    else
        static_cast<float *>(out)[row * D + d] = v;
}

}  // namespace

struct GqaPlan {
    int n_split;
    int tok_per_split;
    int wpi;    // waves per work item
};

// Splits of the sequence: about one resident round of workgroups (two per
// CU up to 8 query heads per K/V head, one above), each split long enough
// that its partial state (R rows of D + 4 floats) stays small against the
// cache bytes it reads.
GqaPlan gqa_plan(int32_t batch, int32_t kv_heads, int32_t group, int32_t kv_len) {
    const int64_t items = (int64_t)batch * kv_heads;
    // enough (sequence, K/V head) pairs for two waves per SIMD: one wave each, no splits
    if (group <= 16 && items >= FGQ_GQA_WAVE_ITEMS) return {1, kv_len, 1};
    constexpr int per_round = kGqBlock * kGqWaves;
    const int64_t target = (group <= 8 ? 2LL : 1LL) * kNumCU;   // workgroups; fewer for wide groups
    int n_split = 1;
    if (items > 0 && items < target) {
        n_split = (int)((target + items - 1) / items);
        const int min_tok = group * 16 > 256 ? group * 16 : 256;
        const int max_split = kv_len / min_tok > 1 ? kv_len / min_tok : 1;
        if (n_split > max_split) n_split = max_split;
    }
    int per = (kv_len + n_split - 1) / n_split;
    per = ((per + per_round - 1) / per_round) * per_round;
    n_split = (kv_len + per - 1) / per;
    return {n_split, per, kGqWaves};
}

size_t gqa_ws_bytes(int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t head_dim, int32_t kv_len) {
    const GqaPlan p = gqa_plan(batch, kv_heads, q_heads / kv_heads, kv_len);
    if (p.n_split <= 1) return 0;
    return (size_t)batch * q_heads * p.n_split * (head_dim + 4) * sizeof(float);
}

fgq_status launch_decode_attn_gqa(const fgq_kv_cache *kv, const void *q, int32_t q_heads, int32_t kv_len,
                                  float scale, void *out, int32_t out_dtype, void *ws, hipStream_t stream) {
    const int R = q_heads / kv->heads;
    const GqaPlan p = gqa_plan(kv->batch, kv->heads, R, kv_len);
    const int64_t items = (int64_t)kv->batch * kv->heads * p.n_split;
    if (items == 0) return FGQ_OK;
    const float sl2 = scale * kGqLog2e;
    const int f16 = out_dtype == FGQ_DTYPE_F16;
    const dim3 grid((unsigned)(p.wpi == 1 ? (items + kGqWaves - 1) / kGqWaves : items)), block(64 * kGqWaves);
    const uint16_t *qh = static_cast<const uint16_t *>(q);
    float *w = static_cast<float *>(ws);
#define FGQ_GQA_LAUNCH(D, NT, WPI)                                                                              \
    attn_gqa_kernel<D, NT, WPI><<<grid, block, 0, stream>>>(kv->k_codes, kv->k_meta, kv->v_codes, kv->v_meta, \
                                                            qh, kv->heads, R, kv->capacity, kv_len, p.n_split, \
                                                            p.tok_per_split, (int)items, sl2, w, out, f16)
    if (kv->head_dim == 128) {
        if (R > 16) FGQ_GQA_LAUNCH(128, 2, kGqWaves);
        else if (p.wpi == 1) FGQ_GQA_LAUNCH(128, 1, 1);
        else FGQ_GQA_LAUNCH(128, 1, kGqWaves);
    } else {
        if (R > 16) FGQ_GQA_LAUNCH(64, 2, kGqWaves);
        else if (p.wpi == 1) FGQ_GQA_LAUNCH(64, 1, 1);
        else FGQ_GQA_LAUNCH(64, 1, kGqWaves);
    }
#undef FGQ_GQA_LAUNCH
    fgq_status s = check_launch("attn_gqa_kernel");
    if (s != FGQ_OK || p.n_split == 1) return s;
    const dim3 mgrid((unsigned)((int64_t)kv->batch * q_heads));
    if (kv->head_dim == 128)
        attn_gqa_merge_kernel<128><<<mgrid, dim3(128), 0, stream>>>(w, p.n_split, out, f16);
    else
        attn_gqa_merge_kernel<64><<<mgrid, dim3(64), 0, stream>>>(w, p.n_split, out, f16);
    return check_launch("attn_gqa_merge_kernel");
}

}  // namespace fgq
