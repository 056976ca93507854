// Decode attention over the 4-bit compressed KV cache (one query per
// sequence and head, every cached position).
//
// What is computed: paper-graph-ui FlexGen summary, section 3.4
// "Computation delegation" (decode attention reads the whole per-layer cache
// and is bound by I/O); FlexGen review on blog.gzher.com, section 3.4 (codes
// are restored before compute).  Per (sequence b, head h):
//   s_j = scale * sum_d q_d * (min_{j,g(d)} + c_{j,d} * step_{j,g(d)})
//   o_d = sum_j softmax(s)_j * (min_{j,g(d)} + c_{j,d} * step_{j,g(d)})
//
// Design (HBM-bound: 1.125 bytes per cached hidden element, ~4 flops):
//  * One wavefront owns one (b, h, split) work item; the sequence is split
//    into n_split ranges when b*h alone would not fill the 256 CUs, and the
//    partial softmax states (m, l, o) are merged by a second kernel.  Long
//    sequences with fewer pairs than that give each item the four waves of a
//    workgroup instead: wave w takes every fourth chunk from chunk w, and the
//    four softmax states are merged in LDS, in wave order (fewer splits, so
//    fewer or no merge launches, and every wave still streams a long run).
//  * Lane = (token slot, part): a token's 64-byte row of codes (head_dim 128)
//    is read by 4 lanes with one 16-byte load each, so a wave streams 16
//    tokens per load instruction, fully coalesced.
//  * The reconstruction is folded out of the element loop:
//      q.k^ = sum_g [ min_g * sum_{d in g} q_d  +  step_g * sum_{d in g} q_d c_d ]
//    and sum q_d c_d uses v_dot2_f32_f16 on pairs of codes placed in the
//    mantissa of fp16 subnormals (c * 2^-24 or c * 2^-20 after a plain AND),
//    so one AND and one dot2 handle two elements with exact products.
//  * P.V is folded the same way: o_d = sum_j p_j min_j + sum_j (p_j step_j) c_{j,d};
//    two tokens share a dot2 (a byte permute interleaves their codes) and the
//    fp16 weight p_j*step_j is split into a high and a low fp16 part so the
//    product keeps ~22 bits.
//  * Scores of a chunk (CH token iterations of 64 / (head_dim / 32) tokens:
//    96 tokens at head_dim 128 with CH = 6) are formed first, the chunk max is
//    taken over the wave, then the exponentials and the P.V pass run with
//    that max: the running accumulators are rescaled at most once per chunk,
//    not per token.
#include <climits>
#include <mutex>
#include <type_traits>

#include "common.h"

namespace fgq {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(as_f16x2(a), as_f16x2(b), c, false);
}

// DPP lane shuffles (a VALU operand modifier, no LDS round trip).
// quad_perm [1,0,3,2] = xor 1, [2,3,0,1] = xor 2; row_ror:n rotates the 16
// lanes of a row by n.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kRowRor4 = 0x124, kRowRor8 = 0x128;

// Sum over the PARTS consecutive lanes of one token.
template <int PARTS>
__device__ __forceinline__ float sum_parts(float v) {
    v += dpp<kQuadXor1>(v);
    if (PARTS == 4) v += dpp<kQuadXor2>(v);
    return v;
}

// Max over all token slots of the wave (the parts of a token hold equal values).
template <int PARTS>
__device__ __forceinline__ float max_slots(float v) {
    if (PARTS == 2) v = fmaxf(v, dpp<kQuadXor2>(v));
    v = fmaxf(v, dpp<kRowRor4>(v));
    v = fmaxf(v, dpp<kRowRor8>(v));
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    v = fmaxf(v, __shfl_xor(v, 32, 64));
    return v;
}

template <int PARTS>
__device__ __forceinline__ float sum_slots(float v) {
#pragma unroll
    for (int s = PARTS; s < 64; s <<= 1) v += __shfl_xor(v, s, 64);
    return v;
}

// 2^x on the transcendental unit (x <= 0 here; tiny results may flush to 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte streaming load: the cache rows are read once per step, so the
// loads are marked nontemporal (they do not displace other data in the
// caches), which streams measurably faster than plain loads on MI355X.
__device__ __forceinline__ uint4 stream_load16(const uint8_t *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// D = head_dim (64 or 128); CH = token iterations per chunk (even): 6 for
// runs of at least 256 tokens per wave (more bytes in flight per wave), 4
// for shorter ones (a deep chunk would mostly load masked positions).  Both
// run at two waves per SIMD: at three the 4-iteration variant spilled 8 to 11
// registers to scratch and was 4-15% slower.
// WPI = waves per work item: 1 (four items per workgroup) or 4 (one item per
// workgroup, its chunks dealt to the waves round-robin).
template <int D, int CH, int WPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void attn_split_kernel(
    const uint8_t *__restrict__ kc, const uint32_t *__restrict__ km, const uint8_t *__restrict__ vc,
    const uint32_t *__restrict__ vm, const uint16_t *__restrict__ q, int64_t ld_q, int H, int cap, int L, int n_split,
    int tok_per_split, int total_items, float sl2, float *__restrict__ ws, void *__restrict__ out,
    int out_f16) {
    constexpr int PARTS = D / 32;   // lanes per token row
    constexpr int TPI = 64 / PARTS; // tokens per wave iteration
    constexpr int G = D / 64;       // groups per token row
    constexpr int EPL = 32 / TPI;   // output elements per lane in the final reduction
    static_assert(CH % 2 == 0, "P.V pairs token iteration it with it + CH/2");
    static_assert(WPI == 1 || WPI == 4, "one item per wave or per workgroup");
    __shared__ float red[4][64 * 33];
    __shared__ float mrg_o[WPI][D];         // WPI > 1: the waves' partial states
    __shared__ float mrg_m[WPI], mrg_l[WPI];

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int item = WPI > 1 ? (int)blockIdx.x : (int)blockIdx.x * 4 + wv;
    const int sub = WPI > 1 ? wv : 0;       // this wave's share of the item
    // wave-uniform; with one item per workgroup the grid is exactly the items
    if (WPI == 1 && item >= total_items) return;

    const int split = item % n_split;
    const int bh = item / n_split;
    const int b = bh / H, hh = bh - b * H;
    const int j0 = split * tok_per_split;
    const int j1 = min(L, j0 + tok_per_split);
    const int slot = lane / PARTS, part = lane % PARTS, grp = part >> 1;

    // ---- query: 32 fp16 values of this lane's part, arranged as dot2 pairs
    const uint4 *qp = reinterpret_cast<const uint4 *>(q + (size_t)b * ld_q + (size_t)hh * D + part * 32);
    uint32_t qw[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 t = qp[i];
        qw[4 * i + 0] = t.x; qw[4 * i + 1] = t.y; qw[4 * i + 2] = t.z; qw[4 * i + 3] = t.w;
    }
    // element 8i + j sits in qw[4i + j/2], half j%2.  Pairs for code word i:
    //   QP[i][0] = (q_{8i+0}, q_{8i+4}), QP[i][1] = (q_{8i+1}, q_{8i+5}),
    //   QP[i][2] = (q_{8i+2}, q_{8i+6}), QP[i][3] = (q_{8i+3}, q_{8i+7}).
    uint32_t QP[4][4];
    float qsum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t a = qw[4 * i + 0], bq = qw[4 * i + 1], c = qw[4 * i + 2], d = qw[4 * i + 3];
        QP[i][0] = __builtin_amdgcn_perm(c, a, 0x05040100u);   // (a.lo, c.lo)
        QP[i][1] = __builtin_amdgcn_perm(c, a, 0x07060302u);   // (a.hi, c.hi)
        QP[i][2] = __builtin_amdgcn_perm(d, bq, 0x05040100u);  // (b.lo, d.lo)
        QP[i][3] = __builtin_amdgcn_perm(d, bq, 0x07060302u);  // (b.hi, d.hi)
#pragma unroll
        for (int h2 = 0; h2 < 4; ++h2) {
            const f16x2 v = as_f16x2(qw[4 * i + h2]);
            qsum += (float)v.x + (float)v.y;
        }
    }

    const size_t rowbase = (size_t)bh * cap;
    const uint8_t *kbase = kc + rowbase * (D / 2) + part * 16;
    const uint8_t *vbase = vc + rowbase * (D / 2) + part * 16;
    const uint32_t *kmb = km + rowbase * G + grp;
    const uint32_t *vmb = vm + rowbase * G + grp;

    float m_run = -INFINITY, l_acc = 0.f, macc = 0.f;
    float o[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) o[e] = 0.f;

    struct Chunk {
        uint4 K[CH], V[CH];
        uint32_t KM[CH], VM[CH];
    };
    // Loads of one chunk of CH*TPI tokens (positions past j1 re-read the
    // last valid row; their probabilities are zero).
    auto load = [&](int c0, Chunk &d) {
#pragma unroll
        for (int it = 0; it < CH; ++it) {
            const int j = c0 + it * TPI + slot;
            const size_t jc = (size_t)(j < j1 ? j : j1 - 1);
            d.K[it] = stream_load16(kbase + jc * (D / 2));
            d.KM[it] = __builtin_nontemporal_load(kmb + jc * G);
            d.V[it] = stream_load16(vbase + jc * (D / 2));
            d.VM[it] = __builtin_nontemporal_load(vmb + jc * G);
        }
    };
    // TAIL: the chunk may reach past the end of the split (the last one).
    auto process = [&](int c0, const Chunk &d, auto tail) {
        constexpr bool TAIL = decltype(tail)::value;
        // ---- scores.  A token iteration wholly past the end of the split
        // (the ragged last chunk) skips its arithmetic: its score is -inf
        // (the test is the same in every lane).
        float s[CH];
#pragma unroll
        for (int it = 0; it < CH; ++it) {
            if (TAIL && c0 + it * TPI >= j1) {
                s[it] = -INFINITY;
                continue;
            }
            const uint32_t w[4] = {d.K[it].x, d.K[it].y, d.K[it].z, d.K[it].w};
            float lo = 0.f, hi = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t w8 = w[i] >> 8;
                lo = dot2(w[i] & 0x000F000Fu, QP[i][0], lo);
                hi = dot2(w[i] & 0x00F000F0u, QP[i][1], hi);
                lo = dot2(w8 & 0x000F000Fu, QP[i][2], lo);
                hi = dot2(w8 & 0x00F000F0u, QP[i][3], hi);
            }
            const float sc = lo * 16777216.0f + hi * 1048576.0f;   // sum_d q_d c_d
            const float step = h2f((uint16_t)(d.KM[it] >> 16));
            const float mn = h2f((uint16_t)(d.KM[it] & 0xffffu));
            const float part_s = step * sc + mn * qsum;
            const float tot = sum_parts<PARTS>(part_s);
            s[it] = (c0 + it * TPI + slot < j1) ? tot * sl2 : -INFINITY;
        }
        float cm = s[0];
#pragma unroll
        for (int it = 1; it < CH; ++it) cm = fmaxf(cm, s[it]);
        cm = max_slots<PARTS>(cm);
        // the running max only moves now and then: rescale only when it does
        // (m_run and cm are the same in every lane, so the branch is uniform)
        if (cm > m_run) {
            const float corr = fast_exp2(m_run - cm);
            m_run = cm;
            l_acc *= corr;
            macc *= corr;
#pragma unroll
            for (int e = 0; e < 32; ++e) o[e] *= corr;
        }
        const float m_new = m_run;

        // ---- P.V, two tokens (it, it + CH/2) per dot2; a pair wholly past
        // the end adds nothing and is skipped (a pair with one token past the
        // end runs with p = 0 for it: its loads re-read the last valid row,
        // so every value is finite)
#pragma unroll
        for (int pi = 0; pi < CH / 2; ++pi) {
            const int ia = pi, ib = pi + CH / 2;
            if (TAIL && c0 + ia * TPI >= j1) continue;
            const float pa = fast_exp2(s[ia] - m_new), pb = fast_exp2(s[ib] - m_new);
            l_acc += pa + pb;
            const float sa = h2f((uint16_t)(d.VM[ia] >> 16)), sb = h2f((uint16_t)(d.VM[ib] >> 16));
            macc += pa * h2f((uint16_t)(d.VM[ia] & 0xffffu)) + pb * h2f((uint16_t)(d.VM[ib] & 0xffffu));
            const float wa = pa * sa, wb = pb * sb;
            const _Float16 wa_h = (_Float16)wa, wb_h = (_Float16)wb;
            const _Float16 wa_l = (_Float16)(wa - (float)wa_h), wb_l = (_Float16)(wb - (float)wb_h);
            f16x2 whi, wlo;
            whi.x = wa_h; whi.y = wb_h;
            wlo.x = wa_l; wlo.y = wb_l;
            const uint32_t WH = as_u32(whi), WL = as_u32(wlo);
            const uint32_t A[4] = {d.V[ia].x, d.V[ia].y, d.V[ia].z, d.V[ia].w};
            const uint32_t Bv[4] = {d.V[ib].x, d.V[ib].y, d.V[ib].z, d.V[ib].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // X = [A.b0, A.b1, B.b0, B.b1], Y = [A.b2, A.b3, B.b2, B.b3]
                const uint32_t X = __builtin_amdgcn_perm(Bv[i], A[i], 0x05040100u);
                const uint32_t Y = __builtin_amdgcn_perm(Bv[i], A[i], 0x07060302u);
                const uint32_t X8 = X >> 8, Y8 = Y >> 8;
                const uint32_t pr[8] = {X & 0x000F000Fu, X & 0x00F000F0u, X8 & 0x000F000Fu, X8 & 0x00F000F0u,
                                        Y & 0x000F000Fu, Y & 0x00F000F0u, Y8 & 0x000F000Fu, Y8 & 0x00F000F0u};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    o[8 * i + e] = dot2(pr[e], WH, o[8 * i + e]);
                    o[8 * i + e] = dot2(pr[e], WL, o[8 * i + e]);
                }
            }
        }
    };

    // Two register buffers: the loads of the wave's next chunk are in flight
    // while the current one is processed.  A chunk with a next one is whole
    // (body); the wave's last chunk may reach past the end (tail).
    constexpr int STEP = CH * TPI;
    constexpr int STRIDE = WPI * STEP;   // the waves of an item take every WPI-th chunk
    Chunk bufA, bufB;
    int c0 = j0 + sub * STEP;
    if (c0 < j1) load(c0, bufA);
    const std::true_type tail;
    const std::false_type body;
    while (c0 < j1) {
        if (c0 + STRIDE < j1) {
            load(c0 + STRIDE, bufB);
            process(c0, bufA, body);
        } else {
            process(c0, bufA, tail);
        }
        c0 += STRIDE;
        if (c0 >= j1) break;
        if (c0 + STRIDE < j1) {
            load(c0 + STRIDE, bufA);
            process(c0, bufB, body);
        } else {
            process(c0, bufB, tail);
        }
        c0 += STRIDE;
    }

    // ---- reduce the token slots: o (per element) through LDS, l and macc by shuffles
    float *r = red[wv];
#pragma unroll
    for (int e = 0; e < 32; ++e) r[lane * 33 + e] = o[e];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const float l_tot = sum_slots<PARTS>(l_acc);
    const float m_tot = sum_slots<PARTS>(macc);
    float val[EPL];
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
        const int e = slot * EPL + k;
        float acc = 0.f;
        for (int s2 = 0; s2 < TPI; ++s2) acc += r[(s2 * PARTS + part) * 33 + e];
        val[k] = acc * ((e & 1) ? 1048576.0f : 16777216.0f) + m_tot;
    }
    const int d0 = part * 32 + slot * EPL;
    float m_out = m_run, l_out = l_tot;
    if constexpr (WPI > 1) {
        // merge the waves' states in wave order: m = max m_w, each wave's o
        // and l scaled by 2^(m_w - m); a wave that took no chunk has
        // m_w = -inf and o = l = 0, and adds nothing
#pragma unroll
        for (int k = 0; k < EPL; ++k) mrg_o[sub][d0 + k] = val[k];
        if (lane == 0) {
            mrg_m[sub] = m_run;
            mrg_l[sub] = l_tot;
        }
        __syncthreads();
        float mx = mrg_m[0];
#pragma unroll
        for (int w = 1; w < WPI; ++w) mx = fmaxf(mx, mrg_m[w]);
        float fw[WPI];
        l_out = 0.f;
#pragma unroll
        for (int w = 0; w < WPI; ++w) {
            fw[w] = mrg_m[w] == -INFINITY ? 0.f : fast_exp2(mrg_m[w] - mx);
            l_out += fw[w] * mrg_l[w];
        }
#pragma unroll
        for (int k = 0; k < EPL; ++k) {
            float acc = 0.f;
#pragma unroll
            for (int w = 0; w < WPI; ++w) acc += fw[w] * mrg_o[w][d0 + k];
            val[k] = acc;
        }
        m_out = mx;
        if (sub != 0) return;   // wave 0 writes the item's result
    }
    if (n_split == 1) {
        const float inv = 1.0f / l_out;
        const size_t ob = ((size_t)b * H + hh) * D + d0;
#pragma unroll
        for (int k = 0; k < EPL; ++k) {
            if (out_f16)
                static_cast<_Float16 *>(out)[ob + k] = (_Float16)(val[k] * inv);
            else   // written once, read by a later launch: keep it out of L2
                __builtin_nontemporal_store(val[k] * inv, static_cast<float *>(out) + ob + k);
        }
    } else {
        float *wrow = ws + ((size_t)bh * n_split + split) * (D + 4);
#pragma unroll
        for (int k = 0; k < EPL; ++k) wrow[d0 + k] = val[k];
        if (lane == 0) {
            wrow[D] = m_out;
            wrow[D + 1] = l_out;
        }
    }
}

// Merge the n_split partial states of each (b, h): one block of D threads.
template <int D>
__global__ __launch_bounds__(128) void attn_merge_kernel(const float *__restrict__ ws, int n_split,
                                                         void *__restrict__ out, int out_f16) {
    const int bh = blockIdx.x;
    const int d = threadIdx.x;
    const float *base = ws + (size_t)bh * n_split * (D + 4);
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
        static_cast<_Float16 *>(out)[(size_t)bh * D + d] = (_Float16)v;
    else
        __builtin_nontemporal_store(v, static_cast<float *>(out) + (size_t)bh * D + d);
}

// Token iterations per chunk: long chunks (two waves per SIMD, more bytes in
// flight per wave) once a wave streams a few hundred tokens, the middle
// setting (three waves per SIMD) for short ranges, where a long chunk would
// mostly load masked positions past the end.
constexpr int kChunkShort = 4, kChunkLong = 6;
constexpr int kLongChunkTokens = 256;   // tokens per wave from which the long chunk is used
// Sequences from this length take four waves per item when the pairs alone
// would not give ~8 waves per SIMD.  Each wave then streams >= 256 tokens (a
// split is never shorter than 4 x 256 tokens), so these items always take
// the long chunk.  Measured: 32 sequences x 96 heads x 4100 positions
// 290 -> 277 us (no split and no merge launch instead of 3 splits),
// 16 x 32 x 16416 203 -> 193 us, 96 x 56 x 1040 138 -> 125 us (a finer last
// round of waves); at 530 positions (2048 pairs) the quarter runs were
// slower (32 -> 34 us).
constexpr int kQuadWaveMinTokens = 1024;

}  // namespace

struct AttnPlan {
    int n_split;
    int tok_per_split;
    int chunk_iters;
    int wpi;    // waves per work item: 1 or 4
};

AttnPlan attn_plan(int32_t batch, int32_t heads, int32_t head_dim, int32_t kv_len) {
    const int tpi = 64 / (head_dim / 32);
    const int64_t target_waves = 8LL * 4 * kNumCU;     // ~8 waves per SIMD in flight
    const int64_t slots = 2LL * 4 * kNumCU;            // one wave per slot at two waves per SIMD
    const int64_t pairs = (int64_t)batch * heads;
    const int wpi = (pairs < target_waves && kv_len >= kQuadWaveMinTokens) ? 4 : 1;
    const int64_t bh = pairs * wpi;                    // waves per split
    int n_split = 1;
    if (bh > 0 && bh < target_waves) {
        n_split = (int)((target_waves + bh - 1) / bh);
        // Once the waves alone occupy every wave slot, a split pays only if each
        // wave still streams a long run (it adds a merge and a wave's setup);
        // with fewer waves than slots, shorter runs are worth the occupancy.
        const int min_tok = (bh >= slots ? 768 : 256) * wpi;
        const int max_split = kv_len / min_tok > 1 ? kv_len / min_tok : 1;
        if (n_split > max_split) n_split = max_split;
    }
    int per = (kv_len + n_split - 1) / n_split;
    const int ch = per / wpi >= kLongChunkTokens ? kChunkLong : kChunkShort;   // wpi 4: always long
    const int chunk = ch * tpi;
    per = ((per + chunk - 1) / chunk) * chunk;
    n_split = (kv_len + per - 1) / per;   // drop empty splits
    return {n_split, per, ch, wpi};
}

// Scratch of the allocation-free entry point: a file-scope device array, one
// copy per GPU the library runs on, held until the process ends.  It holds
// the per-split softmax states, which the split kernel writes in full before
// the merge kernel reads them, so it needs no clearing between calls.  The
// split plan keeps batch * heads * splits below 2 * 8192 (a split count is
// only chosen when batch * heads < 8192 and is then at most
// ceil(8192 / (batch * heads))), so at most 16383 rows of (head_dim + 4)
// floats: 8,650,224 bytes at head_dim 128.
constexpr size_t kAttnScratchBytes = (size_t)9 << 20;
static __device__ __align__(256) uint8_t scratch[kAttnScratchBytes];
constexpr int kMaxDevices = 64;

size_t attn_scratch_bytes() { return kAttnScratchBytes; }

// Device address of `scratch` on the current device.  In host code the
// array's name is only a stand-in for the symbol, so its address is looked
// up once per device (with that device current) and kept.
fgq_status attn_scratch_ptr(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FGQ_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(FGQ_ERR_DEVICE, "device %d beyond %d", dev, kMaxDevices);
    static std::mutex mu;
    static void *addr[kMaxDevices];
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(FGQ_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return FGQ_OK;
}

size_t attn_ws_bytes(int32_t batch, int32_t heads, int32_t head_dim, int32_t kv_len) {
    const AttnPlan p = attn_plan(batch, heads, head_dim, kv_len);
    if (p.n_split <= 1) return 0;
    return (size_t)batch * heads * p.n_split * (head_dim + 4) * sizeof(float);
}

fgq_status launch_decode_attn(const fgq_kv_cache *kv, const void *q, int64_t ld_q, int32_t kv_len, float scale,
                              void *out, int32_t out_dtype, void *ws, hipStream_t stream) {
    if (kv->batch == 0 || kv->heads == 0) return FGQ_OK;
    const AttnPlan p = attn_plan(kv->batch, kv->heads, kv->head_dim, kv_len);
    const int64_t total64 = (int64_t)kv->batch * kv->heads * p.n_split;
    if (total64 > INT32_MAX - 3)
        return fail(FGQ_ERR_SHAPE, "batch * heads * splits = %lld work items exceeds 2^31", (long long)total64);
    const int total = (int)total64;
    const float sl2 = scale * kLog2e;
    const int f16 = out_dtype == FGQ_DTYPE_F16;
    const dim3 grid((unsigned)(p.wpi > 1 ? total : (total + 3) / 4)), block(256);
#define FGQ_ATTN_LAUNCH_W(D, CH, WPI)                                                                          \
    attn_split_kernel<D, CH, WPI><<<grid, block, 0, stream>>>(kv->k_codes, kv->k_meta, kv->v_codes, kv->v_meta,      \
                                                         static_cast<const uint16_t *>(q), ld_q, kv->heads, kv->capacity, \
                                                         kv_len, p.n_split, p.tok_per_split, total, sl2,        \
                                                         static_cast<float *>(ws), out, f16)
    // Four waves per item only come with splits of >= 4 x 256 tokens, so
    // always with the long chunk.
    if (kv->head_dim == 128) {
        if (p.wpi > 1) FGQ_ATTN_LAUNCH_W(128, kChunkLong, 4);
        else if (p.chunk_iters == kChunkLong) FGQ_ATTN_LAUNCH_W(128, kChunkLong, 1);
        else FGQ_ATTN_LAUNCH_W(128, kChunkShort, 1);
    } else {
        if (p.wpi > 1) FGQ_ATTN_LAUNCH_W(64, kChunkLong, 4);
        else if (p.chunk_iters == kChunkLong) FGQ_ATTN_LAUNCH_W(64, kChunkLong, 1);
        else FGQ_ATTN_LAUNCH_W(64, kChunkShort, 1);
    }
#undef FGQ_ATTN_LAUNCH_W
    fgq_status s = check_launch("attn_split_kernel");
    if (s != FGQ_OK || p.n_split == 1) return s;
    const dim3 mgrid((unsigned)(kv->batch * kv->heads));
    if (kv->head_dim == 128)
        attn_merge_kernel<128><<<mgrid, dim3(128), 0, stream>>>(static_cast<const float *>(ws), p.n_split, out, f16);
    else
        attn_merge_kernel<64><<<mgrid, dim3(64), 0, stream>>>(static_cast<const float *>(ws), p.n_split, out, f16);
    return check_launch("attn_merge_kernel");
}

}  // namespace fgq
