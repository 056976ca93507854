// Prefill attention over the prompt's fp16 q, k, v (before the prompt's K
// and V are compressed into the cache by one bulk append).
//
// What is computed: the prefill step runs every prompt token at once and
// leaves each layer's KV cache behind (paper-graph-ui FlexGen summary,
// section 3.4, token 0 of the Figure-2 grid; FlexGen review on
// blog.gzher.com, section 1).  For a decoder-only model each token attends to
// itself and the tokens before it: per (sequence b, head h, token i)
//   o_i = sum_{j<=i} softmax_j(scale * q_i . k_j) v_j
// with q, k, v, o token-major [batch][seq][heads*head_dim].
//
// Design (MFMA-bound: 4*D flops per (i, j) pair, ~2 bytes per pair of HBM):
//  * a wave takes 32 query rows of one (b, h) (two 16-row MFMA tiles, so
//    every K and V fragment read from LDS feeds two MFMAs); a workgroup of 8
//    waves (256 rows, two waves per SIMD) for short prompts, of 12 waves
//    (384 rows, three per SIMD) for long ones, where the Q fragments move
//    from registers to LDS to make room for the third wave; and of 4 waves
//    (128 rows, two workgroups per CU) for prompts up to 640 tokens whose
//    256-row blocks would leave more rows empty, or that are multiples of 256,
//    where the shorter causal blocks also even out the waves' work;
//    key blocks of 64 reach LDS through gfx950's direct global->LDS loads
//    (no registers, no LDS write instructions), dealt to all the waves, into
//    two buffers: block kb + 1 lands in one while block kb is multiplied
//    from the other, with one barrier per block; K and V sit row-major and
//    unpadded, their 16-byte chunks XOR-swizzled per row;
//  * scores are formed transposed, S^T = K Q^T, on v_mfma_f32_16x16x32_f16
//    (A = K rows from LDS, B = the wave's Q fragments), so
//    a lane's accumulators all belong to one query: the running max, the
//    rescale of the output and the exponentials stay in the lane, with two
//    cross-lane steps for the row max; the row sums of P come from the matrix
//    cores too (an all-ones A operand times the same P^T fragments);
//  * P.V is formed transposed too, O^T = V^T P^T, with P^T taken straight
//    from the score accumulators: the 32 k-slots of an MFMA are mapped to
//    keys in the order the accumulators hold them, and the V^T fragments
//    come from the row-major V tile through two transposing 8-byte LDS
//    reads each (ds_read_b64_tr_b16);
//  * online softmax in the log2 domain (exp2 on the transcendental unit);
//    the output is rescaled only when some lane's running max moved; blocks
//    wholly above a wave's diagonal are skipped, blocks that reach it mask
//    j > i;
//  * the causal row blocks differ in length, so the workgroups are numbered
//    to dispatch the last (longest) row block of every (b, h) first, and the
//    short ones fill the tail of the launch.
#include <type_traits>

#include "common.h"

namespace fgq {
namespace {

constexpr float kPfLog2e = 1.4426950408889634f;
constexpr int kPfWaveRows = 32;              // query rows per wave (two 16-row MFMA tiles)
constexpr int kPfQRegWaves = 8;              // up to this many waves per workgroup keep Q in registers
constexpr int kPfLongPrompt = 1024;          // prompts from which 12-wave workgroups are used
constexpr int kPfNarrowMax = 640;            // longest prompt that may take 4-wave workgroups
constexpr int kPfKeys = 64;   // keys per block
constexpr float kPfSlack = 8.0f;   // log2-domain headroom of the lazy rescale

// LDS tiles are unpadded row-major [rows][D] with the 16-byte chunks of a
// row XOR-swizzled (CH = D / 8 chunks per row).  Q and K: chunk ch of row r
// sits at chunk position ch ^ (r % CH), so the 16-byte fragment reads of 16
// consecutive rows (one chunk each) hit 16 distinct positions.  V: at
// ch ^ pf_vsw(r), so the transposing reads of half a wave (8 consecutive
// rows, two adjacent chunks each) hit distinct banks: with 256-byte rows
// (D = 128) an even offset 2r per row; with 128-byte rows (two rows per
// bank cycle) 2 * (r / 2).
template <int D>
__device__ __forceinline__ int pf_pos(int row, int ch) {
    return ch ^ (row & (D / 8 - 1));
}
template <int D>
__device__ __forceinline__ int pf_vsw(int row) {
    return (D == 128 ? 2 * row : 2 * (row >> 1)) & (D / 8 - 1);
}
template <int D>
__device__ __forceinline__ int pf_vpos(int row, int ch) {
    return ch ^ pf_vsw<D>(row);
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t pf_lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Direct global->LDS load of 16 bytes per lane (gfx950's
// global_load_lds_dwordx4): lane i's bytes land at LDS address lds + 16 i
// (lds wave-uniform, passed in M0).  Written as inline assembly so the
// compiler does not count it as an LDS store; the kernel waits for it with
// an explicit vmcnt before the barrier that publishes the tile.  M0 is used
// by nothing else in this kernel.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void pf_dma16(const void *gptr, uint32_t lds) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(m0v) : "memory", "m0");
}
#pragma clang diagnostic pop

// Every load of this wave's loads has landed (vmcnt 0).
__device__ __forceinline__ void pf_wait_loads() {
    // simm16: vmcnt[3:0] = 0 | expcnt[6:4] = 7 | lgkmcnt[11:8] = 15 | vmcnt[5:4] = 0
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
}

// Issue the direct-to-LDS loads of key block kb (K and V, 64 rows each,
// rows past the prompt clamped to its last token): load instruction i fills
// bytes [1024 i, 1024 i + 1024) of a tile, i.e. rows RPI*i .. RPI*i + RPI-1,
// lane L taking row RPI*i + L / CH at chunk position L % CH, so it reads the
// chunk that the tile's swizzle puts there.  Instructions are dealt to the
// waves round-robin.
template <int D, int NW>
__device__ __forceinline__ void pf_issue_tile(const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
                                              size_t base, size_t rs, int S, int kb, int wv, int lane,
                                              uint16_t *kt, uint16_t *vt) {
    constexpr int CH = D / 8;               // 16-byte chunks per row
    constexpr int RPI = 64 / CH;            // rows per load instruction
    constexpr int NI = kPfKeys / RPI;       // load instructions per tile
    const int rl = lane / CH, pl = lane % CH;
#pragma unroll
    for (int i0 = 0; i0 < NI; i0 += NW) {
        const int i = i0 + wv;
        if (NI % NW != 0 && i >= NI) break;
        const int row = RPI * i + rl;
        int j = kb * kPfKeys + row;
        j = j < S ? j : S - 1;
        const size_t rowoff = base + (size_t)j * rs;
        pf_dma16(k + rowoff + 8 * pf_pos<D>(row, pl), pf_lds_addr(kt) + 1024 * i);
        pf_dma16(v + rowoff + 8 * pf_vpos<D>(row, pl), pf_lds_addr(vt) + 1024 * i);
    }
}

// gfx950's transposing LDS read (ds_read_b64_tr_b16).  In each group of 16
// lanes, lane j receives element j % 4 of the 8-byte pieces that lanes
// 4e + j / 4 (e = 0..3) address, as its elements e = 0..3.  With lane
// 16g + s addressing the four halves (row r0 + s / 4, columns c0 + 4 (s % 4)
// .. + 3) of a row-major tile, lane 16g + j gets column c0 + j of rows
// r0 .. r0 + 3.
typedef short pf_v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 pf_read_tr16(const uint16_t *p) {
    const pf_v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) pf_v4s *)(const __attribute__((address_space(3))) void *)p);
    return __builtin_bit_cast(uint2, r);
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW > kPfQRegWaves ? 3 : 2))) void prefill_attn_kernel(const uint16_t *__restrict__ q,
                                                           const uint16_t *__restrict__ k,
                                                           const uint16_t *__restrict__ v, int S, int H,
                                                           float sl2, void *__restrict__ out, int out_f16) {
    constexpr int KSTEP = D / 32;        // MFMA k-steps over d
    constexpr int NDT = D / 16;          // output d-tiles
    constexpr int QT = kPfWaveRows / 16; // query tiles per wave
    constexpr int NTH = 64 * NW;         // threads
    constexpr int ROWS = NW * kPfWaveRows;   // query rows per workgroup
    // Above 8 waves the Q fragments live in LDS (read per k-step) instead of
    // registers, which brings a wave under 168 VGPRs: three waves per SIMD
    constexpr bool QLDS = NW > kPfQRegWaves;
    // Q rows (QLDS), and two K and two V tiles: key block kb is multiplied
    // from buffer kb % 2 while block kb + 1 loads into the other; all
    // unpadded with swizzled chunks (pf_pos for Q and K, pf_vpos for V)
    __shared__ __attribute__((aligned(1024))) uint16_t ktile[2][kPfKeys * D];
    __shared__ __attribute__((aligned(1024))) uint16_t vtile[2][kPfKeys * D];
    __shared__ __attribute__((aligned(16))) uint16_t qs[QLDS ? ROWS * D : 8];

    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;
    // Longest rows first across the whole launch: the workgroups are taken in
    // dispatch order (x fastest), and that order visits the last row block of
    // every (sequence, head) before any earlier one, so the short causal
    // blocks fill the tail.  nqb * heads * batch < 2^31 (checked by the entry).
    const int nqb = gridDim.x, nbh = gridDim.y * gridDim.z;
    const int lin = (int)blockIdx.x + nqb * ((int)blockIdx.y + (int)gridDim.y * (int)blockIdx.z);
    const int qb = nqb - 1 - lin / nbh;
    const int bh = lin - (lin / nbh) * nbh;
    const int h = bh % (int)gridDim.y, b = bh / (int)gridDim.y;
    const size_t rs = (size_t)H * D;               // token stride in halves
    const size_t base = (size_t)b * S * rs + (size_t)h * D;

    // ---- the wave's Q fragments (B operands): query tile n holds query
    // q0 + 16n + c, d = 32*s + 8*g + 0..7 (rows past the prompt clamped)
    const int q0 = qb * ROWS + wv * kPfWaveRows;
    int qi[QT];
    f16x8 qf[QLDS ? 1 : QT][KSTEP];
#pragma unroll
    for (int n = 0; n < QT; ++n) qi[n] = q0 + 16 * n + c;
    if constexpr (QLDS) {
        constexpr int QCH = D / 8;
        for (int idx = tid; idx < ROWS * QCH; idx += NTH) {
            const int row = idx / QCH, ch = idx % QCH;
            int qr = qb * ROWS + row;
            qr = qr < S ? qr : S - 1;
            *reinterpret_cast<u32x4 *>(qs + row * D + 8 * pf_pos<D>(row, ch)) =
                *reinterpret_cast<const u32x4 *>(q + base + (size_t)qr * rs + 8 * ch);
        }
    } else {
#pragma unroll
        for (int n = 0; n < QT; ++n) {
            const int qic = qi[n] < S ? qi[n] : S - 1;
#pragma unroll
            for (int s = 0; s < KSTEP; ++s)
                qf[n][s] = *reinterpret_cast<const f16x8 *>(q + base + (size_t)qic * rs + 32 * s + 8 * g);
        }
    }
    const int qrow = wv * kPfWaveRows + c;      // this lane's first Q row in LDS (QLDS)
    f32x4 o[NDT][QT];
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
        for (int n = 0; n < QT; ++n) o[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[QT];
    // Row sums of P on the matrix cores: an all-ones A operand times the same
    // P^T fragments as P.V, so every row of lsum[n] holds the sum over keys of
    // query tile n's column (the fp16 probabilities that P.V also uses).
    f32x4 lsum[QT];
    const f16x8 ones = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f,
                        (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int n = 0; n < QT; ++n) {
        m_run[n] = -INFINITY;
        lsum[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // key blocks holding a key <= the workgroup's last query (and < S)
    const int q_last = min(qb * ROWS + ROWS, S) - 1;
    const int kb_last = q_last / kPfKeys;
    // a wave whose rows all lie past the prompt multiplies nothing (it still
    // issues its share of every tile's loads and meets every barrier)
    const int wave_q_last = q0 < S ? q0 + kPfWaveRows - 1 : -1;
    pf_issue_tile<D, NW>(k, v, base, rs, S, 0, wv, lane, ktile[0], vtile[0]);
    // One key block; BUF = kb % 2 is a compile-time constant (the loop below
    // takes blocks in pairs), so every LDS fragment address is a per-lane
    // base fixed for the whole kernel plus an immediate offset.
    auto key_block = [&](const int kb, auto bufc) {
        constexpr int BUF = decltype(bufc)::value;
        // block kb has landed (this wave's loads, then every wave's), and
        // every wave is done with block kb - 1, whose buffer block kb + 1
        // now fills while block kb is multiplied
        pf_wait_loads();
        __syncthreads();
        if (kb < kb_last) pf_issue_tile<D, NW>(k, v, base, rs, S, kb + 1, wv, lane, ktile[BUF ^ 1], vtile[BUF ^ 1]);
        if (kb * kPfKeys > wave_q_last) return;   // every key of the block is past this wave's queries
        const uint16_t *ks = ktile[BUF];
        const uint16_t *vs = vtile[BUF];

        // ---- S^T = K Q^T: st[t][n] holds keys 16t + 4g + r (r = 0..3) of query tile n
        f32x4 st[4][QT];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int n = 0; n < QT; ++n) st[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (QLDS) {
            // k-step outer: only one k-step of Q fragments is held at a time
#pragma unroll
            for (int s = 0; s < KSTEP; ++s) {
                f16x8 qs_s[QT];
#pragma unroll
                for (int n = 0; n < QT; ++n)
                    qs_s[n] = *reinterpret_cast<const f16x8 *>(qs + (qrow + 16 * n) * D + 8 * pf_pos<D>(qrow + 16 * n, 4 * s + g));
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const f16x8 a = *reinterpret_cast<const f16x8 *>(ks + (16 * t + c) * D + 8 * pf_pos<D>(16 * t + c, 4 * s + g));
#pragma unroll
                    for (int n = 0; n < QT; ++n)
                        st[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qs_s[n], st[t][n], 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int s = 0; s < KSTEP; ++s) {
                    const f16x8 a = *reinterpret_cast<const f16x8 *>(ks + (16 * t + c) * D + 8 * pf_pos<D>(16 * t + c, 4 * s + g));
#pragma unroll
                    for (int n = 0; n < QT; ++n)
                        st[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qf[QLDS ? 0 : n][s], st[t][n], 0, 0, 0);
                }
        }
        // ---- causal mask (only blocks that reach past the wave's first query
        // need it), running max on the raw scores (the scale is positive);
        // the output is rescaled only when some lane's max moved
        if ((kb + 1) * kPfKeys - 1 > q0) {
#pragma unroll
            for (int n = 0; n < QT; ++n)
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (kb * kPfKeys + 16 * t + 4 * g + r > qi[n]) st[t][n][r] = -INFINITY;
        }
        // Lazy rescale: the reference max m_run only moves when a row's block
        // max passes it by more than kPfSlack (log2 units), so most blocks skip
        // the rescale of the output.  Meanwhile p = 2^(s - m_run) <= 2^kPfSlack
        // = 256, well inside fp16 (P enters P.V as fp16; its relative
        // precision does not depend on the scale), and o / l is unchanged by
        // the choice of reference.
        float corr[QT], msc[QT];
        bool moved = false;
#pragma unroll
        for (int n = 0; n < QT; ++n) {
            float mb = -INFINITY;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                mb = fmaxf(mb, fmaxf(fmaxf(st[t][n][0], st[t][n][1]), fmaxf(st[t][n][2], st[t][n][3])));
            mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
            mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
            const bool up = mb * sl2 > m_run[n] * sl2 + kPfSlack;   // false while mb = -inf (masked rows)
            const float m_new = up ? mb : m_run[n];
            corr[n] = up ? __builtin_amdgcn_exp2f((m_run[n] - m_new) * sl2) : 1.0f;
            moved |= up;
            m_run[n] = m_new;
            msc[n] = m_new * sl2;
        }
        if (__ballot(moved)) {
#pragma unroll
            for (int n = 0; n < QT; ++n) lsum[n] *= corr[n];
#pragma unroll
            for (int t = 0; t < NDT; ++t)
#pragma unroll
                for (int n = 0; n < QT; ++n) o[t][n] *= corr[n];
        }
        // ---- P^T fragments, p = 2^(s*scale*log2e - m*scale*log2e): k-slot
        // (g, e) of k-step kk is key 32kk + 4g + e (e < 4) or 32kk + 16 + 4g +
        // e - 4 (e >= 4), as the accumulators hold them
        f16x8 pb[QT][2];
#pragma unroll
        for (int n = 0; n < QT; ++n)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(st[2 * kk + (e >> 2)][n][e & 3], sl2, -msc[n]));
                    pb[n][kk][e] = (_Float16)pv;
                }
        // ---- O^T += V^T P^T: row d = 16dt + c of V^T, keys in the same
        // k-slot order, read transposed from the row-major V tile: lane
        // (g, c) addresses key 32kk + 4g + c / 4 (and 16 keys on), columns
        // 16dt + 4 (c % 4) .. + 3, and receives column 16dt + c of keys
        // 32kk + 4g .. + 3 (and 32kk + 16 + 4g .. + 3)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int t = 0; t < NDT; ++t) {
                const int vr0 = 32 * kk + 4 * g + (c >> 2), vch = 2 * t + ((c >> 1) & 1), vsub = 4 * (c & 1);
                const uint2 lo = pf_read_tr16(vs + vr0 * D + 8 * pf_vpos<D>(vr0, vch) + vsub);
                const uint2 hi = pf_read_tr16(vs + (vr0 + 16) * D + 8 * pf_vpos<D>(vr0 + 16, vch) + vsub);
                const u32x4 a4 = {lo.x, lo.y, hi.x, hi.y};
                const f16x8 a = __builtin_bit_cast(f16x8, a4);
#pragma unroll
                for (int n = 0; n < QT; ++n)
                    o[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb[n][kk], o[t][n], 0, 0, 0);
            }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int n = 0; n < QT; ++n)
                lsum[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[n][kk], lsum[n], 0, 0, 0);
    };
    for (int kb = 0; kb <= kb_last; kb += 2) {
        key_block(kb, std::integral_constant<int, 0>{});
        if (kb + 1 > kb_last) break;
        key_block(kb + 1, std::integral_constant<int, 1>{});
    }

    // ---- normalise and store: lane holds d = 16dt + 4g + r of query qi[n]
#pragma unroll
    for (int n = 0; n < QT; ++n) {
        const float l = lsum[n][0];   // every row of the tile holds the column's sum
        if (qi[n] >= S) continue;
        const float inv = 1.0f / l;
        const size_t ob = base + (size_t)qi[n] * rs + 4 * g;
#pragma unroll
        for (int t = 0; t < NDT; ++t) {
            const f32x4 val = o[t][n] * inv;
            if (out_f16) {
                _Float16 *op = static_cast<_Float16 *>(out) + ob + 16 * t;
                op[0] = (_Float16)val[0]; op[1] = (_Float16)val[1]; op[2] = (_Float16)val[2]; op[3] = (_Float16)val[3];
            } else {
                *reinterpret_cast<f32x4 *>(static_cast<float *>(out) + ob + 16 * t) = val;
            }
        }
    }
}

}  // namespace

fgq_status launch_prefill_attn(const void *q, const void *k, const void *v, int32_t batch, int32_t seq,
                               int32_t heads, int32_t head_dim, float scale, void *out, int32_t out_dtype,
                               hipStream_t stream) {
    if (batch == 0 || seq == 0 || heads == 0) return FGQ_OK;
    const float sl2 = scale * kPfLog2e;
    const int f16 = out_dtype == FGQ_DTYPE_F16;
    const uint16_t *qh = static_cast<const uint16_t *>(q), *kh = static_cast<const uint16_t *>(k),
                   *vh = static_cast<const uint16_t *>(v);
    // 12-wave workgroups (384 rows, three waves per SIMD) once the prompt is
    // long enough that the last, partly filled block of rows costs little;
    // 8 waves (256 rows, two per SIMD) below, except that prompts up to
    // kPfNarrowMax tokens whose last 256-row block would be full or at most
    // half full take 4 waves (128 rows, two workgroups per CU): fewer empty
    // rows, or (multiples of 256) shorter causal blocks whose waves' work is
    // more even; from 768 tokens the doubled K/V tile loads cost more.
    const int tail = seq % 256;
    const int nw = seq >= kPfLongPrompt ? 12 : (seq <= kPfNarrowMax && tail <= 128) ? 4 : 8;
    const int rows = nw * kPfWaveRows;
    const dim3 grid((unsigned)((seq + rows - 1) / rows), (unsigned)heads, (unsigned)batch);
#define FGQ_PF_LAUNCH(D, NW) \
    prefill_attn_kernel<D, NW><<<grid, dim3(64 * NW), 0, stream>>>(qh, kh, vh, seq, heads, sl2, out, f16)
    if (head_dim == 128) {
        if (nw == 12) FGQ_PF_LAUNCH(128, 12); else if (nw == 8) FGQ_PF_LAUNCH(128, 8); else FGQ_PF_LAUNCH(128, 4);
    } else {
        if (nw == 12) FGQ_PF_LAUNCH(64, 12); else if (nw == 8) FGQ_PF_LAUNCH(64, 8); else FGQ_PF_LAUNCH(64, 4);
    }
#undef FGQ_PF_LAUNCH
    return check_launch("prefill_attn_kernel");
}

}  // namespace fgq
