// Dequantising weight GEMM of one block: Y[M][N] = X[M][K] * W^[K][N] with
// M = g*m rows (m GPU batches of g rows) sharing one read of the compressed
// weight (paper-graph-ui FlexGen summary, section 3.4 "Compute Schedule";
// FlexGen review on jaehun.me, "A block is the unit of weight reuse").
// W^ = fp16(min + q*step) is restored to FP16 before the multiply (FlexGen
// review on blog.gzher.com, section 3.4) and fed to the fp16 matrix cores
// (v_mfma_f32_16x16x32_f16) with fp32 accumulation.
//
// Tiling (gfx950, 64-wide waves):
//  * a wave owns one weight group column (64 output channels = 4 MFMA
//    n-tiles) and every row of its M block (up to 9 m-tiles = 144 rows), so
//    one dequantised B fragment feeds up to 9 MFMAs;
//  * a workgroup is 8 waves (512 output channels, two waves per SIMD) and
//    shares the X rows of each K chunk through LDS;
//  * every operand reaches LDS through gfx950's direct global->LDS loads
//    (global_load_lds_dwordx4) into a ring of 8 one-chunk slots (32 k each:
//    the X rows, each wave's packed code words and its group metadata), so 7
//    chunks are in flight while one is multiplied, with one barrier per chunk
//    and no register spent on prefetching;
//  * the packed weight layout puts the 8 k-values of one output channel in
//    one 32-bit word, in the nibble order that AND/OR with the fp16 magic
//    numbers 0x6400 (1024 + q) and 0x5400 (64 + q) turn into two values per
//    op; a packed subtract and a packed FMA give two fp16 W^ values, and the
//    next chunk is dequantised in the shadow of the current chunk's MFMAs;
//  * X rows sit in LDS with a 16-byte-slot XOR swizzle (slot ^ (row/4)%4),
//    so the 16 rows of an A fragment read hit distinct banks;
//  * K is split across workgroups when the N/512 workgroups cannot fill the
//    CUs; fp32 partial tiles are summed in split order by a second kernel.
#include <cmath>
#include <type_traits>

#include "common.h"

namespace fgq {
namespace {

constexpr int kWaves = 8;                  // waves (weight groups) per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kRing = 8;                   // LDS chunk slots: kRing-1 chunks in flight

// Direct global->LDS load of 16 bytes per lane: lane i's bytes land at
// lds_ptr + 16*i (lds_ptr must be the same in every lane).  Written as inline
// assembly so the compiler does not track it as an LDS store: it would
// otherwise drain every load in flight (s_waitcnt vmcnt(0)) before each LDS
// read of the ring, since it cannot prove that the slot being filled differs
// from the slots being read.  The kernel waits for exactly the chunks it
// needs with explicit vmcnt counts instead.  M0 (the LDS base of the load)
// is used by nothing else in this kernel.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void *gptr, const void *lds_ptr) {
    const uint32_t la = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds_ptr);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(la) : "memory", "m0");
}
#pragma clang diagnostic pop

// Barrier that does not wait for outstanding direct-to-LDS loads (each wave
// waits for exactly the chunks it needs with vmcnt before it).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // simm16: vmcnt[3:0] | expcnt[6:4]=7 | lgkmcnt[11:8]=15 | vmcnt[5:4] in [15:14]
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most `chunks` chunks of this wave's loads are outstanding;
// a wave issues `cnt` (2, 3 or 4) load instructions per chunk.
template <int CHUNKS>
__device__ __forceinline__ void wait_chunks(int cnt) {
    if (cnt == 2) wait_vmcnt<2 * CHUNKS>();
    else if (cnt == 3) wait_vmcnt<3 * CHUNKS>();
    else wait_vmcnt<4 * CHUNKS>();
}

template <int MT>
struct Cfg {
    static constexpr int XBYTES = MT * 1024;           // MT*16 rows x 64 bytes (one 32-k chunk)
    static constexpr int BBYTES = kWaves * 1024;       // packed codes, 1 KB per wave
    static constexpr int MBYTES = kWaves * 128;        // packed meta, 128 B per wave
    static constexpr int SLOT = XBYTES + BBYTES + MBYTES;
    static constexpr int LDS = kRing * SLOT;
};

template <int MT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void dq_gemm_kernel(const uint16_t *__restrict__ x, int M, int64_t K, int64_t N,
                    const uint32_t *__restrict__ pc, const uint32_t *__restrict__ pm, int chunks_per_split,
                    float *__restrict__ part, void *__restrict__ y, int y_f16, int ksplit) {
    using C = Cfg<MT>;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS];

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int64_t ng = N >> 6;
    const int64_t g = (int64_t)blockIdx.x * kWaves + wv;
    const bool gvalid = g < ng;
    const int64_t gl = gvalid ? g : ng - 1;      // clamped group for loads
    const int split = blockIdx.y;
    const int m0 = blockIdx.z * MT * 16;
    const int64_t nchunks = K >> 5;
    const int64_t c_begin = (int64_t)split * chunks_per_split;
    int64_t c_end = c_begin + chunks_per_split;
    if (c_end > nchunks) c_end = nchunks;

    // X blocks (16 rows x 64 B) of a chunk are spread over the waves:
    // block b is loaded by wave b % kWaves.
    const int nx = MT / kWaves + (wv < MT % kWaves ? 1 : 0);
    const int cnt = nx + 2;                      // load instructions per chunk for this wave

    f32x4 acc[MT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int arow = lane & 15, akq = lane >> 4;

    // Issue this wave's direct-to-LDS loads of chunk kc into ring slot `slot`.
    // Chunks past c_end (the tail of the ring) and rows past M are clamped to
    // valid addresses; those values are never used for a stored output.
    auto issue = [&](int64_t kc, int slot) {
        if (kc >= c_end) kc = c_end - 1;
        uint8_t *base = lds + slot * C::SLOT;
#pragma unroll
        for (int t = 0; t < (MT + kWaves - 1) / kWaves; ++t) {
            const int blk = t * kWaves + wv;
            if (blk < MT) {
                const int row = blk * 16 + (lane >> 2);
                const int c16 = (lane & 3) ^ ((row >> 2) & 3);     // swizzled source column
                const int grow = (m0 + row < M) ? m0 + row : M - 1;
                dma16(x + (int64_t)grow * K + kc * 32 + c16 * 8, base + blk * 1024);
            }
        }
        const int64_t tile = kc * ng + gl;
        dma16(pc + (tile * 64 + lane) * 4, base + C::XBYTES + wv * 1024);
        if (lane < 8) dma16(pm + tile * 32 + lane * 4, base + C::XBYTES + C::BBYTES + wv * 128);
    };

    // Packed codes + (step, min) pairs of one chunk -> B fragment j.
    auto dequant_j = [&](const uint4 cw, const uint4 ms, const uint4 mm, int j) -> f16x8 {
        const uint32_t W[4] = {cw.x, cw.y, cw.z, cw.w};
        const uint32_t w = W[j], w8 = w >> 8;
        const uint32_t p0 = (w & 0x000F000Fu) | 0x64006400u;    // 1024 + q (k0, k1)
        const uint32_t p1 = (w & 0x00F000F0u) | 0x54005400u;    // 64 + q   (k2, k3)
        const uint32_t p2 = (w8 & 0x000F000Fu) | 0x64006400u;   // 1024 + q (k4, k5)
        const uint32_t p3 = (w8 & 0x00F000F0u) | 0x54005400u;   // 64 + q   (k6, k7)
        const f16x2 c01 = as_f16x2(p0) - f16x2{(_Float16)1024.0f, (_Float16)1024.0f};
        const f16x2 c23 = as_f16x2(p1) - f16x2{(_Float16)64.0f, (_Float16)64.0f};
        const f16x2 c45 = as_f16x2(p2) - f16x2{(_Float16)1024.0f, (_Float16)1024.0f};
        const f16x2 c67 = as_f16x2(p3) - f16x2{(_Float16)64.0f, (_Float16)64.0f};
        const f16x2 w01 = __builtin_elementwise_fma(c01, as_f16x2(ms.x), as_f16x2(mm.x));
        const f16x2 w23 = __builtin_elementwise_fma(c23, as_f16x2(ms.y), as_f16x2(mm.y));
        const f16x2 w45 = __builtin_elementwise_fma(c45, as_f16x2(ms.z), as_f16x2(mm.z));
        const f16x2 w67 = __builtin_elementwise_fma(c67, as_f16x2(ms.w), as_f16x2(mm.w));
        return f16x8{w01.x, w01.y, w23.x, w23.y, w45.x, w45.y, w67.x, w67.y};
    };
    // B words of ring slot `slot` for this wave; keep == 0 turns them into a
    // zero weight (step 0, min 0), used for a chunk past the end of the split.
    auto load_b = [&](int slot, uint32_t keep, uint4 &cw, uint4 &ms, uint4 &mm) {
        const uint8_t *base = lds + slot * C::SLOT;
        cw = *reinterpret_cast<const uint4 *>(base + C::XBYTES + wv * 1024 + lane * 16);
        const uint8_t *mb = base + C::XBYTES + C::BBYTES + wv * 128 + akq * 32;
        ms = *reinterpret_cast<const uint4 *>(mb);
        mm = *reinterpret_cast<const uint4 *>(mb + 16);
        ms.x &= keep; ms.y &= keep; ms.z &= keep; ms.w &= keep;
        mm.x &= keep; mm.y &= keep; mm.z &= keep; mm.w &= keep;
    };
    auto a_frag = [&](int slot, int i) {
        const int row = i * 16 + arow;
        return *reinterpret_cast<const f16x8 *>(lds + slot * C::SLOT + row * 64 + ((akq ^ ((row >> 2) & 3)) * 16));
    };

    const int64_t nmine = c_end - c_begin;       // chunks of this split (>= 1 when the loop runs)
    f16x8 bcur[4], bnext[4];
    if (nmine > 0) {
#pragma unroll
        for (int r = 0; r < kRing - 1; ++r) issue(c_begin + r, r);
        wait_chunks<kRing - 2>(cnt);             // this wave's B words of the first chunk
        uint4 cw, ms, mm;
        load_b(0, 0xFFFFFFFFu, cw, ms, mm);
#pragma unroll
        for (int j = 0; j < 4; ++j) bcur[j] = dequant_j(cw, ms, mm, j);
    }
    for (int64_t it = 0; it < nmine; ++it) {
        const int slot = (int)(it % kRing);
        wait_chunks<kRing - 3>(cnt);             // chunks it and it+1 of this wave have landed
        lds_barrier();                           // ... for every wave; slot it-1 is free again
        issue(c_begin + it + kRing - 1, (int)((it + kRing - 1) % kRing));
        // MFMAs of chunk it, m-tile by m-tile; the A fragment of the next
        // m-tile is read first and, after the first m-tiles, one n-tile of the
        // next chunk's B fragments is dequantised; the scheduling fences keep
        // the VALU work and the LDS latency under the matrix-core time.
        uint4 cw, ms, mm;
        load_b((int)((it + 1) % kRing), it + 1 < nmine ? 0xFFFFFFFFu : 0u, cw, ms, mm);
        f16x8 a_cur = a_frag(slot, 0);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            f16x8 a_nxt;
            if (i + 1 < MT) a_nxt = a_frag(slot, i + 1);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_cur, bcur[j], acc[i][j], 0, 0, 0);
            if (MT >= 4) {
                if (i < 4) bnext[i] = dequant_j(cw, ms, mm, i);
            } else if (i == MT - 1) {
#pragma unroll
                for (int j = 0; j < 4; ++j) bnext[j] = dequant_j(cw, ms, mm, j);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (i + 1 < MT) a_cur = a_nxt;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) bcur[j] = bnext[j];
    }
    wait_vmcnt<0>();     // no load may still be writing LDS when the workgroup ends

    if (!gvalid) return;
    // ---- store: lane holds rows 4*(lane/16)+r, column lane%16 of each 16x16 tile
    const int crow = (lane >> 4) * 4, ccol = lane & 15;
    const int64_t col0 = g * 64 + ccol;
    if (ksplit > 1) {
        float *pbase = part + (int64_t)split * M * N;
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + i * 16 + crow + r;
                if (row < M) {
                    float *prow = pbase + (int64_t)row * N + col0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) prow[j * 16] = acc[i][j][r];
                }
            }
    } else if (y_f16) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + i * 16 + crow + r;
                if (row < M) {
                    _Float16 *yrow = static_cast<_Float16 *>(y) + (int64_t)row * N + col0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) yrow[j * 16] = (_Float16)acc[i][j][r];
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + i * 16 + crow + r;
                if (row < M) {
                    float *yrow = static_cast<float *>(y) + (int64_t)row * N + col0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) yrow[j * 16] = acc[i][j][r];
                }
            }
    }
}

// Y = sum over splits of the partial tiles, in split order.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ part, int ksplit,
                                                            int64_t MN, void *__restrict__ y, int y_f16) {
    const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i4 >= MN) return;
    float4 s = *reinterpret_cast<const float4 *>(part + i4);
    for (int k = 1; k < ksplit; ++k) {
        const float4 v = *reinterpret_cast<const float4 *>(part + (int64_t)k * MN + i4);
        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    if (y_f16) {
        _Float16 *o = static_cast<_Float16 *>(y) + i4;
        o[0] = (_Float16)s.x; o[1] = (_Float16)s.y; o[2] = (_Float16)s.z; o[3] = (_Float16)s.w;
    } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(y) + i4) = s;
    }
}

template <int MT>
void launch_mt(dim3 grid, hipStream_t stream, const uint16_t *x, int M, int64_t K, int64_t N, const uint32_t *pc,
               const uint32_t *pm, int cps, float *part, void *y, int f16, int ksplit) {
    dq_gemm_kernel<MT><<<grid, dim3(kThreads), 0, stream>>>(x, M, K, N, pc, pm, cps, part, y, f16, ksplit);
}

}  // namespace

struct GemmPlan {
    int mt;              // 16-row tiles per M block
    int mblocks;
    int64_t nblocks;     // workgroups along N
    int ksplit;
    int chunks_per_split;
};

// Split-K plan.  One 8-wave workgroup per CU (the LDS ring takes most of
// the CU's 160 KB).  The time of a plan is modelled as (workgroups per CU) x
// (chunks per split) x (time of one 32-k chunk of one workgroup, ~0.8 us at
// 144 rows) plus writing and re-reading the fp32 partial tiles (~5 TB/s) and
// one extra launch for the reduction.
GemmPlan gemm_plan(int64_t M, int64_t K, int64_t N) {
    GemmPlan p{};
    const int64_t mt_needed = (M + 15) / 16;
    p.mt = (int)(mt_needed < 9 ? (mt_needed < 1 ? 1 : mt_needed) : 9);
    p.mblocks = (int)((M + 16 * p.mt - 1) / (16 * p.mt));
    p.nblocks = ((N / 64) + kWaves - 1) / kWaves;
    const int64_t nchunks = K / 32;
    const int64_t base = p.nblocks * (p.mblocks > 0 ? p.mblocks : 1);
    const double chunk_us = 0.1 + 0.7 * p.mt / 9.0;
    const double bytes_per_us = 5.0e6;
    double best = 1e300;
    int best_ks = 1;
    for (int ks = 1; ks <= 64; ++ks) {
        const int64_t cps = (nchunks + ks - 1) / ks;
        if (ks > 1 && (cps * (ks - 1) >= nchunks || cps < 8)) break;   // empty or too short splits
        const double per_cu = std::ceil((double)base * ks / kNumCU);
        const double t = per_cu * (double)cps * chunk_us +
                         (ks > 1 ? (double)(ks + 1) * (double)M * (double)N * 4.0 / bytes_per_us + 4.0 : 0.0);
        if (t < best) { best = t; best_ks = ks; }
    }
    int64_t cps = (nchunks + best_ks - 1) / best_ks;
    if (cps < 1) cps = 1;
    p.chunks_per_split = (int)cps;
    p.ksplit = nchunks > 0 ? (int)((nchunks + cps - 1) / cps) : 1;
    return p;
}

size_t gemm_ws_bytes(int64_t M, int64_t K, int64_t N) {
    const GemmPlan p = gemm_plan(M, K, N);
    if (p.ksplit <= 1) return 0;
    return (size_t)p.ksplit * (size_t)M * (size_t)N * sizeof(float);
}

fgq_status launch_dequant_gemm(const void *x, int64_t M, int64_t K, int64_t N, const uint32_t *pc,
                               const uint32_t *pm, void *y, int32_t y_dtype, void *ws, hipStream_t stream) {
    if (M == 0 || N == 0) return FGQ_OK;
    const GemmPlan p = gemm_plan(M, K, N);
    const int f16 = y_dtype == FGQ_DTYPE_F16;
    const dim3 grid((unsigned)p.nblocks, (unsigned)p.ksplit, (unsigned)p.mblocks);
    const uint16_t *xh = static_cast<const uint16_t *>(x);
    float *part = static_cast<float *>(ws);
    switch (p.mt) {
        case 1: launch_mt<1>(grid, stream, xh, (int)M, K, N, pc, pm, p.chunks_per_split, part, y, f16, p.ksplit); break;
        case 2: launch_mt<2>(grid, stream, xh, (int)M, K, N, pc, pm, p.chunks_per_split, part, y, f16, p.ksplit); break;
        case 3: launch_mt<3>(grid, stream, xh, (int)M, K, N, pc, pm, p.chunks_per_split, part, y, f16, p.ksplit); break;
        case 4: launch_mt<4>(grid, stream, xh, (int)M, K, N, pc, pm, p.chunks_per_split, part, y, f16, p.ksplit); break;
        case 5: launch_mt<5>(grid, stream, xh, (int)M, K, N, pc, pm, p.chunks_per_split, part, y, f16, p.ksplit); break;
        case 6: launch_mt<6>(grid, stream, xh, (int)M, K, N, pc, pm, p.chunks_per_split, part, y, f16, p.ksplit); break;
        case 7: launch_mt<7>(grid, stream, xh, (int)M, K, N, pc, pm, p.chunks_per_split, part, y, f16, p.ksplit); break;
        case 8: launch_mt<8>(grid, stream, xh, (int)M, K, N, pc, pm, p.chunks_per_split, part, y, f16, p.ksplit); break;
        default: launch_mt<9>(grid, stream, xh, (int)M, K, N, pc, pm, p.chunks_per_split, part, y, f16, p.ksplit); break;
    }
    fgq_status s = check_launch("dq_gemm_kernel");
    if (s != FGQ_OK || p.ksplit == 1) return s;
    const int64_t MN = M * N;   // N % 64 == 0, so MN % 4 == 0
    splitk_reduce_kernel<<<dim3((unsigned)((MN / 4 + 255) / 256)), dim3(256), 0, stream>>>(part, p.ksplit, MN, y, f16);
    return check_launch("splitk_reduce_kernel");
}

}  // namespace fgq
