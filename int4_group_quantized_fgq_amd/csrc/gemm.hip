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
//    (global_load_lds_dwordx4) into a ring of 4 slots of two 32-k chunks
//    each (the X rows, each wave's packed code words and its group
//    metadata), so 3 slots are in flight while one is multiplied, with one
//    barrier per slot and no register spent on prefetching;
//  * the packed weight layout puts the 8 k-values of one output channel in
//    one 32-bit word, in the nibble order that AND/OR with the fp16 magic
//    numbers 0x6400 (1024 + q) and 0x5400 (64 + q) turn into two values per
//    op; a packed subtract and a packed FMA give two fp16 W^ values, and the
//    next chunk is dequantised in the shadow of the current chunk's MFMAs;
//  * X rows sit in LDS with a 16-byte-slot XOR swizzle, so the rows of an A
//    fragment read hit distinct banks;
//  * K is split across workgroups when the N/512 workgroups cannot fill the
//    CUs; fp32 partial tiles are summed in split order by a second kernel.
#include <cmath>
#include <type_traits>

#include "common.h"

namespace fgq {
namespace {

constexpr int kWaves = 8;                  // waves (weight groups) per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kSC = 2;                     // 32-k chunks per LDS ring slot (one barrier per slot)
constexpr int kRing = 8 / kSC;             // ring slots: kRing-1 slots in flight

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

// Wait until at most `SLOTS` ring slots of this wave's loads are
// outstanding; a wave issues `cnt` (2..7) load instructions per slot.
template <int SLOTS>
__device__ __forceinline__ void wait_slots(int cnt) {
    switch (cnt) {
        case 2: wait_vmcnt<2 * SLOTS>(); break;
        case 3: wait_vmcnt<3 * SLOTS>(); break;
        case 4: wait_vmcnt<4 * SLOTS>(); break;
        case 5: wait_vmcnt<5 * SLOTS>(); break;
        case 6: wait_vmcnt<6 * SLOTS>(); break;
        default: wait_vmcnt<7 * SLOTS>(); break;
    }
}

// 16-byte slot swizzle of the X rows in LDS: element (row, slot c) is stored
// at slot c ^ xswz(row).  For the 16 rows of one A-fragment read (one slot
// column each), any 8 consecutive rows then cover all eight 16-byte pieces
// of a 128-byte bank cycle and the 16 rows cover all sixteen pieces of a
// 256-byte cycle, so the read is free of bank conflicts.
__device__ __forceinline__ int xswz(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

template <int MT>
struct Cfg {
    static constexpr int XCHUNK = MT * 1024;           // MT*16 rows x 64 bytes (one 32-k chunk)
    static constexpr int XBYTES = kSC * XCHUNK;
    static constexpr int BBYTES = kWaves * kSC * 1024; // packed codes, 1 KB per wave and chunk
    static constexpr int MBYTES = kWaves * kSC * 128;  // packed meta, 128 B per wave and chunk
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

    // X blocks (16 rows x 64 B) of a slot are spread over the waves:
    // block b is loaded by wave b % kWaves.
    constexpr int XBLK = MT * kSC;
    const int nx = XBLK / kWaves + (wv < XBLK % kWaves ? 1 : 0);
    const int cnt = nx + kSC + 1;                // load instructions per slot for this wave

    f32x4 acc[MT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int arow = lane & 15, akq = lane >> 4;

    // Issue this wave's direct-to-LDS loads of the kSC chunks that start at
    // chunk kc into ring slot `slot`.  Chunks past c_end (the tail of the
    // ring) and rows past M are clamped to valid addresses; those values are
    // never used for a stored output.
    auto issue = [&](int64_t kc0, int slot) {
        uint8_t *base = lds + slot * C::SLOT;
#pragma unroll
        for (int t = 0; t < (XBLK + kWaves - 1) / kWaves; ++t) {
            const int blk = t * kWaves + wv;
            if (blk < XBLK) {
                const int ch = blk / MT, rb = blk - ch * MT;
                int64_t kc = kc0 + ch;
                if (kc >= c_end) kc = c_end - 1;
                const int row = rb * 16 + (lane >> 2);
                const int c16 = (lane & 3) ^ xswz(row);            // swizzled source column
                const int grow = (m0 + row < M) ? m0 + row : M - 1;
                dma16(x + (int64_t)grow * K + kc * 32 + c16 * 8, base + blk * 1024);
            }
        }
#pragma unroll
        for (int ch = 0; ch < kSC; ++ch) {
            int64_t kc = kc0 + ch;
            if (kc >= c_end) kc = c_end - 1;
            const int64_t tile = kc * ng + gl;
            dma16(pc + (tile * 64 + lane) * 4, base + C::XBYTES + (wv * kSC + ch) * 1024);
        }
        if (lane < 8 * kSC) {
            int64_t kc = kc0 + (lane >> 3);
            if (kc >= c_end) kc = c_end - 1;
            const int64_t tile = kc * ng + gl;
            dma16(pm + tile * 32 + (lane & 7) * 4, base + C::XBYTES + C::BBYTES + wv * kSC * 128);
        }
    };

    // The fp16 magic numbers live in VGPRs so that the AND/OR pairs below
    // become single v_and_or_b32 (a VOP3 operand may not be a literal here).
    uint32_t mag1024, mag64;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(mag1024));
    asm volatile("v_mov_b32 %0, 0x54005400" : "=v"(mag64));

    // Packed codes + (step, min) pairs of one chunk -> B fragment j.
    auto dequant_j = [&](const uint4 cw, const uint4 ms, const uint4 mm, int j) -> f16x8 {
        const uint32_t W[4] = {cw.x, cw.y, cw.z, cw.w};
        const uint32_t w = W[j], w8 = w >> 8;
        const uint32_t p0 = (w & 0x000F000Fu) | mag1024;    // 1024 + q (k0, k1)
        const uint32_t p1 = (w & 0x00F000F0u) | mag64;      // 64 + q   (k2, k3)
        const uint32_t p2 = (w8 & 0x000F000Fu) | mag1024;   // 1024 + q (k4, k5)
        const uint32_t p3 = (w8 & 0x00F000F0u) | mag64;     // 64 + q   (k6, k7)
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
    // B words of chunk `ch` of ring slot `slot` for this wave.  A chunk past
    // the end of the split (its data is a clamped copy) gets step 0 and min 0,
    // so its W^ is zero and it adds nothing (a uniform branch: the chunk index
    // is the same in every lane).
    auto load_b = [&](int slot, int ch, bool valid, uint4 &cw, uint4 &ms, uint4 &mm) {
        const uint8_t *base = lds + slot * C::SLOT;
        cw = *reinterpret_cast<const uint4 *>(base + C::XBYTES + (wv * kSC + ch) * 1024 + lane * 16);
        const uint8_t *mb = base + C::XBYTES + C::BBYTES + (wv * kSC + ch) * 128 + akq * 32;
        ms = *reinterpret_cast<const uint4 *>(mb);
        mm = *reinterpret_cast<const uint4 *>(mb + 16);
        if (!valid) {
            ms = make_uint4(0u, 0u, 0u, 0u);
            mm = ms;
        }
    };
    auto a_frag = [&](int slot, int ch, int i) {
        const int row = i * 16 + arow;
        return *reinterpret_cast<const f16x8 *>(lds + slot * C::SLOT + ch * C::XCHUNK + row * 64 +
                                                ((akq ^ xswz(row)) * 16));
    };

    const int64_t nmine = c_end - c_begin;       // chunks of this split
    const int64_t nslots = (nmine + kSC - 1) / kSC;
    // B fragments: bf[ch % 2] feeds chunk ch of a slot while bf[(ch+1) % 2]
    // receives the next chunk's; with an even number of chunks per slot the
    // roles swap statically and no register copy is needed.
    static_assert(kSC % 2 == 0, "B fragment double buffer assumes an even number of chunks per slot");
    f16x8 bf[2][4];
    if (nmine > 0) {
#pragma unroll
        for (int r = 0; r < kRing - 1; ++r) issue(c_begin + (int64_t)r * kSC, r);
        wait_slots<kRing - 2>(cnt);              // this wave's B words of the first slot
        uint4 cw, ms, mm;
        load_b(0, 0, true, cw, ms, mm);
#pragma unroll
        for (int j = 0; j < 4; ++j) bf[0][j] = dequant_j(cw, ms, mm, j);
    }
    for (int64_t st = 0; st < nslots; ++st) {
        const int slot = (int)(st % kRing);
        const int nslot = (int)((st + 1) % kRing);
        wait_slots<kRing - 3>(cnt);              // slots st and st+1 of this wave have landed
        lds_barrier();                           // ... for every wave; slot st-1 is free again
#pragma unroll
        for (int ch = 0; ch < kSC; ++ch) {
            // MFMAs of one chunk, m-tile by m-tile.  A fragments are read two
            // m-tiles ahead; in the first chunk of the slot, the loads refilling
            // the freed slot are issued once the first MFMAs are in flight;
            // after each of the first m-tiles one n-tile of the next chunk's B
            // fragments is dequantised.  The scheduling fences keep that order,
            // so the address arithmetic, the VALU dequant and the LDS latency
            // sit under the matrix-core time.
            const int64_t chunk = st * kSC + ch;
            uint4 cw, ms, mm;
            if (ch + 1 < kSC)
                load_b(slot, ch + 1, chunk + 1 < nmine, cw, ms, mm);
            else
                load_b(nslot, 0, chunk + 1 < nmine, cw, ms, mm);
            const f16x8(&bcur)[4] = bf[ch % 2];
            f16x8(&bnext)[4] = bf[(ch + 1) % 2];
            f16x8 a0 = a_frag(slot, ch, 0);
            f16x8 a1 = a_frag(slot, ch, MT > 1 ? 1 : 0);
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                f16x8 a2;
                if (i + 2 < MT) a2 = a_frag(slot, ch, i + 2);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bcur[j], acc[i][j], 0, 0, 0);
                if (ch == 0 && i == 0)
                    issue(c_begin + (st + kRing - 1) * kSC, (int)((st + kRing - 1) % kRing));
                if (MT >= 4) {
                    if (i < 4) bnext[i] = dequant_j(cw, ms, mm, i);
                } else if (i == MT - 1) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) bnext[j] = dequant_j(cw, ms, mm, j);
                }
                __builtin_amdgcn_sched_barrier(0);
                a0 = a1;
                if (i + 2 < MT) a1 = a2;
            }
        }
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
// (chunks per split x time of one 32-k chunk, ~0.88 us at 144 rows, plus the
// ring fill and epilogue) plus writing and re-reading the fp32 partial tiles
// and one extra launch for the reduction; the constants are fitted to split
// sweeps on MI355X over the OPT-shaped weights.
GemmPlan gemm_plan(int64_t M, int64_t K, int64_t N) {
    GemmPlan p{};
    const int64_t mt_needed = (M + 15) / 16;
    p.mt = (int)(mt_needed < 9 ? (mt_needed < 1 ? 1 : mt_needed) : 9);
    p.mblocks = (int)((M + 16 * p.mt - 1) / (16 * p.mt));
    p.nblocks = ((N / 64) + kWaves - 1) / kWaves;
    const int64_t nchunks = K / 32;
    const int64_t base = p.nblocks * (p.mblocks > 0 ? p.mblocks : 1);
    const double chunk_us = 0.1 + 0.78 * p.mt / 9.0;    // one 32-k chunk of one workgroup
    const double ramp_us = 4.0;                          // ring fill and epilogue of a workgroup
    const double bytes_per_us = 3.0e6;                   // partial tile write + read, ~6 TB/s each
    double best = 1e300;
    int best_ks = 1;
    for (int ks = 1; ks <= 64; ++ks) {
        const int64_t cps = (nchunks + ks - 1) / ks;
        if (ks > 1 && (cps * (ks - 1) >= nchunks || cps < 8)) break;   // empty or too short splits
        const double per_cu = std::ceil((double)base * ks / kNumCU);
        const double t = per_cu * ((double)cps * chunk_us + ramp_us) +
                         (ks > 1 ? (double)ks * (double)M * (double)N * 4.0 / bytes_per_us + 3.0 : 0.0);
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
