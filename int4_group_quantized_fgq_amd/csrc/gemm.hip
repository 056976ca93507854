// Dequantising weight GEMM of one block: Y[M][N] = X[M][K] * W^[K][N] with
// M = g*m rows (m GPU batches of g rows) sharing one read of the compressed
// weight (paper-graph-ui FlexGen summary, section 3.4 "Compute Schedule";
// FlexGen review on jaehun.me, "A block is the unit of weight reuse").
// W^ = fp16(min + q*step) is restored to FP16 before the multiply (FlexGen
// review on blog.gzher.com, section 3.4) and fed to the fp16 matrix cores
// (v_mfma_f32_16x16x32_f16) with fp32 accumulation.
//
// Two weight layouts share one kernel template:
//  * CANON: the codes [K][N/2] and metadata [K][N/64] exactly as the
//    quantiser writes them (groups of 64 output channels at one input k);
//  * packed: a one-time re-layout of the same codes and metadata made
//    offline with the quantisation (word-per-fragment codes, steps
//    pre-scaled for the subnormal code placement below).
//
// Tiling (gfx950, 64-wide waves):
//  * a wave owns one weight group column (64 output channels = 4 MFMA
//    n-tiles) and every row of its M block (up to 9 m-tiles = 144 rows), so
//    one dequantised B fragment feeds up to 9 MFMAs;
//  * a workgroup is 8 waves (two per SIMD): 8/KP column groups times KP
//    k-phases (KP = 1 or 2; also 4 or 8 with the packed layout for blocks of
//    at most 4 m-tiles); the phases multiply interleaved chunks of K and are
//    summed through LDS at the end, and all waves share the X rows of each
//    K chunk through LDS;
//  * every operand reaches LDS through gfx950's direct global->LDS loads
//    (global_load_lds_dword[x4], scalar base + loop-invariant lane offset,
//    so no vector ALU work) into a ring of slots of max(2, KP) chunks, twice
//    that for k-phased workgroups where three slots still fit (the X rows,
//    the code words and the group metadata), as deep as the LDS allows, all
//    but one slot in flight, one barrier per slot;
//  * packed layout: the 8 k-values of one output channel sit in one 32-bit
//    word, in a nibble order where one AND leaves two codes in the mantissas
//    of two fp16 subnormals (q * 2^-24 or q * 2^-20); the packed metadata
//    holds the steps pre-scaled to match and everything scaled by a
//    per-column-group power of two 2^-e that keeps the scaled steps finite,
//    so one packed FMA gives two values 2^-e * W^ and the epilogue
//    multiplies by 2^e;
//  * canonical layout: the code rows of a chunk land in LDS as they are
//    (an XOR swizzle of their 16-byte pieces keeps the reads conflict-free);
//    MFMA column c of n-tile j is output channel 4c + j of the group, so a
//    lane's four n-tiles are the four nibbles of one 16-bit read per k row;
//    an AND-OR places a code in the mantissa of 1024 + q (or 64 + q), one
//    packed subtract leaves q exactly, and one packed FMA with the row's
//    step and minimum gives W^ rounded once;
//  * the next chunk is dequantised between the current chunk's MFMAs;
//  * A fragments stream three m-tiles ahead across chunk and slot boundaries;
//    X rows sit in LDS with a 16-byte-slot XOR swizzle, so the rows of an A
//    fragment read hit distinct banks;
//  * K is further split across workgroups when the column blocks cannot fill
//    the CUs; fp32 partial tiles are summed in split order by a second
//    kernel.
#include <cmath>
#include <type_traits>

#include "common.h"

namespace fgq {
namespace {

constexpr int kWaves = 8;                  // waves (weight groups) per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kSCMin = 2;                  // 32-k chunks per LDS ring slot at KP <= 2 (one barrier per slot)
constexpr int kLdsBudget = 152 * 1024;     // LDS bytes the ring may take (of 160 KB)

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Direct global->LDS load of 16 bytes per lane from sbase + voff (sbase is
// wave-uniform and lives in SGPRs, voff is the lane's 32-bit byte offset);
// lane i's bytes land at LDS address lds + 16*i (lds wave-uniform).  Written
// as inline assembly so the compiler does not track it as an LDS store: it
// would otherwise drain every load in flight (s_waitcnt vmcnt(0)) before each
// LDS read of the ring, since it cannot prove that the slot being filled
// differs from the slots being read.  The kernel waits for exactly the chunks
// it needs with explicit vmcnt counts instead.  M0 (the LDS base of the load)
// is used by nothing else in this kernel.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t lds) {
    // readfirstlane keeps the LDS address in an SGPR also inside a lane-masked
    // branch, where the compiler may otherwise hold the uniform value in a VGPR.
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0v)
                 : "memory", "m0");
}
// The same with 4 bytes per lane: lane i's dword lands at lds + 4*i.
__device__ __forceinline__ void dma4(const void *sbase, uint32_t voff, uint32_t lds) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(m0v)
                 : "memory", "m0");
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
// outstanding; a wave issues `cnt` (1..7) load instructions per slot.
template <int SLOTS>
__device__ __forceinline__ void wait_slots(int cnt) {
    switch (cnt) {
        case 1: wait_vmcnt<1 * SLOTS>(); break;
        case 2: wait_vmcnt<2 * SLOTS>(); break;
        case 3: wait_vmcnt<3 * SLOTS>(); break;
        case 4: wait_vmcnt<4 * SLOTS>(); break;
        case 5: wait_vmcnt<5 * SLOTS>(); break;
        case 6: wait_vmcnt<6 * SLOTS>(); break;
        default: wait_vmcnt<7 * SLOTS>(); break;
    }
}

// 16-byte slot swizzle of the X rows in LDS: element (row, slot c) is stored
// at slot c ^ xswz(row).  Among any 8 consecutive rows of an A-fragment read
// (one slot column each), the four rows of equal parity get four different
// slots, so the 8 lanes of one 128-byte bank cycle hit distinct banks.  The
// swizzle repeats every 8 rows, so it is the same for every 16-row m-tile.
__device__ __forceinline__ int xswz(int row) { return (row >> 1) & 3; }

// Canonical layout: a chunk's code rows (32 k rows x CG groups x 32 bytes)
// sit in LDS row-major, 16-byte piece p of row r stored at piece p ^ cswz(r).
// A 16-bit read of one k row by the lanes of an A/B fragment touches rows
// r, r+8, r+16, r+24 and the two pieces of one group: the swizzle gives the
// four rows four different piece pairs, so the eight pieces land on eight
// different 16-byte bank ranges.
__device__ __forceinline__ int cswz(int row) { return ((row >> 3) & 3) << 1; }
// Canonical layout: a chunk's metadata rows (32 k rows x CG groups, one
// dword each) sit row-major, group c of row r stored at c ^ mswz(r), so the
// four rows r, r+8, r+16, r+24 that a 32-bit read by one wave touches fall
// on four different banks.
__device__ __forceinline__ int mswz(int row) { return (row >> 3) & 3; }

// Ring and LDS layout of a workgroup with MT m-tiles and KP k-phases: the
// 8 waves are CG = 8/KP column groups x KP phases; a ring slot holds SC
// chunks, phase p multiplies the chunks p, p+KP, ... of every slot, and the
// phases' accumulators are summed through LDS at the end.
template <int MT, int KP>
struct Cfg {
    // Chunks per slot: at least kSCMin and one per phase; doubled (two of a
    // wave's own chunks per slot, half the barriers per chunk) for k-phased
    // workgroups whenever the ring still holds three slots.
    static constexpr int SC0 = KP > kSCMin ? KP : kSCMin;
    static constexpr int slot_bytes(int sc) { return sc * MT * 1024 + kWaves * (sc / KP) * (1024 + 128); }
    static constexpr int SC = (KP >= 2 && kLdsBudget / slot_bytes(2 * SC0) >= 3) ? 2 * SC0 : SC0;
    static constexpr int CG = kWaves / KP;             // column groups (64 channels each)
    static constexpr int LC = SC / KP;                 // chunks per wave and slot
    static constexpr int XCHUNK = MT * 1024;           // MT*16 rows x 64 bytes (one 32-k chunk)
    static constexpr int XBYTES = SC * XCHUNK;
    static constexpr int BBYTES = kWaves * LC * 1024;  // packed codes, 1 KB per wave and chunk
    static constexpr int MBYTES = kWaves * LC * 128;   // packed meta, 128 B per wave and chunk
    static constexpr int SLOT = XBYTES + BBYTES + MBYTES;
    // Ring slots: as many as the LDS budget holds (up to 8), NR-1 in flight.
    static constexpr int NR = kLdsBudget / SLOT < 8 ? kLdsBudget / SLOT : 8;
    // Slots per unrolled loop turn: the B double buffer alternates per chunk,
    // so a turn must hold an even number of this wave's chunks.
    static constexpr int UNROLL = (NR * LC) % 2 ? 2 * NR : NR;
    static constexpr int RING = NR * SLOT;
    static constexpr int RED = (KP - 1) * CG * MT * 4 * 64 * 16;   // accumulators of phases 1..KP-1
    static constexpr int LDS = RING > RED ? RING : RED;
    static_assert(SC % KP == 0, "every phase takes the same number of chunks of a slot");
    static_assert(NR >= 3, "ring too shallow");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Raw B operands of one chunk as read from LDS, before dequantisation.
struct BRawPacked {
    uint4 cw, ms, mm;        // code word (4 n-tiles), scaled step pairs, scaled minimum pairs
};
struct BRawCanon {
    uint32_t v[4];           // k rows (2p, 2p+1) of the lane's 8: nibble j of each half is n-tile j
    uint32_t sp[4], mp[4];   // fp16 (step, step) and (min, min) of rows 2p, 2p+1
};

// wc / wm: the weight's codes and metadata, canonical (CANON: uint8 codes
// [K][N/2], uint32 meta [K][N/64]) or packed.
template <int MT, int KP, bool CANON>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void dq_gemm_kernel(const uint16_t *__restrict__ x, int M, int64_t K, int64_t N,
                    const void *__restrict__ wc, const uint32_t *__restrict__ wm, int chunks_per_split,
                    float *__restrict__ part, void *__restrict__ y, int y_f16, int ksplit) {
    using C = Cfg<MT, KP>;
    constexpr int CG = C::CG, LC = C::LC, NR = C::NR;
    using BRaw = std::conditional_t<CANON, BRawCanon, BRawPacked>;
    const uint32_t *pc = static_cast<const uint32_t *>(wc);
    const uint8_t *cc = static_cast<const uint8_t *>(wc);
    __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS];
    const uint32_t lds0 = lds_addr(lds);

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int cg = wv % CG, phase = wv / CG;

    // Workgroups are dealt to the 8 XCDs round-robin in launch order.  Remap
    // the launch index so that each XCD gets a contiguous run of tiles in
    // (column block fastest, then split) order: the tiles of one split share
    // their X slice, which then stays in that XCD's L2 instead of being
    // fetched by every XCD.
    const int nbx = gridDim.x, nby = gridDim.y;
    const int total = nbx * nby * gridDim.z;
    const int lin = blockIdx.x + nbx * (blockIdx.y + nby * blockIdx.z);
    const int xcd = lin & 7, per = total >> 3, extra = total & 7;
    const int tile = xcd * per + (xcd < extra ? xcd : extra) + (lin >> 3);
    const int bx = tile % nbx, by = (tile / nbx) % nby, bz = tile / (nbx * nby);

    const int64_t ng = N >> 6;
    const int64_t g = (int64_t)bx * CG + cg;
    const bool gvalid = g < ng;
    const int64_t gl = gvalid ? g : ng - 1;      // clamped group for loads
    const int split = by;
    const int m0 = bz * MT * 16;
    // Chunk indices fit in 32 bits (K <= 2^23), so their compares stay scalar.
    const int nchunks = (int)(K >> 5);
    const int c_begin = split * chunks_per_split;
    int c_end = c_begin + chunks_per_split;
    if (c_end > nchunks) c_end = nchunks;

    // X blocks (16 rows x 64 B) of a slot are spread over the waves:
    // block b is loaded by wave b % kWaves.
    constexpr int SC = C::SC;
    constexpr int XBLK = MT * SC;
    constexpr int XT = (XBLK + kWaves - 1) / kWaves;
    const int nx = XBLK / kWaves + (wv < XBLK % kWaves ? 1 : 0);
    // Canonical metadata of a slot (SC chunks x 32 rows x CG groups x 4 B)
    // goes in 256-byte instructions, instruction e by wave e.
    constexpr int NMETA = SC * 32 * CG * 4 / 256;
    const int nm = CANON ? (wv < NMETA ? 1 : 0) : 1;
    const int cnt = nx + LC + nm;                // load instructions per slot for this wave

    // Loop-invariant lane offsets of the loads (the per-chunk part of every
    // address is wave-uniform and stays in SGPRs).  X rows past M are
    // clamped to row M-1; those rows are never stored.
    const uint16_t *xm = x + (int64_t)m0 * K;
    uint32_t xoff[XT];
#pragma unroll
    for (int t = 0; t < XT; ++t) {
        const int blk = t * kWaves + wv;
        const int rb = blk % MT;
        const int row = rb * 16 + (lane >> 2);
        const int64_t grow = (m0 + row < M) ? row : M - 1 - m0;
        xoff[t] = (uint32_t)(grow * K * 2 + (((lane & 3) ^ xswz(row)) * 16));
    }
    const uint32_t coff = (uint32_t)lane * 16;
    uint32_t moff = (uint32_t)((lane >> 3) * KP * ng * 128 + (lane & 7) * 16);
    constexpr int RPM = 64 / CG;                 // canonical metadata rows per instruction
    int mchunk = 0;                              // chunk of the slot that this wave's instruction fills
    if constexpr (CANON) {
        const int srow = wv * RPM + lane / CG;   // row of the slot (0..63)
        const int row = srow % 32;
        int64_t grp = (int64_t)bx * CG + ((lane % CG) ^ mswz(row));
        if (grp >= ng) grp = ng - 1;
        moff = (uint32_t)((row * ng + grp) * 4);
        mchunk = (wv * RPM) / 32;
    }
    // Canonical codes: the workgroup's code rows of a slot (SC chunks x 32
    // rows x CG groups x 32 bytes) are loaded 1 KB per instruction, RPD rows
    // each, instruction d by wave d / LC.  Lane l takes 16-byte piece
    // (l % (2 CG)) ^ cswz(row) of row l / (2 CG), so the pieces land
    // swizzled; pieces of groups past N re-read the last group.
    constexpr int RPD = 32 / CG;
    const int64_t halfN = N >> 1;
    uint32_t ccoff[LC];
#pragma unroll
    for (int lc = 0; lc < LC; ++lc) {
        const int d = wv * LC + lc;
        const int row = (d * RPD) % 32 + lane / (2 * CG);
        const int p = (lane % (2 * CG)) ^ cswz(row);
        int64_t grp = (int64_t)bx * CG + (p >> 1);
        if (grp >= ng) grp = ng - 1;
        ccoff[lc] = (uint32_t)(row * halfN + grp * 32 + (p & 1) * 16);
    }

    f32x4 acc[MT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int arow = lane & 15, akq = lane >> 4;
    // The AND-OR masks and magic numbers of the canonical dequantisation, held
    // in VGPRs so that each AND-OR is one three-operand bit operation (two of
    // its operands could not both be scalar or literal).
    uint32_t kmask[2] = {0x000F000Fu, 0x00F000F0u}, kmagic[2] = {0x64006400u, 0x54005400u};
    if constexpr (CANON) {
        asm volatile("" : "+v"(kmask[0]), "+v"(kmask[1]), "+v"(kmagic[0]), "+v"(kmagic[1]));
    }
    const int aoff = phase * C::XCHUNK + arow * 64 + ((akq ^ xswz(arow)) * 16);

    // Issue this wave's direct-to-LDS loads for the slot of SC chunks that
    // starts at chunk kc0: its share of the X blocks and the code words and
    // metadata of its own chunks kc0 + phase + lc*KP.  Chunks past c_end (the
    // tail of the ring) are clamped to the last chunk of the split; a chunk
    // past c_end is never multiplied.
    auto issue = [&](int kc0, int slot) {
        const uint32_t sb = lds0 + slot * C::SLOT;
#pragma unroll
        for (int t = 0; t < XT; ++t) {
            const int blk = t * kWaves + wv;
            if (blk < XBLK) {
                int kc = kc0 + blk / MT;
                if (kc >= c_end) kc = c_end - 1;
                dma16(xm + (int64_t)kc * 32, xoff[t], sb + blk * 1024);
            }
        }
        const int k1 = kc0 + phase;              // this wave's first chunk of the slot
#pragma unroll
        for (int lc = 0; lc < LC; ++lc) {
            if constexpr (CANON) {
                const int d = wv * LC + lc;
                int kc = kc0 + (d * RPD) / 32;
                if (kc >= c_end) kc = c_end - 1;
                dma16(cc + (int64_t)kc * 32 * halfN, ccoff[lc], sb + C::XBYTES + d * 1024);
            } else {
                int kc = k1 + lc * KP;
                if (kc >= c_end) kc = c_end - 1;
                dma16(pc + ((int64_t)kc * ng + gl) * 256, coff, sb + C::XBYTES + (wv * LC + lc) * 1024);
            }
        }
        const int kc = k1 < c_end ? k1 : c_end - 1;
        const int left = (c_end - kc + KP - 1) / KP;     // own chunks left from kc on (>= 1)
        // canonical: instruction wv fills bytes [256 wv, 256 wv + 256) of the
        // slot's metadata; packed: each wave's 128 bytes per own chunk
        const uint32_t mdst = sb + C::XBYTES + C::BBYTES + wv * (CANON ? 256 : LC * 128);
        if constexpr (CANON) {
            if (wv < NMETA) {
                int mk = kc0 + mchunk;
                if (mk >= c_end) mk = c_end - 1;
                dma4(wm + (int64_t)mk * 32 * ng, moff, mdst);
            }
        } else {
            const int nmeta = 8 * (left < LC ? left : LC);
            if (lane < nmeta) dma16(wm + ((int64_t)kc * ng + gl) * 32, moff, mdst);
        }
    };

    // Half h (0..7) of the dequantisation of one chunk's B fragments: n-tile
    // j = h/2, k-values 0..3 (h even) or 4..7 (h odd).
    //  * packed: one AND leaves a code pair in the mantissas of two fp16
    //    subnormals, q * 2^-24 (codes 0, 1 of the pair of pairs) or q * 2^-20
    //    (codes 2, 3); the packed steps are pre-scaled by 2^(24 - e) and
    //    2^(20 - e) and the minima by 2^-e, so one packed FMA gives
    //    2^-e * fp16(min + q * step) with a single rounding (the product is
    //    exact); the epilogue multiplies by 2^e.
    //  * canonical: nibble j of a row's 16-bit read is the code of output
    //    channel 4c + j.  An AND-OR puts it in the mantissa of 1024 + q
    //    (nibbles 0, 2: bits 0-3) or 64 + q (nibbles 1, 3: bits 4-7), an
    //    exact packed subtract leaves q, and one packed FMA gives
    //    fp16(min + q * step) rounded once, for two k rows at a time.
    auto dequant_half = [&](const BRaw &raw, int h, u32x4(&b)[4]) {
        const int j = h >> 1;
        uint32_t u0, u1;
        if constexpr (CANON) {
            const bool odd = j & 1;
            const uint32_t mask = odd ? kmask[1] : kmask[0];
            const uint32_t magic = odd ? kmagic[1] : kmagic[0];
            const _Float16 bias = odd ? (_Float16)64.0f : (_Float16)1024.0f;
            const f16x2 b2 = {bias, bias};
            uint32_t uu[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int p = (h & 1) * 2 + e;
                const uint32_t src = j >= 2 ? raw.v[p] >> 8 : raw.v[p];
                const f16x2 q = as_f16x2((src & mask) | magic) - b2;
                uu[e] = as_u32(__builtin_elementwise_fma(q, as_f16x2(raw.sp[p]), as_f16x2(raw.mp[p])));
            }
            u0 = uu[0];
            u1 = uu[1];
        } else {
            const uint4 cw = raw.cw, ms = raw.ms, mm = raw.mm;
            const uint32_t W[4] = {cw.x, cw.y, cw.z, cw.w};
            const uint32_t w = (h & 1) ? W[j] >> 8 : W[j];
            const uint32_t s0 = (h & 1) ? ms.z : ms.x, s1 = (h & 1) ? ms.w : ms.y;
            const uint32_t n0 = (h & 1) ? mm.z : mm.x, n1 = (h & 1) ? mm.w : mm.y;
            const f16x2 c0 = as_f16x2(w & 0x000F000Fu);
            const f16x2 c1 = as_f16x2(w & 0x00F000F0u);
            u0 = as_u32(__builtin_elementwise_fma(c0, as_f16x2(s0), as_f16x2(n0)));
            u1 = as_u32(__builtin_elementwise_fma(c1, as_f16x2(s1), as_f16x2(n1)));
        }
        // An empty use pins the values here: the next chunk may be past the
        // end of the split, and without it the compiler sinks this work past
        // that test, out of the MFMA shadow.
        asm volatile("" ::"v"(u0), "v"(u1));
        b[j][(h & 1) * 2] = u0;
        b[j][(h & 1) * 2 + 1] = u1;
    };
    // Canonical layout: lane (q = lane/16, c = lane%16) reads bytes 2c, 2c+1
    // of its group's 32 bytes in k rows 8q..8q+7 of a chunk (rows CG*32
    // bytes apart, pieces swizzled by cswz(8q + i) = 2q).
    const int cboff = akq * 8 * CG * 32 + (((2 * cg + (arow >> 3)) ^ (2 * akq)) * 16) + ((2 * arow) & 15);
    // ... and the metadata of its group in those rows (mswz(8q + i) = q).
    const int cmoff = (akq * 8 * CG + (cg ^ akq)) * 4;
    // Raw B operands of this wave's chunk lc of ring slot `slot`: the packed
    // code words and (step, min) pairs, or the canonical code rows and
    // metadata words.
    auto load_b = [&](int slot, int lc, BRaw &raw) {
        const uint8_t *base = lds + slot * C::SLOT;
        const uint8_t *mb = base + C::XBYTES + C::BBYTES + (wv * LC + lc) * 128 + akq * 32;
        if constexpr (CANON) {
            const uint8_t *mc = base + C::XBYTES + C::BBYTES + (phase + lc * KP) * 32 * CG * 4 + cmoff;
            const uint8_t *cb = base + C::XBYTES + (phase + lc * KP) * CG * 1024 + cboff;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t lo = *reinterpret_cast<const uint16_t *>(cb + (2 * p) * CG * 32);
                const uint32_t hi = *reinterpret_cast<const uint16_t *>(cb + (2 * p + 1) * CG * 32);
                raw.v[p] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);   // (lo.b0, lo.b1, hi.b0, hi.b1)
            }
            uint32_t mw[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) mw[i] = *reinterpret_cast<const uint32_t *>(mc + i * CG * 4);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                raw.sp[p] = __builtin_amdgcn_perm(mw[2 * p + 1], mw[2 * p], 0x07060302u);   // (step, step)
                raw.mp[p] = __builtin_amdgcn_perm(mw[2 * p + 1], mw[2 * p], 0x05040100u);   // (min, min)
            }
        } else {
            raw.cw = *reinterpret_cast<const uint4 *>(base + C::XBYTES + (wv * LC + lc) * 1024 + lane * 16);
            raw.ms = *reinterpret_cast<const uint4 *>(mb);
            raw.mm = *reinterpret_cast<const uint4 *>(mb + 16);
        }
    };
    // A fragment of m-tile i of this wave's chunk lc of ring slot `slot`.
    auto a_frag = [&](int slot, int lc, int i) {
        return *reinterpret_cast<const f16x8 *>(lds + slot * C::SLOT + lc * KP * C::XCHUNK + i * 1024 + aoff);
    };

    const int nmine = c_end - c_begin;           // chunks of this split
    const int nslots = (nmine + SC - 1) / SC;
    // B fragments: bf[n % 2] feeds this wave's n-th chunk of a ring turn
    // while bf[(n+1) % 2] receives the next one's; with an even number of
    // chunks per ring turn the roles swap statically, with no register copy.
    u32x4 bf[2][4];
    // A fragments stream through PD registers, PD m-tiles ahead of the
    // MFMAs, across chunk and slot boundaries.  The barrier that makes slot
    // st+1 visible (every wave's loads of it have landed) and frees slot st
    // (every wave's LDS reads of it are complete) is taken inside the last
    // chunk of slot st, just before the first read of slot st+1, while PD
    // m-tiles of MFMAs with operands already in registers remain: the LDS
    // latency after the barrier hides behind them.
    constexpr int PD = MT >= 3 ? 3 : MT;
    f16x8 ap[PD];                                // ap[d]: fragment d m-tiles ahead
    if (nmine > 0) {
#pragma unroll
        for (int r = 0; r < NR - 1; ++r) issue(c_begin + r * SC, r);
        wait_slots<NR - 2>(cnt);                 // this wave's loads of the first slot
        lds_barrier();                           // ... and every wave's
        BRaw raw;
        load_b(0, 0, raw);
#pragma unroll
        for (int h = 0; h < 8; ++h) dequant_half(raw, h, bf[0]);
#pragma unroll
        for (int d = 0; d < PD; ++d) ap[d] = a_frag(0, 0, d);
    }
    // The ring is unrolled so that every slot offset is an immediate.
    for (int s0 = 0; s0 < nslots; s0 += C::UNROLL) {
#pragma unroll
        for (int u = 0; u < C::UNROLL; ++u) {
            const int st = s0 + u, r = u % NR;
            if (st >= nslots) break;
#pragma unroll
            for (int lc = 0; lc < LC; ++lc) {
                // MFMAs of one chunk, m-tile by m-tile.  With the first chunk
                // of the slot, the loads refilling slot st-1 are issued once
                // the first MFMAs are in flight; the next chunk's B fragments
                // are dequantised in eight halves spread over the m-tiles,
                // each half interleaved with the MFMAs so the VALU work runs
                // in their shadow.  A wave only leaves this loop early in the
                // last slot, which takes no barrier.
                if (st * SC + phase + lc * KP >= nmine) break;
                // The next chunk's B words: in this slot, or (last chunk of
                // the slot) this wave's own loads of the next slot (packed),
                // for which its vmcnt is enough.  Slot st+1 is only certain
                // to have landed once this slot's refill is issued (at most
                // NR-2 slots outstanding after it), so in a slot's first
                // chunk that load waits for the refill and the
                // dequantisation starts one m-tile later.  The canonical
                // code rows and metadata of a slot come from every wave's
                // loads, so there a barrier publishes the next slot first
                // (the barrier later in the chunk still frees this slot).
                const bool last = lc + 1 == LC;
                const bool late = last && lc == 0;
                BRaw raw;
                auto load_next_slot = [&]() {
                    wait_slots<NR - 2>(cnt);
                    if constexpr (CANON) {
                        if (st + 1 < nslots) {
                            lds_barrier();
                            load_b((r + 1) % NR, 0, raw);
                        } else {
                            raw = BRaw{};
                        }
                    } else {
                        load_b((r + 1) % NR, 0, raw);
                    }
                };
                if (!last) {
                    load_b(r, lc + 1, raw);
                } else if (!late) {
                    load_next_slot();
                }
                const int bi = (u * LC + lc) % 2;
                const u32x4(&bcur)[4] = bf[bi];
                u32x4(&bnext)[4] = bf[bi ^ 1];
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const int f = i + PD;                // fragment to prefetch
                    f16x8 an;
                    if (f < MT) {
                        an = a_frag(r, lc, f);
                    } else if (!last) {
                        an = a_frag(r, lc + 1, f - MT);
                    } else {
                        if (f == MT && st + 1 < nslots) {
                            wait_slots<NR - 2>(cnt);  // slot st+1 of this wave has landed
                            lds_barrier();
                        }
                        an = a_frag((r + 1) % NR, 0, f - MT);
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            ap[0], __builtin_bit_cast(f16x8, bcur[j]), acc[i][j], 0, 0, 0);
                    if (lc == 0 && i == 0) {
                        issue(c_begin + (st + NR - 1) * SC, (r + NR - 1) % NR);
                        if (late) load_next_slot();
                    }
#pragma unroll
                    for (int h = 0; h < 8; ++h) {
                        const int at = (late && MT > 1) ? 1 + (h * (MT - 1)) / 8 : (h * MT) / 8;
                        if (at == i) dequant_half(raw, h, bnext);
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // then two VALU ops
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int d = 0; d + 1 < PD; ++d) ap[d] = ap[d + 1];
                    ap[PD - 1] = an;
                }
            }
        }
    }
    wait_vmcnt<0>();     // no load may still be writing LDS when the ring is reused or the workgroup ends

    if constexpr (KP > 1) {
        // Sum the phases in LDS, in phase order: phases 1..KP-1 park their
        // accumulators (lane-major, so reads and writes are conflict-free),
        // phase 0 adds them.
        f32x4 *red = reinterpret_cast<f32x4 *>(lds);
        lds_barrier();                           // every wave is done with the ring
        if (phase > 0) {
            f32x4 *mine = red + (size_t)((phase - 1) * CG + cg) * MT * 4 * 64 + lane;
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) mine[(i * 4 + j) * 64] = acc[i][j];
        }
        lds_barrier();
        if (phase == 0) {
#pragma unroll
            for (int p = 1; p < KP; ++p) {
                const f32x4 *other = red + (size_t)((p - 1) * CG + cg) * MT * 4 * 64 + lane;
#pragma unroll
                for (int i = 0; i < MT; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] += other[(i * 4 + j) * 64];
            }
        }
    }

    // Phase 0 of each valid column group holds the workgroup's result.
    const bool active = gvalid && phase == 0;
    if constexpr (!CANON) {
        // ---- undo the column group's exponent (a power of two: exact)
        const float gscale = __builtin_amdgcn_ldexpf(1.0f, active ? (int)wm[(int64_t)nchunks * ng * 32 + g] : 0);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] *= gscale;
    }
    // ---- store: lane holds rows 4*(lane/16)+r of each 16x16 tile, MFMA
    // column lane%16, which is output channel 64g + 16j + lane%16 (packed)
    // or 64g + 4(lane%16) + j (canonical: four consecutive channels)
    const int crow = (lane >> 4) * 4, ccol = lane & 15;
    const int64_t col0 = g * 64 + (CANON ? 4 * ccol : ccol);
    auto store_row = [&](auto *dst, const f32x4 *v) {
        using T = std::remove_pointer_t<decltype(dst)>;
        if constexpr (CANON) {
            if constexpr (std::is_same_v<T, float>) {
                *reinterpret_cast<f32x4 *>(dst) = f32x4{v[0][0], v[1][0], v[2][0], v[3][0]};
            } else {
                typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
                *reinterpret_cast<f16x4 *>(dst) =
                    f16x4{(_Float16)v[0][0], (_Float16)v[1][0], (_Float16)v[2][0], (_Float16)v[3][0]};
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[j * 16] = (T)v[j][0];
        }
    };
    // value (i, j, r) of this lane as the first component of a vector, so
    // that store_row takes one row's four values
    auto row_vals = [&](int i, int r, f32x4 (&v)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = f32x4{acc[i][j][r], 0.f, 0.f, 0.f};
    };
    auto store_final = [&]() {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + i * 16 + crow + r;
                if (row < M) {
                    f32x4 v[4];
                    row_vals(i, r, v);
                    if (y_f16)
                        store_row(static_cast<_Float16 *>(y) + (int64_t)row * N + col0, v);
                    else
                        store_row(static_cast<float *>(y) + (int64_t)row * N + col0, v);
                }
            }
    };
    if (ksplit == 1) {
        if (active) store_final();
        return;
    }
    // ---- split-K: this split's partial tile, summed in split order by a
    // second kernel
    if (!active) return;
    float *pbase = part + (int64_t)split * M * N;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = m0 + i * 16 + crow + r;
            if (row < M) {
                f32x4 v[4];
                row_vals(i, r, v);
                store_row(pbase + (int64_t)row * N + col0, v);
            }
        }
}

struct LaunchArgs {
    dim3 grid;
    hipStream_t stream;
    const uint16_t *x;
    int M;
    int64_t K, N;
    const void *wc;
    const uint32_t *wm;
    int cps;
    float *part;
    void *y;
    int f16, ksplit;
};

template <int MT, int KP, bool CANON>
void launch_one(const LaunchArgs &a) {
    dq_gemm_kernel<MT, KP, CANON><<<a.grid, dim3(kThreads), 0, a.stream>>>(
        a.x, a.M, a.K, a.N, a.wc, a.wm, a.cps, a.part, a.y, a.f16, a.ksplit);
}

// k-phases per workgroup: 1 and 2 for every row count; 4 and 8 (one or two
// column groups per workgroup, phases summed in LDS) for up to 64 rows with
// the packed layout.
// Y = sum over splits of the partial tiles, in split order.  The loads of up
// to eight splits are in flight together (one memory latency per eight
// splits, not per split); the sum still runs in split order.
constexpr int kReduceBatch = 8;
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ part, int ksplit,
                                                            int64_t MN, void *__restrict__ y, int y_f16) {
    const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i4 >= MN) return;
    float4 s = *reinterpret_cast<const float4 *>(part + i4);
    for (int k = 1; k < ksplit; k += kReduceBatch) {
        float4 v[kReduceBatch];
#pragma unroll
        for (int u = 0; u < kReduceBatch; ++u)
            if (k + u < ksplit) v[u] = *reinterpret_cast<const float4 *>(part + (int64_t)(k + u) * MN + i4);
#pragma unroll
        for (int u = 0; u < kReduceBatch; ++u)
            if (k + u < ksplit) {
                s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w;
            }
    }
    if (y_f16) {
        _Float16 *o = static_cast<_Float16 *>(y) + i4;
        o[0] = (_Float16)s.x; o[1] = (_Float16)s.y; o[2] = (_Float16)s.z; o[3] = (_Float16)s.w;
    } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(y) + i4) = s;
    }
}

template <int MT, bool CANON>
void launch_mt(int kp, const LaunchArgs &a) {
    if constexpr (MT <= 4 && !CANON) {
        if (kp == 8) return launch_one<MT, 8, CANON>(a);
        if (kp == 4) return launch_one<MT, 4, CANON>(a);
    }
    if (kp == 2) return launch_one<MT, 2, CANON>(a);
    launch_one<MT, 1, CANON>(a);
}

template <bool CANON>
void launch_layout(int mt, int kp, const LaunchArgs &a) {
    switch (mt) {
        case 1: launch_mt<1, CANON>(kp, a); break;
        case 2: launch_mt<2, CANON>(kp, a); break;
        case 3: launch_mt<3, CANON>(kp, a); break;
        case 4: launch_mt<4, CANON>(kp, a); break;
        case 5: launch_mt<5, CANON>(kp, a); break;
        case 6: launch_mt<6, CANON>(kp, a); break;
        case 7: launch_mt<7, CANON>(kp, a); break;
        case 8: launch_mt<8, CANON>(kp, a); break;
        default: launch_mt<9, CANON>(kp, a); break;
    }
}

}  // namespace

struct GemmPlan {
    int mt;              // 16-row tiles per M block
    int mblocks;
    int kp;              // k-phases inside a workgroup (1, 2, 4 or 8)
    int64_t nblocks;     // workgroups along N (each 64 * 8 / kp channels)
    int ksplit;
    int chunks_per_split;
};

// Work split.  One 8-wave workgroup per CU (the LDS ring takes most of the
// CU's 160 KB).  K is shared out first between the kp phases of a workgroup
// (summed in LDS), then between ksplit workgroups (fp32 partial tiles summed
// by a second kernel).  The time of a plan is modelled as, per round of
// workgroups on the 256 CUs, the chunks of one wave times the time of one
// 32-k chunk (which grows with the rows), the ring fill and epilogue and the
// phase sum, plus the partial tiles' traffic; the constants are a
// least-squares fit to a sweep of forced plans (k-phases 1..8, 1..32 splits)
// over the OPT-6.7B, OPT-30B and OPT-175B weight shapes at their block sizes
// on MI355X (median error 7%).
GemmPlan gemm_plan(int64_t M, int64_t K, int64_t N, bool canonical) {
    GemmPlan p{};
    const int64_t mt_needed = (M + 15) / 16;
    p.mt = (int)(mt_needed < 9 ? (mt_needed < 1 ? 1 : mt_needed) : 9);
    p.mblocks = (int)((M + 16 * p.mt - 1) / (16 * p.mt));
    const int64_t ng = N / 64;
    const int64_t nchunks = K / 32;
    const double chunk_us = 0.095 + 0.074 * p.mt;       // one 32-k chunk of one wave
    const double round_us = 1.87;                        // ring fill and epilogue of a round of workgroups
    const double partial_us_per_mb = 0.364;              // partial tiles written, re-read and summed
    double best = 1e300;
    int best_ks = 1, best_kp = 1;
    const int kp_max = (!canonical && p.mt <= 4) ? 8 : 2;
    for (int kp = 1; kp <= kp_max; kp *= 2) {
        const int64_t cols = kWaves / kp;
        const int64_t base = ((ng + cols - 1) / cols) * (p.mblocks > 0 ? p.mblocks : 1);
        const double phase_us = 0.67 * (kp - 1) * p.mt / 4.0;   // LDS sum of the phases
        for (int ks = 1; ks <= 64; ++ks) {
            const int64_t cps = (nchunks + ks - 1) / ks;
            if (ks > 1 && (cps * (ks - 1) >= nchunks || cps < 8 * kp)) break;   // empty or too short splits
            if (ks > 1 && (double)ks * (double)M * (double)N * 4.0 > 1099511627776.0) break;   // partials > 1 TiB
            const double rounds = std::ceil((double)base * ks / kNumCU);
            const double per_wave = std::ceil((double)cps / kp);
            const double t = rounds * (round_us + per_wave * chunk_us + phase_us) +
                             (ks > 1 ? (double)ks * (double)M * (double)N * 4e-6 * partial_us_per_mb : 0.0);
            if (t < best) { best = t; best_ks = ks; best_kp = kp; }
        }
    }
    p.kp = best_kp;
    p.nblocks = (ng + kWaves / p.kp - 1) / (kWaves / p.kp);
    int64_t cps = (nchunks + best_ks - 1) / best_ks;
    if (cps < 1) cps = 1;
    p.chunks_per_split = (int)cps;
    p.ksplit = nchunks > 0 ? (int)((nchunks + cps - 1) / cps) : 1;
    return p;
}

// The workspace (split-K partial tiles) covers both layouts' plans.
size_t gemm_ws_bytes(int64_t M, int64_t K, int64_t N) {
    const GemmPlan a = gemm_plan(M, K, N, false), b = gemm_plan(M, K, N, true);
    const int ks = a.ksplit > b.ksplit ? a.ksplit : b.ksplit;
    if (ks <= 1) return 0;
    return (size_t)ks * (size_t)M * (size_t)N * sizeof(float);
}

// canonical: wc = uint8 codes [K][N/2], wm = uint32 meta [K][N/64];
// otherwise the packed layout of fgq_pack_weight_g64.
fgq_status launch_dequant_gemm(const void *x, int64_t M, int64_t K, int64_t N, const void *wc, const uint32_t *wm,
                               bool canonical, void *y, int32_t y_dtype, void *ws, hipStream_t stream) {
    if (M == 0 || N == 0) return FGQ_OK;
    const GemmPlan p = gemm_plan(M, K, N, canonical);
    if (p.mblocks > 65535 || (double)p.nblocks * p.ksplit * p.mblocks >= 2147483648.0)
        return fail(FGQ_ERR_SHAPE, "dequant GEMM grid too large (M=%lld N=%lld)", (long long)M, (long long)N);
    LaunchArgs a{};
    a.grid = dim3((unsigned)p.nblocks, (unsigned)p.ksplit, (unsigned)p.mblocks);
    a.stream = stream;
    a.x = static_cast<const uint16_t *>(x);
    a.M = (int)M;
    a.K = K;
    a.N = N;
    a.wc = wc;
    a.wm = wm;
    a.cps = p.chunks_per_split;
    a.part = static_cast<float *>(ws);
    a.y = y;
    a.f16 = y_dtype == FGQ_DTYPE_F16;
    a.ksplit = p.ksplit;
    if (canonical)
        launch_layout<true>(p.mt, p.kp, a);
    else
        launch_layout<false>(p.mt, p.kp, a);
    fgq_status s = check_launch("dq_gemm_kernel");
    if (s != FGQ_OK || p.ksplit == 1) return s;
    const int64_t MN = M * N;   // N % 64 == 0, so MN % 4 == 0
    splitk_reduce_kernel<<<dim3((unsigned)((MN / 4 + 255) / 256)), dim3(256), 0, stream>>>(
        a.part, p.ksplit, MN, y, a.f16);
    return check_launch("splitk_reduce_kernel");
}

}  // namespace fgq
