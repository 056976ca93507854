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
//  * a workgroup is 4 waves (256 output channels); the X rows of the current
//    K stage are staged once in LDS and read by all 4 waves;
//  * the packed weight layout puts the 8 k-values of one output channel in
//    one 32-bit word, in the nibble order that two AND-OR ops per pair turn
//    into the fp16 "1024 + q" / "64 + q" magic numbers; one packed subtract
//    and one packed FMA then give two fp16 W^ values;
//  * K is split across workgroups when N/256 workgroups cannot fill the 256
//    CUs; the fp32 partial tiles are summed in a fixed order by a second
//    kernel, so results are deterministic.
#include "common.h"

namespace fgq {
namespace {

constexpr int kWaves = 4;          // waves (weight groups) per workgroup
constexpr int kStageK = 64;        // K rows of X staged in LDS per step
constexpr int kLdsRow = kStageK + 8;  // halves per LDS row (16-byte pad)

template <int MT>
__global__ __launch_bounds__(256) void dq_gemm_kernel(const uint16_t *__restrict__ x, int M, int64_t K, int64_t N,
                                                      const uint32_t *__restrict__ pc,
                                                      const uint32_t *__restrict__ pm, int chunks_per_split,
                                                      float *__restrict__ part, void *__restrict__ y, int y_f16,
                                                      int ksplit) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[MT * 16 * kLdsRow];

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int64_t ng = N >> 6;
    const int64_t g = (int64_t)blockIdx.x * kWaves + wv;
    const bool gvalid = g < ng;
    const int split = blockIdx.y;
    const int m0 = blockIdx.z * MT * 16;
    const int64_t nchunks = K >> 5;
    const int64_t c_begin = (int64_t)split * chunks_per_split;
    int64_t c_end = c_begin + chunks_per_split;
    if (c_end > nchunks) c_end = nchunks;

    f32x4 acc[MT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int arow = lane & 15, akq = lane >> 4;
    constexpr int kPieces = MT * 16 * (kStageK / 8);             // 16-byte pieces per full stage
    constexpr int kPerThread = (kPieces + 255) / 256;

    // X stage prefetch registers (one stage ahead) and B fragment prefetch (one chunk ahead)
    uint4 xr[kPerThread];
    auto load_x = [&](int64_t cs) {
        const int64_t kb = cs * 32;
        const int nst = (int)((c_end - cs) < (kStageK / 32) ? (c_end - cs) : (kStageK / 32));
        const int ppr = nst * 4;
#pragma unroll
        for (int t = 0; t < kPerThread; ++t) {
            const int p = threadIdx.x + t * 256;
            const int r = p / (kStageK / 8), c = p - r * (kStageK / 8);
            xr[t] = make_uint4(0u, 0u, 0u, 0u);
            if (p < kPieces && c < ppr && m0 + r < M)
                xr[t] = *reinterpret_cast<const uint4 *>(x + (int64_t)(m0 + r) * K + kb + c * 8);
        }
    };
    auto store_x = [&]() {
#pragma unroll
        for (int t = 0; t < kPerThread; ++t) {
            const int p = threadIdx.x + t * 256;
            const int r = p / (kStageK / 8), c = p - r * (kStageK / 8);
            if (p < kPieces) *reinterpret_cast<uint4 *>(&xs[r * kLdsRow + c * 8]) = xr[t];
        }
    };
    uint4 cw = make_uint4(0u, 0u, 0u, 0u), ms = cw, mm = cw;
    auto load_b = [&](int64_t kc) {
        const int64_t tile = kc * ng + g;
        cw = *reinterpret_cast<const uint4 *>(pc + (tile * 64 + lane) * 4);
        ms = *reinterpret_cast<const uint4 *>(pm + (tile * 4 + akq) * 8);
        mm = *reinterpret_cast<const uint4 *>(pm + (tile * 4 + akq) * 8 + 4);
    };
    if (c_begin < c_end) {
        load_x(c_begin);
        if (gvalid) load_b(c_begin);
    }

    for (int64_t cs = c_begin; cs < c_end; cs += kStageK / 32) {
        const int nst = (int)((c_end - cs) < (kStageK / 32) ? (c_end - cs) : (kStageK / 32));
        __syncthreads();
        store_x();
        __syncthreads();
        if (cs + kStageK / 32 < c_end) load_x(cs + kStageK / 32);
        if (!gvalid) continue;
        for (int sc = 0; sc < nst; ++sc) {
            const int64_t kc = cs + sc;
            const uint32_t S[4] = {ms.x, ms.y, ms.z, ms.w};
            const uint32_t Mn[4] = {mm.x, mm.y, mm.z, mm.w};
            const uint32_t W[4] = {cw.x, cw.y, cw.z, cw.w};
            if (kc + 1 < c_end) load_b(kc + 1);
            f16x8 bfrag[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t w = W[j], w8 = w >> 8;
                const uint32_t p0 = (w & 0x000F000Fu) | 0x64006400u;    // 1024 + q (k0, k1)
                const uint32_t p1 = (w & 0x00F000F0u) | 0x54005400u;    // 64 + q   (k2, k3)
                const uint32_t p2 = (w8 & 0x000F000Fu) | 0x64006400u;   // 1024 + q (k4, k5)
                const uint32_t p3 = (w8 & 0x00F000F0u) | 0x54005400u;   // 64 + q   (k6, k7)
                const f16x2 c01 = as_f16x2(p0) - f16x2{(_Float16)1024.0f, (_Float16)1024.0f};
                const f16x2 c23 = as_f16x2(p1) - f16x2{(_Float16)64.0f, (_Float16)64.0f};
                const f16x2 c45 = as_f16x2(p2) - f16x2{(_Float16)1024.0f, (_Float16)1024.0f};
                const f16x2 c67 = as_f16x2(p3) - f16x2{(_Float16)64.0f, (_Float16)64.0f};
                const f16x2 w01 = __builtin_elementwise_fma(c01, as_f16x2(S[0]), as_f16x2(Mn[0]));
                const f16x2 w23 = __builtin_elementwise_fma(c23, as_f16x2(S[1]), as_f16x2(Mn[1]));
                const f16x2 w45 = __builtin_elementwise_fma(c45, as_f16x2(S[2]), as_f16x2(Mn[2]));
                const f16x2 w67 = __builtin_elementwise_fma(c67, as_f16x2(S[3]), as_f16x2(Mn[3]));
                bfrag[j] = f16x8{w01.x, w01.y, w23.x, w23.y, w45.x, w45.y, w67.x, w67.y};
            }
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const f16x8 a = *reinterpret_cast<const f16x8 *>(&xs[(i * 16 + arow) * kLdsRow + sc * 32 + akq * 8]);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bfrag[j], acc[i][j], 0, 0, 0);
            }
        }
    }
    if (!gvalid) return;
    // ---- store: lane holds rows 4*(lane/16)+r, column lane%16 of each 16x16 tile
    const int crow = (lane >> 4) * 4, ccol = lane & 15;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + i * 16 + crow + r;
                if (row >= M) continue;
                const int64_t col = g * 64 + j * 16 + ccol;
                const float v = acc[i][j][r];
                if (ksplit > 1)
                    part[((int64_t)split * M + row) * N + col] = v;
                else if (y_f16)
                    static_cast<_Float16 *>(y)[(int64_t)row * N + col] = (_Float16)v;
                else
                    static_cast<float *>(y)[(int64_t)row * N + col] = v;
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
    dq_gemm_kernel<MT><<<grid, dim3(256), 0, stream>>>(x, M, K, N, pc, pm, cps, part, y, f16, ksplit);
}

}  // namespace

struct GemmPlan {
    int mt;              // 16-row tiles per M block
    int mblocks;
    int64_t nblocks;     // workgroups along N
    int ksplit;
    int chunks_per_split;
};

GemmPlan gemm_plan(int64_t M, int64_t K, int64_t N) {
    GemmPlan p{};
    const int64_t mt_needed = (M + 15) / 16;
    p.mt = (int)(mt_needed < 9 ? (mt_needed < 1 ? 1 : mt_needed) : 9);
    p.mblocks = (int)((M + 16 * p.mt - 1) / (16 * p.mt));
    p.nblocks = ((N / 64) + kWaves - 1) / kWaves;
    const int64_t nchunks = K / 32;
    // split K until the grid covers the CUs about twice, keeping >= 8 stages per split
    int ks = 1;
    const int64_t base = p.nblocks * (p.mblocks > 0 ? p.mblocks : 1);
    while (base * ks < 2 * kNumCU && nchunks / (ks * 2) >= 16) ks *= 2;
    p.ksplit = ks;
    int64_t cps = (nchunks + ks - 1) / ks;
    cps = ((cps + 1) / 2) * 2;                   // whole LDS stages
    p.chunks_per_split = (int)(cps > 0 ? cps : 2);
    p.ksplit = nchunks > 0 ? (int)((nchunks + p.chunks_per_split - 1) / p.chunks_per_split) : 1;
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
