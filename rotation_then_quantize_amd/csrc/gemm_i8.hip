// gemm_i8.hip -- the W8A8 product in the rotated basis on gfx950 INT8 matrix cores.
//
//   acc[t][n] = sum_j qa[t][j] * qw[n][j]          (exact int32; the rotation has cancelled:
//                                                    OrbitQuant article, 2.2, W'x' = W Pi^T Pi x)
//   y[t][n]   = acc[t][n] * a_scale[t] * w_scale[n] (dequantisation s*q of both operands,
//                                                    cloud.baidu.com/article/9432521, 4)
//
// Both operands are K-contiguous (row-major [T][d] and [N][d]), so each 16-byte chunk of a row is
// exactly one lane's operand of v_mfma_i32_16x16x64_i8 for either side.
// Tiling: 256 threads = 4 waves in a 2x2 grid; workgroup tile BM x BN, wave tile (BM/2) x (BN/2)
// built from 16x16 MFMA tiles; K staged BK bytes at a time through double-buffered LDS whose
// 16-byte chunks are XOR-swizzled by row (chunk ^ (row & 7)) so fragment reads are conflict-free.
// The epilogue converts the exact int32 accumulators to fp32 and applies both scales.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rtq_internal.h"

namespace rtq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 128;                       // bytes of K per LDS stage
constexpr int kChunksPerRow = BK / 16;        // 8
constexpr int WM = BM / 2, WN = BN / 2;       // wave tile
constexpr int TM = WM / 16, TN = WN / 16;     // MFMA tiles per wave
constexpr int kTileBytes = BM * BK;           // A (and B) bytes per stage

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 4); }

template <int kYKind, bool kWScaleBF16>
__global__ void __launch_bounds__(kThreads)
gemm_i8_kernel(const int8_t* __restrict__ A, const float* __restrict__ a_scale, const int8_t* __restrict__ W,
               const void* __restrict__ w_scale, int64_t T, int64_t N, int d, void* __restrict__ Y) {
    __shared__ __attribute__((aligned(16))) int8_t lds[2][2][kTileBytes];  // [buf][A|B]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * BN;

    // global -> register staging: each thread moves 4 chunks of A and 4 of B per stage
    constexpr int kLoads = BM * kChunksPerRow / kThreads;
    uint4 ra[kLoads], rb[kLoads];

    auto load_stage = [&](int k0) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int c = tid + i * kThreads;
            const int row = c / kChunksPerRow, ch = c % kChunksPerRow;
            const int k = k0 + ch * 16;
            const int64_t ga = m0 + row, gb = n0 + row;
            ra[i] = (ga < T && k < d) ? *reinterpret_cast<const uint4*>(A + ga * d + k) : make_uint4(0u, 0u, 0u, 0u);
            rb[i] = (gb < N && k < d) ? *reinterpret_cast<const uint4*>(W + gb * d + k) : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int c = tid + i * kThreads;
            const int row = c / kChunksPerRow, ch = c % kChunksPerRow;
            *reinterpret_cast<uint4*>(&lds[buf][0][swz(row, ch)]) = ra[i];
            *reinterpret_cast<uint4*>(&lds[buf][1][swz(row, ch)]) = rb[i];
        }
    };

    v4i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    const int nk = (d + BK - 1) / BK;
    load_stage(0);
    store_stage(0);
    __syncthreads();

    const int frow = lane & 15;   // row (A) / column (B) inside a 16x16 tile
    const int fk = lane >> 4;     // which 16-byte K slice of the 64-deep MFMA step

    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_stage((kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 64; ++ks) {
            v4i fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm * WM + i * 16 + frow;
                fa[i] = *reinterpret_cast<const v4i*>(&lds[buf][0][swz(row, ks * 4 + fk)]);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = wn * WN + j * 16 + frow;
                fb[j] = *reinterpret_cast<const v4i*>(&lds[buf][1][swz(row, ks * 4 + fk)]);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) store_stage(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds D[4*(lane/16) + r][lane % 16] of each 16x16 tile
    const int ocol = lane & 15;
    const int orow = (lane >> 4) * 4;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + wn * WN + j * 16 + ocol;
        if (n >= N) continue;
        float ws = 1.0f;
        if (kYKind != 2) {
            if (kWScaleBF16)
                ws = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(w_scale)[n]) << 16);
            else
                ws = static_cast<const float*>(w_scale)[n];
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t t = m0 + wm * WM + i * 16 + orow + r;
                if (t >= T) continue;
                const int32_t a = acc[i][j][r];
                if (kYKind == 2) {
                    static_cast<int32_t*>(Y)[t * N + n] = a;
                } else {
                    const float y = static_cast<float>(a) * a_scale[t] * ws;
                    if (kYKind == 0)
                        static_cast<float*>(Y)[t * N + n] = y;
                    else
                        static_cast<uint16_t*>(Y)[t * N + n] = static_cast<uint16_t>(f32_to_bf16(y));
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_i8(const GemmI8Args& g, hipStream_t stream) {
    if (g.T <= 0 || g.N <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((g.N + BN - 1) / BN), static_cast<unsigned>((g.T + BM - 1) / BM));
    if (grid.y > 65535u) return hipErrorInvalidValue;
#define RTQ_LAUNCH(YK, WB)                                                                                   \
    hipLaunchKernelGGL((gemm_i8_kernel<YK, WB>), grid, dim3(kThreads), 0, stream, g.a, g.a_scale, g.w,       \
                       g.w_scale, g.T, g.N, g.d, g.y)
    if (g.w_scale_bf16) {
        if (g.y_kind == 0) RTQ_LAUNCH(0, true);
        else if (g.y_kind == 1) RTQ_LAUNCH(1, true);
        else RTQ_LAUNCH(2, true);
    } else {
        if (g.y_kind == 0) RTQ_LAUNCH(0, false);
        else if (g.y_kind == 1) RTQ_LAUNCH(1, false);
        else RTQ_LAUNCH(2, false);
    }
#undef RTQ_LAUNCH
    return hipGetLastError();
}

}  // namespace rtq
