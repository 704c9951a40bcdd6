// gemm_i8.hip -- the W8A8 product in the rotated basis on gfx950 INT8 matrix cores.
//
//   acc[t][n] = sum_j qa[t][j] * qw[n][j]          (exact int32; the rotation has cancelled:
//                                                    OrbitQuant article, 2.2, W'x' = W Pi^T Pi x)
//   y[t][n]   = acc[t][n] * a_scale[t] * w_scale[n] (dequantisation s*q of both operands,
//                                                    cloud.baidu.com/article/9432521, 4)
//
// Both operands are K-contiguous (row-major [T][d] and [N][d]); v_mfma_i32_32x32x32_i8 takes, per
// lane, 16 consecutive K bytes of one row (lanes 0-31 the first 16 bytes of a 32-byte K step,
// lanes 32-63 the second), so a 16-byte chunk of a row is one lane's operand for either side.
//
// Tiling.  A workgroup of 8 waves (2 per SIMD) owns a 256 x 256 output tile; wave w computes rows
// 128*(w/4) .. +128 and columns 64*(w%4) .. +64 with v_mfma_i32_32x32x32_i8 (4 x 2 MFMA tiles,
// 128 int32 accumulators per lane in AGPRs).  Two waves share each SIMD, so one wave's MFMAs
// cover the other's LDS reads.  K advances in LDS stages of 128 bytes (4 MFMA steps), double
// buffered: the next stage's global loads are in flight while the current stage is multiplied.
// Per MFMA step a wave reads 4 A and 2 W fragments (6 KB of LDS) for 8 MFMAs.
// LDS rows are 128 bytes; 16-byte chunk c of row r sits at chunk c ^ f(r) with
// f(r) = ((r >> 1) & 7) ^ ((r & 1) << 2), which keeps fragment reads and staging writes free of
// bank conflicts whether the LDS has 32 or 64 four-byte banks.
//
// Order.  Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2), so the
// block index is remapped: the workgroups resident on one XCD cover a compact band of output
// tiles that share A rows and W rows in that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rtq_internal.h"

namespace rtq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;
constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 128;                       // bytes of K per LDS stage
constexpr int kChunks = BK / 16;              // 16-byte chunks per tile row per stage (8)
constexpr int WM = 128, WN = 64;              // per wave
constexpr int TM = WM / 32, TN = WN / 32;     // 4 x 2 MFMA tiles of 32 x 32
constexpr int kTileBytes = BM * BK;           // 32 KB per operand per stage
constexpr int kXcds = 8;

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ int swz(int row, int chunk) {
    const int f = ((row >> 1) & 7) ^ ((row & 1) << 2);
    return row * BK + ((chunk ^ f) << 4);
}

// Block index -> (tile_m, tile_n).  Blocks i and i + 8 land on the same XCD; each XCD walks its own
// contiguous range of tiles, ordered in bands of 8 N-tiles so concurrent blocks share panels.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int* tm, int* tn) {
    const int total = tiles_m * tiles_n;
    const int xcd = bid % kXcds;
    const int local = bid / kXcds;
    const int per = (total + kXcds - 1) / kXcds;
    const int lin = xcd * per + local;
    if (lin >= total) {  // padding blocks of the last round: no tile
        *tm = tiles_m;
        *tn = 0;
        return;
    }
    constexpr int kBand = 8;      // N-tiles per band
    const int band = lin / (kBand * tiles_m);
    const int in_band = lin % (kBand * tiles_m);
    const int band_w = min(kBand, tiles_n - band * kBand);
    *tm = in_band / band_w;
    *tn = band * kBand + in_band % band_w;
}

template <int kYKind, bool kWScaleBF16>
__global__ void __launch_bounds__(kThreads, 1)
gemm_i8_kernel(const int8_t* __restrict__ A, const float* __restrict__ a_scale, const int8_t* __restrict__ W,
               const void* __restrict__ w_scale, int64_t T, int64_t N, int d, void* __restrict__ Y,
               int tiles_m, int tiles_n) {
    extern __shared__ __attribute__((aligned(16))) int8_t lds[];   // [buf][A|W][kTileBytes]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    int tile_m, tile_n;
    tile_of(blockIdx.x, tiles_m, tiles_n, &tile_m, &tile_n);
    if (tile_m >= tiles_m || tile_n >= tiles_n) return;   // padding block: before any barrier
    const int64_t m0 = static_cast<int64_t>(tile_m) * BM;
    const int64_t n0 = static_cast<int64_t>(tile_n) * BN;

    // staging: chunk c = tid + 512*i covers tile row c / 8, 16-byte column c % 8; 4 chunks of A and
    // 4 of W per thread per stage (consecutive threads read consecutive 16 bytes of a row)
    constexpr int kLoads = BM * kChunks / kThreads;   // 4
    uint4 ra[kLoads], rb[kLoads];
    const bool full = (m0 + BM <= T) && (n0 + BN <= N);
    const bool kfull = (d % BK) == 0;

    auto load_stage = [&](int k0) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int c = tid + i * kThreads;
            const int row = c >> 3, ch = c & 7;
            const int k = k0 + ch * 16;
            const int64_t ga = m0 + row, gb = n0 + row;
            if (full && kfull) {
                ra[i] = *reinterpret_cast<const uint4*>(A + ga * d + k);
                rb[i] = *reinterpret_cast<const uint4*>(W + gb * d + k);
            } else {
                ra[i] = (ga < T && k < d) ? *reinterpret_cast<const uint4*>(A + ga * d + k) : make_uint4(0u, 0u, 0u, 0u);
                rb[i] = (gb < N && k < d) ? *reinterpret_cast<const uint4*>(W + gb * d + k) : make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };
    auto store_stage = [&](int buf) {
        int8_t* la = lds + buf * 2 * kTileBytes;
        int8_t* lb = la + kTileBytes;
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int c = tid + i * kThreads;
            const int row = c >> 3, ch = c & 7;
            *reinterpret_cast<uint4*>(la + swz(row, ch)) = ra[i];
            *reinterpret_cast<uint4*>(lb + swz(row, ch)) = rb[i];
        }
    };

    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = v16i{};

    const int nk = (d + BK - 1) / BK;
    load_stage(0);
    store_stage(0);
    __syncthreads();

    const int frow = lane & 31;   // row (A) / column (W) inside a 32x32 tile
    const int fk = lane >> 5;     // which 16-byte half of the 32-byte MFMA K step

    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        const int8_t* la = lds + buf * 2 * kTileBytes;
        const int8_t* lb = la + kTileBytes;
        if (kt + 1 < nk) load_stage((kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            v4i fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                fa[i] = *reinterpret_cast<const v4i*>(la + swz(wm * WM + i * 32 + frow, 2 * ks + fk));
#pragma unroll
            for (int j = 0; j < TN; ++j)
                fb[j] = *reinterpret_cast<const v4i*>(lb + swz(wn * WN + j * 32 + frow, 2 * ks + fk));
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) store_stage(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: for a 32x32 tile, lane holds D[8*(r/4) + 4*(lane/32) + r%4][lane % 32]
    const int ocol = lane & 31;
    const int orow = (lane >> 5) * 4;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + wn * WN + j * 32 + ocol;
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
            for (int r = 0; r < 16; ++r) {
                const int64_t t = m0 + wm * WM + i * 32 + 8 * (r >> 2) + orow + (r & 3);
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
    if (g.d % 64 != 0) return hipErrorInvalidValue;
    constexpr size_t kLds = 2 * 2 * kTileBytes;   // 128 KB: two stages of A and W
    static const hipError_t attr_err = [] {
        hipError_t e = hipSuccess;
        for (const void* k : {reinterpret_cast<const void*>(gemm_i8_kernel<0, true>),
                              reinterpret_cast<const void*>(gemm_i8_kernel<1, true>),
                              reinterpret_cast<const void*>(gemm_i8_kernel<2, true>),
                              reinterpret_cast<const void*>(gemm_i8_kernel<0, false>),
                              reinterpret_cast<const void*>(gemm_i8_kernel<1, false>),
                              reinterpret_cast<const void*>(gemm_i8_kernel<2, false>)}) {
            const hipError_t r = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLds));
            if (r != hipSuccess) e = r;
        }
        return e;
    }();
    if (attr_err != hipSuccess) return attr_err;
    const int64_t tiles_m = (g.T + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
    const int64_t total = tiles_m * tiles_n;
    if (total > (int64_t(1) << 30)) return hipErrorInvalidValue;
    // round the grid up to a multiple of the XCD count so every XCD gets the same share
    const int64_t grid = (total + kXcds - 1) / kXcds * kXcds;
#define RTQ_LAUNCH(YK, WB)                                                                                   \
    hipLaunchKernelGGL((gemm_i8_kernel<YK, WB>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), kLds, stream,  \
                       g.a, g.a_scale, g.w, g.w_scale, g.T, g.N, g.d, g.y, static_cast<int>(tiles_m),          \
                       static_cast<int>(tiles_n))
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
