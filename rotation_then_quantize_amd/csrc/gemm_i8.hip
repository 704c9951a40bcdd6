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

#include <algorithm>

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
constexpr int kBufferWord3 = 0x00020000;     // gfx9 buffer descriptor word 3 (raw, 32-bit dwords)
constexpr int kOutOfRange = 0x7ffffff0;      // byte offset past any descriptor range: loads 0

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
    extern __shared__ __attribute__((aligned(16))) int8_t lds[];   // [buf][A|W][kTileBytes], scales

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;

    // Persistent schedule: the tiles are split into 8 contiguous ranges, one per XCD; the blocks of
    // an XCD (block b runs on XCD b % 8) take its range round-robin.
    const int total = tiles_m * tiles_n;
    const int xcd = blockIdx.x % kXcds;
    const int stride = gridDim.x / kXcds;
    const int per = (total + kXcds - 1) / kXcds;
    const int lin_end = min((xcd + 1) * per, total);
    int lin = xcd * per + static_cast<int>(blockIdx.x / kXcds);
    if (lin >= lin_end) return;   // no tile for this block: before any barrier

    int64_t m0 = 0, n0 = 0;
    __amdgpu_buffer_rsrc_t rsa, rsw;
    // staging: chunk c = tid + 512*i covers tile row c / 8, 16-byte column c % 8; 4 chunks of A and
    // 4 of W per thread per stage (consecutive threads read consecutive 16 bytes of a row).  The
    // loads are buffer loads against descriptors that end at the tile's last valid row, so rows past
    // T or N (and K past d, sent to an offset beyond the range) read as zero without a branch.
    auto set_tile = [&](int l) {
        int tm, tn;
        tile_of(l, tiles_m, tiles_n, &tm, &tn);
        m0 = static_cast<int64_t>(tm) * BM;
        n0 = static_cast<int64_t>(tn) * BN;
        const int rows_a = static_cast<int>(min<int64_t>(BM, T - m0));
        const int rows_w = static_cast<int>(min<int64_t>(BN, N - n0));
        rsa = __builtin_amdgcn_make_buffer_rsrc((void*)(A + m0 * d), (short)0, rows_a * d, kBufferWord3);
        rsw = __builtin_amdgcn_make_buffer_rsrc((void*)(W + n0 * d), (short)0, rows_w * d, kBufferWord3);
    };
    constexpr int kLoads = BM * kChunks / kThreads;   // 4
    uint4 ra[kLoads], rb[kLoads];
    auto load_stage = [&](int k0) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int c = tid + i * kThreads;
            const int row = c >> 3, ch = c & 7;
            const int k = k0 + ch * 16;
            const int off = k < d ? row * d + k : kOutOfRange;
            const v4i va = __builtin_amdgcn_raw_buffer_load_b128(rsa, off, 0, 0);
            const v4i vw = __builtin_amdgcn_raw_buffer_load_b128(rsw, off, 0, 0);
            ra[i] = make_uint4(va.x, va.y, va.z, va.w);
            rb[i] = make_uint4(vw.x, vw.y, vw.z, vw.w);
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
    // The tile's token scales (threads 0-255) and output-row scales (threads 256-511), staged in LDS
    // behind the operand stages for the epilogue.
    float* s_as = reinterpret_cast<float*>(lds + 2 * 2 * kTileBytes);
    float* s_ws = s_as + BM;
    auto load_scale = [&]() -> float {
        if (kYKind == 2) return 0.0f;
        if (tid < BM) return m0 + tid < T ? a_scale[m0 + tid] : 0.0f;
        const int64_t n = n0 + (tid - BM);
        if (n >= N) return 0.0f;
        if (kWScaleBF16) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(w_scale)[n]) << 16);
        return static_cast<const float*>(w_scale)[n];
    };

    const int nk = (d + BK - 1) / BK;
    set_tile(lin);
    load_stage(0);
    float sc = load_scale();

    for (;;) {
    store_stage(0);
    if (kYKind != 2) s_as[tid] = sc;
    __syncthreads();

    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = v16i{};

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
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[j], fa[i], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) store_stage(buf ^ 1);
        __syncthreads();
    }

    // The next tile's first stage and scales are fetched now, so their latency (and the stores below)
    // overlap the epilogue; LDS is rewritten only after the epilogue's last barrier.
    const int64_t cm0 = m0, cn0 = n0;
    const int next = lin + stride;
    const bool more = next < lin_end;
    if (more) {
        set_tile(next);
        load_stage(0);
        sc = load_scale();
    }

    // ---- epilogue.  The MFMA computed the transposed tile (W fragment as the first operand), so a
    // lane holds D[n][t] at n = 8*(r/4) + 4*(lane/32) + r%4, t = lane % 32: four consecutive output
    // columns of one token row per group r/4.  Each wave scales its 128 x 64 block 32 token rows at a
    // time into its own LDS region (row pitch padded by 16 bytes against bank conflicts), then writes
    // it out row-contiguously: every 16-byte store lands in a 128- or 256-byte run of one Y row.
    constexpr int kOutBytes = kYKind == 1 ? 2 : 4;
    constexpr int kRowBytes = WN * kOutBytes;            // one wave's row segment
    constexpr int kPitch = kRowBytes + 16;
    constexpr int kPerChunk = 16 / kOutBytes;            // outputs per 16-byte store
    constexpr int kChunksPerRow = kRowBytes / 16;
    constexpr int kRowsPerPass = 64 / kChunksPerRow;
    int8_t* ep = lds + wave * (32 * kPitch);
    const bool vec_ok = (N % kPerChunk) == 0;
    const int tl = lane & 31;
    const int nq = (lane >> 5) * 4;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const float as = s_as[wm * WM + i * 32 + tl];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = j * 32 + 8 * g + nq;
                const int32_t a0 = acc[i][j][4 * g], a1 = acc[i][j][4 * g + 1];
                const int32_t a2 = acc[i][j][4 * g + 2], a3 = acc[i][j][4 * g + 3];
                int8_t* dst = ep + tl * kPitch + col * kOutBytes;
                if (kYKind == 2) {
                    *reinterpret_cast<int4*>(dst) = make_int4(a0, a1, a2, a3);
                } else {
                    const float4 ws = *reinterpret_cast<const float4*>(s_ws + wn * WN + col);
                    const float y0 = static_cast<float>(a0) * as * ws.x;
                    const float y1 = static_cast<float>(a1) * as * ws.y;
                    const float y2 = static_cast<float>(a2) * as * ws.z;
                    const float y3 = static_cast<float>(a3) * as * ws.w;
                    if (kYKind == 0)
                        *reinterpret_cast<float4*>(dst) = make_float4(y0, y1, y2, y3);
                    else
                        *reinterpret_cast<uint2*>(dst) = make_uint2(f32_to_bf16(y0) | (f32_to_bf16(y1) << 16),
                                                                    f32_to_bf16(y2) | (f32_to_bf16(y3) << 16));
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < 32 / kRowsPerPass; ++p) {
            const int row = p * kRowsPerPass + lane / kChunksPerRow;
            const int ch = lane % kChunksPerRow;
            const int64_t t = cm0 + wm * WM + i * 32 + row;
            const int64_t n = cn0 + wn * WN + ch * kPerChunk;
            if (t < T && n < N) {
                const uint4 v = *reinterpret_cast<const uint4*>(ep + row * kPitch + ch * 16);
                int8_t* yp = static_cast<int8_t*>(Y) + (t * N + n) * kOutBytes;
                if (vec_ok && n + kPerChunk <= N) {
                    // streaming store: Y is written once, and letting it allocate in the caches
                    // evicts the operand panels that later tiles re-read
                    __builtin_nontemporal_store(*reinterpret_cast<const v4i*>(&v), reinterpret_cast<v4i*>(yp));
                } else {
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < kPerChunk; ++e) {
                        if (n + e >= N) break;
                        if (kOutBytes == 4)
                            reinterpret_cast<uint32_t*>(yp)[e] = w[e];
                        else
                            reinterpret_cast<uint16_t*>(yp)[e] = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
                    }
                }
            }
        }
        __syncthreads();
    }
    if (!more) break;
    lin = next;
    }
}

}  // namespace

hipError_t launch_gemm_i8(const GemmI8Args& g, hipStream_t stream) {
    if (g.T <= 0 || g.N <= 0) return hipSuccess;
    if (g.d % 64 != 0) return hipErrorInvalidValue;
    constexpr size_t kLds = 2 * 2 * kTileBytes + (BM + BN) * sizeof(float);   // two stages of A and W + scales
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
    // persistent grid: one block per compute unit (the LDS allows one), a multiple of the XCD count,
    // and no more blocks than tiles (rounded up to that multiple)
    const int cus = device_cu_count();
    if (cus <= 0) return hipErrorInvalidDevice;
    const int64_t slots = std::max<int64_t>(kXcds, cus / kXcds * kXcds);
    const int64_t grid = std::min<int64_t>(slots, (total + kXcds - 1) / kXcds * kXcds);
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
