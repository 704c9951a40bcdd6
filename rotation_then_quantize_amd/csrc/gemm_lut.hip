// gemm_lut.hip -- the W4A4 / W2A4 product of Lloyd-Max codes on gfx950 fp16 matrix cores.
//
//   y[t][n] = r[n] * s[t] * sum_j c_w[qw[n][j]] * c_a[qa[t][j]]
// with x_hat' = s * Q(x'/s) and w_hat' = r * Q(w'/r) (OrbitQuant article, 2.1 step 4 and 2.2
// step 5); the rotation has cancelled (2.2), so the product runs directly on the codes.
//
// The codes are decoded while a K-slice is staged into LDS: each packed byte indexes a 256-entry
// LDS table holding the fp16 centroids of every code in that byte (two for 4-bit codes, four for
// 2-bit codes), so one LDS read decodes a whole byte.  The centroids are scaled by 2^e ~ sqrt(d)
// (an exact power of two) before rounding to fp16, which keeps them in fp16's full-precision
// range for any d; the epilogue multiplies by 2^-2e.  Accumulation is fp32 in the MFMA.
// Tiling mirrors the INT8 kernel: 256 threads, 2x2 waves, 128x128 tile, 64 K-elements
// (128 bytes of fp16) per double-buffered LDS stage with XOR-swizzled 16-byte chunks.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "rtq_internal.h"

namespace rtq {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BKE = 64;                       // K elements per stage
constexpr int kRowBytes = BKE * 2;            // fp16 bytes per tile row per stage
constexpr int WM = BM / 2, WN = BN / 2;
constexpr int TM = WM / 16, TN = WN / 16;
constexpr int kTileBytes = BM * kRowBytes;

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ uint32_t half_bits(float v) {
    return static_cast<uint32_t>(__half_as_ushort(__float2half_rn(v)));
}

template <int kBitsW, int kYKind, bool kWScaleBF16>
__global__ void __launch_bounds__(kThreads)
gemm_lut_kernel(const uint8_t* __restrict__ A, const float* __restrict__ a_scale, const uint8_t* __restrict__ W,
                const void* __restrict__ w_scale, const float* __restrict__ ca, const float* __restrict__ cw,
                int64_t T, int64_t N, int d, float lut_scale, float out_scale, void* __restrict__ Y) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kTileBytes];
    __shared__ uint32_t lut_a[256];                    // byte of two 4-bit codes -> two fp16
    __shared__ uint2 lut_w[256];                       // byte -> two (4-bit) or four (2-bit) fp16

    const int tid = threadIdx.x;
    {
        const int b = tid;  // 256 threads, one table entry each
        lut_a[b] = half_bits(ca[b & 15] * lut_scale) | (half_bits(ca[b >> 4] * lut_scale) << 16);
        if (kBitsW == 4) {
            lut_w[b] = make_uint2(half_bits(cw[b & 15] * lut_scale) | (half_bits(cw[b >> 4] * lut_scale) << 16), 0u);
        } else {
            lut_w[b] = make_uint2(half_bits(cw[b & 3] * lut_scale) | (half_bits(cw[(b >> 2) & 3] * lut_scale) << 16),
                                  half_bits(cw[(b >> 4) & 3] * lut_scale) | (half_bits(cw[b >> 6] * lut_scale) << 16));
        }
    }

    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * BN;
    const int64_t a_row_bytes = d / 2;
    const int64_t w_row_bytes = static_cast<int64_t>(d) * kBitsW / 8;

    // staging: thread t covers 32 K-elements of tile row t/2 (half t%2) for both operands
    const int srow = tid >> 1, shalf = tid & 1;
    uint4 ra;                                    // 16 bytes = 32 four-bit codes
    uint4 rb;                                    // 16 bytes (4-bit) or 8 bytes (2-bit, in .x/.y)
    auto load_stage = [&](int k0) {
        const int64_t ga = m0 + srow, gb = n0 + srow;
        const int ke = k0 + shalf * 32;
        ra = ga < T ? *reinterpret_cast<const uint4*>(A + ga * a_row_bytes + ke / 2) : make_uint4(0u, 0u, 0u, 0u);
        if (kBitsW == 4) {
            rb = gb < N ? *reinterpret_cast<const uint4*>(W + gb * w_row_bytes + ke / 2) : make_uint4(0u, 0u, 0u, 0u);
        } else {
            const uint2 v = gb < N ? *reinterpret_cast<const uint2*>(W + gb * w_row_bytes + ke / 4) : make_uint2(0u, 0u);
            rb = make_uint4(v.x, v.y, 0u, 0u);
        }
    };
    auto store_stage = [&](int buf) {
        uint32_t out[16];
        const uint32_t in_a[4] = {ra.x, ra.y, ra.z, ra.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int b = 0; b < 4; ++b) out[q * 4 + b] = lut_a[(in_a[q] >> (8 * b)) & 0xffu];
#pragma unroll
        for (int c = 0; c < 4; ++c)
            *reinterpret_cast<uint4*>(&lds[buf][0][swz(srow, shalf * 4 + c)]) =
                make_uint4(out[4 * c], out[4 * c + 1], out[4 * c + 2], out[4 * c + 3]);
        if (kBitsW == 4) {
            const uint32_t in_b[4] = {rb.x, rb.y, rb.z, rb.w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int b = 0; b < 4; ++b) out[q * 4 + b] = lut_w[(in_b[q] >> (8 * b)) & 0xffu].x;
        } else {
            const uint32_t in_b[2] = {rb.x, rb.y};
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint2 e = lut_w[(in_b[q] >> (8 * b)) & 0xffu];
                    out[q * 8 + 2 * b] = e.x;
                    out[q * 8 + 2 * b + 1] = e.y;
                }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
            *reinterpret_cast<uint4*>(&lds[buf][1][swz(srow, shalf * 4 + c)]) =
                make_uint4(out[4 * c], out[4 * c + 1], out[4 * c + 2], out[4 * c + 3]);
    };

    v4f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int nk = d / BKE;
    __syncthreads();  // tables ready
    load_stage(0);
    store_stage(0);
    __syncthreads();

    const int frow = lane & 15;
    const int fk = lane >> 4;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_stage((kt + 1) * BKE);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            v8h fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                fa[i] = *reinterpret_cast<const v8h*>(&lds[buf][0][swz(wm * WM + i * 16 + frow, ks * 4 + fk)]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                fb[j] = *reinterpret_cast<const v8h*>(&lds[buf][1][swz(wn * WN + j * 16 + frow, ks * 4 + fk)]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) store_stage(buf ^ 1);
        __syncthreads();
    }

    const int ocol = lane & 15;
    const int orow = (lane >> 4) * 4;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + wn * WN + j * 16 + ocol;
        if (n >= N) continue;
        float ws;
        if (kWScaleBF16)
            ws = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(w_scale)[n]) << 16);
        else
            ws = static_cast<const float*>(w_scale)[n];
        ws *= out_scale;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t t = m0 + wm * WM + i * 16 + orow + r;
                if (t >= T) continue;
                const float y = acc[i][j][r] * ws * a_scale[t];
                if (kYKind == 0)
                    static_cast<float*>(Y)[t * N + n] = y;
                else
                    static_cast<uint16_t*>(Y)[t * N + n] = static_cast<uint16_t>(f32_to_bf16(y));
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_lut(const GemmLutArgs& g, hipStream_t stream) {
    if (g.T <= 0 || g.N <= 0) return hipSuccess;
    // 2^e closest to sqrt(d): centroids for N(0, 1/d) become O(1) before the fp16 rounding.
    const int e = static_cast<int>(lround(0.5 * log2(static_cast<double>(g.d))));
    const float lut_scale = ldexpf(1.0f, e);
    const float out_scale = ldexpf(1.0f, -2 * e);
    const dim3 grid(static_cast<unsigned>((g.N + BN - 1) / BN), static_cast<unsigned>((g.T + BM - 1) / BM));
    if (grid.y > 65535u) return hipErrorInvalidValue;
#define RTQ_LAUNCH(BW, YK, WB)                                                                                 \
    hipLaunchKernelGGL((gemm_lut_kernel<BW, YK, WB>), grid, dim3(kThreads), 0, stream, g.a, g.a_scale, g.w,    \
                       g.w_scale, g.ca, g.cw, g.T, g.N, g.d, lut_scale, out_scale, g.y)
    if (g.bits_w == 4) {
        if (g.w_scale_bf16) {
            if (g.y_kind == 0) RTQ_LAUNCH(4, 0, true); else RTQ_LAUNCH(4, 1, true);
        } else {
            if (g.y_kind == 0) RTQ_LAUNCH(4, 0, false); else RTQ_LAUNCH(4, 1, false);
        }
    } else {
        if (g.w_scale_bf16) {
            if (g.y_kind == 0) RTQ_LAUNCH(2, 0, true); else RTQ_LAUNCH(2, 1, true);
        } else {
            if (g.y_kind == 0) RTQ_LAUNCH(2, 0, false); else RTQ_LAUNCH(2, 1, false);
        }
    }
#undef RTQ_LAUNCH
    return hipGetLastError();
}

}  // namespace rtq
