// rpbh_rows.hip -- the fused RPBH rotate + per-row quantise kernel for gfx950.
//
// Computes, for every row v of x (a token online, a weight row offline):
//   v' = Pi_d v,  Pi_d = blkdiag(H_64 D_1, ..., H_64 D_{d/64}) P_pi     (OrbitQuant article, 2.3)
// then one of
//   - the rotated row itself (fp32 / bf16),
//   - symmetric INT8: s = max|v'|/127, q = rne(v'/s)        (cloud.baidu.com/article/9432521, 4)
//   - Lloyd-Max codes of v'/(||v'|| + eps), packed 4- or 2-bit, plus the norm
//                                                          (OrbitQuant article, 2.1 and 2.2)
//
// Work decomposition.  A 256-thread workgroup stages 256*64 = 16384 elements at a time (a
// "group" of 16384/d whole rows) in LDS.  Lane l owns Hadamard block (l mod d/64) of row
// (l / (d/64)) of the group and holds that block's 64 values in registers, so all six butterfly
// stages of the 64-point transform run in-register with no cross-lane traffic.
//   1. Coalesced 16-byte loads of the rows into LDS.  The Rademacher signs are applied here, on
//      the source side: element k is flipped by the sign of the output slot it is gathered into
//      (sign[j] with perm[j] == k); the XOR masks for that live in LDS, built once per workgroup.
//   2. Each lane gathers its 64 inputs through perm (addresses precomputed once per workgroup).
//   3. FWHT-64 in fp64.  With bf16 inputs (8 significant bits) every partial sum of a block is
//      exact in fp64 while the block's magnitudes span at most 2^39, so after the single rounding
//      to fp32 the rotated value is the correctly rounded Pi v -- identical to a dense product
//      accumulated exactly.  The 1/8 normalisation is folded into the scale (exact power of two),
//      so the registers hold 8*v'.
//   4. Row reduction (max |v'| or sum v'^2 in fp64) across the d/64 lanes of the row: xor
//      shuffles inside a wave, LDS across waves.
//   5. Quantise, pack, and store 16-byte vectors.
// The workgroups are persistent (grid = what fits on the chip), so the per-workgroup set-up
// (sign masks, gather addresses) is paid once per workgroup, not once per group.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codebook_int8.h"
#include "rtq_internal.h"

namespace rtq {
namespace {

constexpr int kThreads = 256;
constexpr int kH = 64;                       // Walsh-Hadamard block size
constexpr int kGroup = kThreads * kH;        // elements staged per workgroup iteration
constexpr int kRedBytes = 256;               // cross-wave reduction scratch

__device__ __forceinline__ float bf16_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// y = H_64 v in natural (Sylvester) order: radix-2 butterflies, spans 1..32.
__device__ __forceinline__ void fwht64(double (&v)[kH]) {
#pragma unroll
    for (int span = 1; span < kH; span <<= 1) {
#pragma unroll
        for (int i = 0; i < kH; i += 2 * span) {
#pragma unroll
            for (int j = i; j < i + span; ++j) {
                const double a = v[j], b = v[j + span];
                v[j] = a + b;
                v[j + span] = a - b;
            }
        }
    }
}

struct MaxOp {
    __device__ double operator()(double a, double b) const { return fmax(a, b); }
};
struct SumOp {
    __device__ double operator()(double a, double b) const { return a + b; }
};

// Combine v over the nb = 2^log2nb consecutive lanes that hold one row.  Every thread of the
// workgroup must call this (it may contain barriers).  The result is returned to all lanes.
template <typename Op>
__device__ __forceinline__ double row_reduce(double v, int log2nb, double* red, Op op) {
    const int wave_steps = log2nb < 6 ? log2nb : 6;
    for (int s = 0; s < wave_steps; ++s) v = op(v, __shfl_xor(v, 1 << s));
    if (log2nb > 6) {
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) red[wave] = v;
        __syncthreads();
        const int wpr = 1 << (log2nb - 6);
        const int w0 = wave & ~(wpr - 1);
        double acc = red[w0];
        for (int i = 1; i < wpr; ++i) acc = op(acc, red[w0 + i]);
        v = acc;
        __syncthreads();
    }
    return v;
}

template <bool kBF16In, bool kRotate, int kOut>
__global__ void __launch_bounds__(kThreads)
rpbh_rows_kernel(const void* __restrict__ xin, int64_t rows, int d, int log2d, int log2nb,
                 const int32_t* __restrict__ perm, const int8_t* __restrict__ signs, void* __restrict__ out,
                 void* __restrict__ scale_out, int scale_bf16, const float* __restrict__ bounds, float eps,
                 const float* __restrict__ cent, int tiled) {
    constexpr int ES = kBF16In ? 2 : 4;
    // codebook outputs: kRowCode* pack the codes, kRowLut* write each code's int8 codebook value
    constexpr bool k4 = kOut == kRowCode4 || kOut == kRowLut4;
    constexpr bool kLut = kOut == kRowLut4 || kOut == kRowLut2;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned char* rowbuf = smem;                          // kGroup elements
    unsigned char* maskbuf = smem + kGroup * ES;           // d sign masks (source order)
    double* red = reinterpret_cast<double*>(smem + kGroup * ES + d * ES);

    const int tid = threadIdx.x;
    const int nb = 1 << log2nb;
    const int rpg = kThreads >> log2nb;                    // rows per group
    const int rg = tid >> log2nb;                          // my row inside the group
    const int blk = tid & (nb - 1);                        // my Hadamard block inside the row
    const uint32_t dmask = static_cast<uint32_t>(d - 1);

    // ---- once per workgroup: source-side sign masks and gather addresses
    uint32_t addr[kH];
    if (kRotate) {
        for (int j = tid; j < d; j += kThreads) {
            const uint32_t p = static_cast<uint32_t>(perm[j]) & dmask;
            const bool neg = signs[j] < 0;
            if (kBF16In)
                reinterpret_cast<uint16_t*>(maskbuf)[p] = neg ? 0x8000u : 0u;
            else
                reinterpret_cast<uint32_t*>(maskbuf)[p] = neg ? 0x80000000u : 0u;
        }
        const int4* pp = reinterpret_cast<const int4*>(perm + blk * kH);
#pragma unroll
        for (int q = 0; q < kH / 4; ++q) {
            const int4 v = pp[q];
            const uint32_t base = static_cast<uint32_t>(rg) << log2d;
            addr[4 * q + 0] = (base + (static_cast<uint32_t>(v.x) & dmask)) * ES;
            addr[4 * q + 1] = (base + (static_cast<uint32_t>(v.y) & dmask)) * ES;
            addr[4 * q + 2] = (base + (static_cast<uint32_t>(v.z) & dmask)) * ES;
            addr[4 * q + 3] = (base + (static_cast<uint32_t>(v.w) & dmask)) * ES;
        }
    } else {
        for (int j = tid; j < d; j += kThreads) {
            if (kBF16In)
                reinterpret_cast<uint16_t*>(maskbuf)[j] = 0u;
            else
                reinterpret_cast<uint32_t*>(maskbuf)[j] = 0u;
        }
#pragma unroll
        for (int b = 0; b < kH; ++b) addr[b] = ((static_cast<uint32_t>(rg) << log2d) + blk * kH + b) * ES;
    }
    float tb[15];
    constexpr int kNB = k4 ? 15 : ((kOut == kRowCode2 || kOut == kRowLut2) ? 3 : 0);
#pragma unroll
    for (int k = 0; k < kNB; ++k) tb[k] = bounds[k];
    uint32_t lut[4] = {0u, 0u, 0u, 0u};
    if (kLut) codebook_int8_table(cent, kNB + 1, codebook_int8_scale(cent, kNB + 1), lut);
    __syncthreads();

    const int64_t ngroups = (rows + rpg - 1) / rpg;
    constexpr int kChunks = kGroup * ES / 16;              // 16-byte chunks per group
    const unsigned char* xb = static_cast<const unsigned char*>(xin);

    for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
        const int64_t row0 = g * rpg;
        // ---- 1. stage the group's rows (coalesced), source-side signs applied
#pragma unroll 4
        for (int c = tid; c < kChunks; c += kThreads) {
            const int e = c * (16 / ES);
            const int r = e >> log2d;
            const int col = e & static_cast<int>(dmask);
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (row0 + r < rows)
                v = *reinterpret_cast<const uint4*>(xb + ((row0 + r) * static_cast<int64_t>(d) + col) * ES);
            const uint4 m = *reinterpret_cast<const uint4*>(maskbuf + col * ES);
            v.x ^= m.x;
            v.y ^= m.y;
            v.z ^= m.z;
            v.w ^= m.w;
            *reinterpret_cast<uint4*>(rowbuf + e * ES) = v;
        }
        __syncthreads();

        // ---- 2. gather my block, 3. transform (registers hold 8 * v')
        double acc[kH];
#pragma unroll
        for (int b = 0; b < kH; ++b) {
            float f;
            if (kBF16In)
                f = bf16_to_f32(*reinterpret_cast<const uint16_t*>(rowbuf + addr[b]));
            else
                f = *reinterpret_cast<const float*>(rowbuf + addr[b]);
            acc[b] = static_cast<double>(f);
        }
        __syncthreads();  // the next iteration may overwrite rowbuf
        if (kRotate) {
            fwht64(acc);
        } else {
#pragma unroll
            for (int b = 0; b < kH; ++b) acc[b] *= 8.0;
        }

        const int64_t row = row0 + rg;
        const bool valid = row < rows;

        if (kOut == kRowRotF32 || kOut == kRowRotBF16) {
            if (valid) {
                if (kOut == kRowRotF32) {
                    float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + row * d + blk * kH);
#pragma unroll
                    for (int q = 0; q < kH / 4; ++q)
                        o[q] = make_float4(static_cast<float>(acc[4 * q] * 0.125),
                                           static_cast<float>(acc[4 * q + 1] * 0.125),
                                           static_cast<float>(acc[4 * q + 2] * 0.125),
                                           static_cast<float>(acc[4 * q + 3] * 0.125));
                } else {
                    uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + row * d + blk * kH);
#pragma unroll
                    for (int q = 0; q < kH / 8; ++q) {
                        uint32_t w[4];
#pragma unroll
                        for (int p = 0; p < 4; ++p) {
                            const uint32_t lo = f32_to_bf16(static_cast<float>(acc[8 * q + 2 * p] * 0.125));
                            const uint32_t hi = f32_to_bf16(static_cast<float>(acc[8 * q + 2 * p + 1] * 0.125));
                            w[p] = lo | (hi << 16);
                        }
                        o[q] = make_uint4(w[0], w[1], w[2], w[3]);
                    }
                }
            }
            continue;
        }

        if (kOut == kRowInt8) {
            // s = fl32( fl32(max|8v'| / 8) / 127 ); codes q = rne(v' / s_stored).
            double m = 0.0;
#pragma unroll
            for (int b = 0; b < kH; ++b) m = fmax(m, fabs(acc[b]));
            m = row_reduce(m, log2nb, red, MaxOp());
            const float amax = static_cast<float>(m * 0.125);
            float s = amax / 127.0f;
            if (scale_bf16) s = bf16_to_f32(f32_to_bf16(s));
            // Fast form: v'/s == fl32(8v') / (8s) whenever v' is a normal fp32 number; when the
            // row's maximum is >= 2^-100 any subnormal v' maps to code 0 either way.
            const bool fast = m >= 0x1p-100;
            const float s8 = s * 8.0f;
            uint32_t w[kH / 4];
#pragma unroll
            for (int q = 0; q < kH / 4; ++q) w[q] = 0u;
            if (s != 0.0f) {
#pragma unroll
                for (int b = 0; b < kH; ++b) {
                    float t;
                    if (fast)
                        t = static_cast<float>(acc[b]) / s8;
                    else
                        t = static_cast<float>(acc[b] * 0.125) / s;
                    float r = rintf(t);
                    r = fminf(fmaxf(r, -127.0f), 127.0f);
                    const uint32_t byte = static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xffu;
                    w[b >> 2] |= byte << ((b & 3) * 8);
                }
            }
            if (valid) {
                if (tiled) {
                    int8_t* o = static_cast<int8_t*>(out) + tiled_slot_offset(row, blk, d);
#pragma unroll
                    for (int q = 0; q < kH / 16; ++q)
                        *reinterpret_cast<uint4*>(o + 16 * tiled_chunk(row, q)) =
                            make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
                } else {
                    uint4* o = reinterpret_cast<uint4*>(static_cast<int8_t*>(out) + row * d + blk * kH);
#pragma unroll
                    for (int q = 0; q < kH / 16; ++q) o[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
                }
                if (blk == 0) {
                    if (scale_bf16)
                        static_cast<uint16_t*>(scale_out)[row] = static_cast<uint16_t>(f32_to_bf16(s));
                    else
                        static_cast<float*>(scale_out)[row] = s;
                }
            }
            continue;
        }

        // ---- codebook: s = ||v'||, u = v' / (s + eps), code = #{k : t_k < u}
        {
            double ss = 0.0;
#pragma unroll
            for (int b = 0; b < kH; ++b) {
                const double f = static_cast<double>(static_cast<float>(acc[b]));
                ss += f * f;
            }
            ss = row_reduce(ss, log2nb, red, SumOp());
            const float s = static_cast<float>(sqrt(ss) * 0.125);
            const float den = (eps == 0.0f) ? s : s + eps;
            const bool fast = s >= 0x1p-100f;
            const float den8 = den * 8.0f;
            constexpr int kBits = k4 ? 4 : 2;
            constexpr int kSlot = kLut ? 8 : kBits;      // bits per code in the output words
            constexpr int kPerWord = 32 / kSlot;
            uint32_t w[kH / kPerWord];
#pragma unroll
            for (int q = 0; q < kH / kPerWord; ++q) w[q] = 0u;
#pragma unroll
            for (int b = 0; b < kH; ++b) {
                float u = 0.0f;
                if (den != 0.0f) {
                    if (fast)
                        u = static_cast<float>(acc[b]) / den8;
                    else
                        u = static_cast<float>(acc[b] * 0.125) / den;
                }
                uint32_t code = 0;
#pragma unroll
                for (int k = 0; k < kNB; ++k) code += (tb[k] < u) ? 1u : 0u;
                w[b / kPerWord] |= code << ((b % kPerWord) * kSlot);
            }
            if (kLut) {
#pragma unroll
                for (int q = 0; q < kH / kPerWord; ++q) w[q] = k4 ? lut16_x4(lut, w[q]) : lut4_x4(lut, w[q]);
            }
            if (valid && tiled) {
                if (kLut) {   // int8 values in the INT8 tiled layout
                    int8_t* o = static_cast<int8_t*>(out) + tiled_slot_offset(row, blk, d);
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<uint4*>(o + 16 * tiled_chunk(row, q)) =
                            make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
                } else {      // packed codes in the tiled code layout
                    uint4* o = reinterpret_cast<uint4*>(static_cast<uint8_t*>(out) + tiled_code_offset(row, blk, d, kBits));
                    o[0] = make_uint4(w[0], w[1], w[2], w[3]);
                    if (kBits == 4) o[1] = make_uint4(w[4], w[5], w[6], w[7]);
                }
            } else if (valid) {
                uint32_t* o = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(out) + (row * d + blk * kH) * kSlot / 8);
                if (kLut) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        reinterpret_cast<uint4*>(o)[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
                } else if (kBits == 4) {
                    reinterpret_cast<uint4*>(o)[0] = make_uint4(w[0], w[1], w[2], w[3]);
                    reinterpret_cast<uint4*>(o)[1] = make_uint4(w[4], w[5], w[6], w[7]);
                } else {
                    reinterpret_cast<uint4*>(o)[0] = make_uint4(w[0], w[1], w[2], w[3]);
                }
            }
            if (valid && blk == 0) {
                if (scale_bf16)
                    static_cast<uint16_t*>(scale_out)[row] = static_cast<uint16_t>(f32_to_bf16(s));
                else
                    static_cast<float*>(scale_out)[row] = s;
            }
        }
    }
}

// x = Pi^T y:  x[perm[j]] = sign[j] * (H_64 y_block)_j / 8.  Used to check Pi^T Pi = I on the device
// and by callers that need to leave the rotated basis; not on the inference path.
template <bool kBF16In, bool kBF16Out>
__global__ void __launch_bounds__(kThreads)
rpbh_inverse_kernel(const void* __restrict__ yin, int64_t rows, int d, int log2d, int log2nb,
                    const int32_t* __restrict__ perm, const int8_t* __restrict__ signs, void* __restrict__ xout) {
    constexpr int ES = kBF16In ? 2 : 4;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    float* outbuf = reinterpret_cast<float*>(smem);                      // kGroup fp32
    unsigned char* inbuf = smem + kGroup * 4;                            // kGroup inputs
    const int tid = threadIdx.x;
    const int rpg = kThreads >> log2nb;
    const int rg = tid >> log2nb;
    const int blk = tid & ((1 << log2nb) - 1);
    const uint32_t dmask = static_cast<uint32_t>(d - 1);
    uint32_t dst[kH];
    uint64_t neg = 0;
#pragma unroll
    for (int b = 0; b < kH; ++b) {
        dst[b] = (static_cast<uint32_t>(rg) << log2d) + (static_cast<uint32_t>(perm[blk * kH + b]) & dmask);
        if (signs[blk * kH + b] < 0) neg |= (1ull << b);
    }
    const int64_t ngroups = (rows + rpg - 1) / rpg;
    constexpr int kChunks = kGroup * ES / 16;
    const unsigned char* yb = static_cast<const unsigned char*>(yin);
    for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
        const int64_t row0 = g * rpg;
        for (int c = tid; c < kChunks; c += kThreads) {
            const int e = c * (16 / ES);
            const int r = e >> log2d;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (row0 + r < rows)
                v = *reinterpret_cast<const uint4*>(yb + ((row0 + r) * static_cast<int64_t>(d) + (e & dmask)) * ES);
            *reinterpret_cast<uint4*>(inbuf + e * ES) = v;
        }
        __syncthreads();
        double acc[kH];
        const int base = (rg << log2d) + blk * kH;
#pragma unroll
        for (int b = 0; b < kH; ++b) {
            float f;
            if (kBF16In)
                f = bf16_to_f32(reinterpret_cast<const uint16_t*>(inbuf)[base + b]);
            else
                f = reinterpret_cast<const float*>(inbuf)[base + b];
            acc[b] = static_cast<double>(f);
        }
        fwht64(acc);
#pragma unroll
        for (int b = 0; b < kH; ++b) {
            const double v = ((neg >> b) & 1ull) ? -acc[b] : acc[b];
            outbuf[dst[b]] = static_cast<float>(v * 0.125);
        }
        __syncthreads();
        const int nvec = kGroup / 4;
        for (int c = tid; c < nvec; c += kThreads) {
            const int e = c * 4;
            const int r = e >> log2d;
            if (row0 + r >= rows) continue;
            const float4 v = reinterpret_cast<const float4*>(outbuf)[c];
            const int64_t off = (row0 + r) * static_cast<int64_t>(d) + (e & dmask);
            if (kBF16Out) {
                uint2 p;
                p.x = f32_to_bf16(v.x) | (f32_to_bf16(v.y) << 16);
                p.y = f32_to_bf16(v.z) | (f32_to_bf16(v.w) << 16);
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(xout) + off) = p;
            } else {
                *reinterpret_cast<float4*>(static_cast<float*>(xout) + off) = v;
            }
        }
        __syncthreads();
    }
}

int ilog2(int v) {
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}

template <typename Kernel, typename... Args>
hipError_t launch_persistent(Kernel kernel, size_t lds, int64_t ngroups, hipStream_t stream, Args... args) {
    int per_cu = 0;
    const hipError_t e = kernel_blocks_per_cu(reinterpret_cast<const void*>(kernel), kThreads, lds, &per_cu);
    if (e != hipSuccess) return e;
    const int64_t cap = static_cast<int64_t>(per_cu) * device_cu_count();
    const int grid = static_cast<int>(ngroups < cap ? ngroups : cap);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), lds, stream, args...);
    return hipGetLastError();
}

template <bool kBF16In, bool kRotate, int kOut>
hipError_t launch_rows_t(const RowArgs& a, hipStream_t stream) {
    constexpr int ES = kBF16In ? 2 : 4;
    const int log2d = ilog2(a.d);
    const int log2nb = log2d - 6;
    const int64_t rpg = kThreads >> log2nb;
    const int64_t ngroups = (a.rows + rpg - 1) / rpg;
    const size_t lds = static_cast<size_t>(kGroup) * ES + static_cast<size_t>(a.d) * ES + kRedBytes;
    return launch_persistent(rpbh_rows_kernel<kBF16In, kRotate, kOut>, lds, ngroups, stream, a.x, a.rows, a.d,
                             log2d, log2nb, a.perm, a.signs, a.out, a.scale, a.scale_bf16 ? 1 : 0, a.bounds, a.eps,
                             a.centroids, a.tiled ? 1 : 0);
}

template <bool kBF16In, bool kRotate>
hipError_t launch_rows_kind(const RowArgs& a, hipStream_t stream) {
    switch (a.out_kind) {
        case kRowRotF32: return launch_rows_t<kBF16In, kRotate, kRowRotF32>(a, stream);
        case kRowRotBF16: return launch_rows_t<kBF16In, kRotate, kRowRotBF16>(a, stream);
        case kRowInt8: return launch_rows_t<kBF16In, kRotate, kRowInt8>(a, stream);
        case kRowCode4: return launch_rows_t<kBF16In, kRotate, kRowCode4>(a, stream);
        case kRowCode2: return launch_rows_t<kBF16In, kRotate, kRowCode2>(a, stream);
        case kRowLut4: return launch_rows_t<kBF16In, kRotate, kRowLut4>(a, stream);
        case kRowLut2: return launch_rows_t<kBF16In, kRotate, kRowLut2>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_rpbh_rows(const RowArgs& a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    if (rpbh_quant_bf16_supported(a)) return launch_rpbh_quant_bf16(a, stream);   // it zeroes a.clear itself
    const bool rot = a.perm != nullptr;
    const hipError_t e = a.x_bf16 ? (rot ? launch_rows_kind<true, true>(a, stream) : launch_rows_kind<true, false>(a, stream))
                                  : (rot ? launch_rows_kind<false, true>(a, stream) : launch_rows_kind<false, false>(a, stream));
    if (e != hipSuccess) return e;
    return launch_split_clear(a.clear, a.nclear, stream);
}

hipError_t launch_rpbh_inverse(const void* y, bool y_bf16, void* x, bool x_bf16, int64_t rows, int d,
                               const int32_t* perm, const int8_t* signs, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    const int log2d = ilog2(d);
    const int log2nb = log2d - 6;
    const int64_t rpg = kThreads >> log2nb;
    const int64_t ngroups = (rows + rpg - 1) / rpg;
    const size_t lds = static_cast<size_t>(kGroup) * 4 + static_cast<size_t>(kGroup) * (y_bf16 ? 2 : 4);
    if (y_bf16)
        return x_bf16 ? launch_persistent(rpbh_inverse_kernel<true, true>, lds, ngroups, stream, y, rows, d, log2d,
                                          log2nb, perm, signs, x)
                      : launch_persistent(rpbh_inverse_kernel<true, false>, lds, ngroups, stream, y, rows, d, log2d,
                                          log2nb, perm, signs, x);
    return x_bf16 ? launch_persistent(rpbh_inverse_kernel<false, true>, lds, ngroups, stream, y, rows, d, log2d,
                                      log2nb, perm, signs, x)
                  : launch_persistent(rpbh_inverse_kernel<false, false>, lds, ngroups, stream, y, rows, d, log2d,
                                      log2nb, perm, signs, x);
}

}  // namespace rtq
