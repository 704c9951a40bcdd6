// rpbh_quant.hip -- the hot RPBH rotate + quantise kernel for bf16 rows on gfx950.
//
// Same arithmetic as rpbh_rows.hip (x' = Pi_d x via fp64 butterflies, exact while a block's
// magnitudes span at most 2^39, OrbitQuant article 2.3; INT8 s = max|x'|/127, q = rne(x'/s),
// cloud.baidu.com/article/9432521 4; Lloyd-Max codes of x'/(||x'|| + eps), OrbitQuant article
// 2.1-2.2), organised for HBM throughput:
//
//  * Scatter on staging.  Each lane loads 16-byte chunks of bf16 inputs and writes each element
//    straight to the LDS slot of the rotated block it feeds (the inverse permutation, as LDS
//    offsets), XOR-ing the Rademacher sign of that slot into the bf16 sign bit on the way.
//  * d <= 4096 (rpbh_wave_bf16_kernel): a row never spans waves, so every wave works alone on
//    units of 4096 consecutive elements (4096/d rows, 64 blocks, one per lane) in its own LDS
//    buffer, with the offset and sign tables shared by the workgroup; no barrier after the
//    prologue.  d > 4096 (rpbh_quant_bf16_kernel): a 256-thread workgroup moves groups of 16384
//    elements, rows span waves, and the row reductions cross waves through LDS.
//  * LDS blocks are 128 bytes of data + 16 bytes of padding, so lane l reads its own 64-element
//    block contiguously (eight 16-byte reads) without bank conflicts.
//  * Register prefetch: the next unit's (group's) global loads are issued before the current one
//    is transformed, so HBM traffic overlaps the butterflies and quantisation.
//  * Division-free INT8: the correctly rounded quotient x'/s comes from the row's reciprocal and
//    one fma correction step, then one add of 1.5*2^23 rounds it half-to-even into the low mantissa
//    bits; branch-free, and bit-identical to rne(fl32(x'/s)).  Only rows whose max |x'| is below
//    2^-103 (subnormals could round differently) take an IEEE-division path.
//  * Division-free codebook codes: for each row the exact fp32 thresholds Y_k = min{x' : fl32(x' /
//    (s+eps)) > t_k} are found once (IEEE divisions, a few ulp steps), so code = #{k : x' >= Y_k}
//    needs no division.  For 8, 16 and 64 levels the candidate boundary comes from a grid over the
//    boundary range (64 or 256 cells, each holding at most one boundary even when widened by the
//    rounding slack): one LDS table read per element gives the cell's threshold, the count below
//    it and the int8 values, and one compare settles the code.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "codebook_int8.h"
#include "rtq_internal.h"

namespace rtq {
namespace {

constexpr int kThreads = 256;
constexpr int kH = 64;
constexpr int kGroup = kThreads * kH;         // 16384 elements per group
constexpr int kBlockPitch = 144;              // bytes per 64-element bf16 block in LDS (128 + 16 pad)
constexpr int kRowBuf = kThreads * kBlockPitch;   // 36864
constexpr int kChunkStride = 32 * kBlockPitch;    // LDS distance of 2048 consecutive elements
constexpr int kMaxD = 16384;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float next_up(float y) {
    if (y == 0.0f) return 0x1p-149f;
    const int32_t u = __float_as_int(y);
    return __int_as_float(u >= 0 ? u + 1 : u - 1);
}

__device__ __forceinline__ float next_down(float y) {
    if (y == 0.0f) return -0x1p-149f;
    const int32_t u = __float_as_int(y);
    return __int_as_float(u >= 0 ? u - 1 : u + 1);
}

// Smallest fp32 x with fl32(x / den) > t (division is IEEE, so this is the exact switch point of
// the code decision; x / den is non-decreasing in x).  Starts from fl32(t * den), which is within a
// couple of ulps of it, and walks one ulp at a time.
__device__ float exact_threshold(float t, float den) {
    float y = t * den;
    if (y / den > t) {
        for (int i = 0; i < 16; ++i) {
            const float yd = next_down(y);
            if (yd / den > t) y = yd; else break;
        }
    } else {
        for (int i = 0; i < 16; ++i) {
            y = next_up(y);
            if (y / den > t) break;
        }
    }
    return y;
}

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

// My block from LDS (already permuted and signed), widened to fp64 and transformed: v = 8 * x'.
// A lane's 64-element block from LDS (already permuted and signed), widened to fp64 and
// transformed: v = 8 * x'.
__device__ __forceinline__ void load_block_fwht(const unsigned char* block, double (&acc)[kH]) {
    const uint4* bp = reinterpret_cast<const uint4*>(block);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const uint4 v = bp[q];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            acc[8 * q + 2 * p] = static_cast<double>(__uint_as_float(w[p] << 16));
            acc[8 * q + 2 * p + 1] = static_cast<double>(__uint_as_float(w[p] & 0xffff0000u));
        }
    }
    fwht64(acc);
}
// ---- reductions over the nb = 2^log2nb consecutive lanes that hold one row (DPP inside a
//      16-lane row, lane reads across rows, LDS across waves).  Every thread of the workgroup
//      must call these together (the cross-wave step has a barrier); the result reaches every
//      lane of the row.
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ int dpp(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, kCtrl, kRowMask, 0xf, false);
}

__device__ __forceinline__ float row_max(float v, int log2nb, float* red) {
    // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
    if (log2nb >= 1) v = fmaxf(v, __int_as_float(dpp<0xB1>(__float_as_int(v), __float_as_int(v))));
    if (log2nb >= 2) v = fmaxf(v, __int_as_float(dpp<0x4E>(__float_as_int(v), __float_as_int(v))));
    if (log2nb >= 3) v = fmaxf(v, __int_as_float(dpp<0x141>(__float_as_int(v), __float_as_int(v))));
    if (log2nb >= 4) v = fmaxf(v, __int_as_float(dpp<0x140>(__float_as_int(v), __float_as_int(v))));
    if (log2nb >= 5) {
        const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15));
        const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
        const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47));
        const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
        if (log2nb == 5)
            v = (threadIdx.x & 32) ? fmaxf(r2, r3) : fmaxf(r0, r1);
        else
            v = fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
    }
    if (log2nb > 6) {
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) red[wave] = v;
        __syncthreads();
        const int wpr = 1 << (log2nb - 6);
        const int w0 = wave & ~(wpr - 1);
        float m = red[w0];
        for (int i = 1; i < wpr; ++i) m = fmaxf(m, red[w0 + i]);
        v = m;
    }
    return v;
}

template <int kCtrl>
__device__ __forceinline__ double dpp_add_f64(double v) {
    const int lo = __double2loint(v), hi = __double2hiint(v);
    return v + __hiloint2double(dpp<kCtrl>(0, hi), dpp<kCtrl>(0, lo));
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), lane),
                            __builtin_amdgcn_readlane(__double2loint(v), lane));
}

__device__ __forceinline__ double row_sum(double v, int log2nb, double* red) {
    if (log2nb >= 1) v = dpp_add_f64<0xB1>(v);
    if (log2nb >= 2) v = dpp_add_f64<0x4E>(v);
    if (log2nb >= 3) v = dpp_add_f64<0x141>(v);
    if (log2nb >= 4) v = dpp_add_f64<0x140>(v);
    if (log2nb >= 5) {
        const double r0 = readlane_f64(v, 15), r1 = readlane_f64(v, 31);
        const double r2 = readlane_f64(v, 47), r3 = readlane_f64(v, 63);
        if (log2nb == 5)
            v = (threadIdx.x & 32) ? r2 + r3 : r0 + r1;
        else
            v = (r0 + r1) + (r2 + r3);
    }
    if (log2nb > 6) {
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) red[wave] = v;
        __syncthreads();
        const int wpr = 1 << (log2nb - 6);
        const int w0 = wave & ~(wpr - 1);
        double m = red[w0];
        for (int i = 1; i < wpr; ++i) m += red[w0 + i];
        v = m;
    }
    return v;
}

// Per-lane codebook state for one launch: the lane's boundary slot, the lane's cells of the
// boundary grid, and the int8 value table for kRowLut*.
//
// Boundary grid (3, 4 and 6-bit codes).  kCells cells over u = x' / den: 2 * kHalfSpan of them
// cover [-tmax, tmax] (tmax = the largest |boundary|) and the two end cells take everything
// beyond.  Each cell is widened by a small slack, so a boundary near a cell edge belongs to both
// neighbours, and the grid is used only if no widened cell holds two boundaries (true for the
// Lloyd-Max tables of 8, 16 and 64 levels: their closest boundaries are 1.9 cells or more apart).  Per row, each wave
// keeps an LDS table with one 8-byte entry per (row of the wave, cell): the exact threshold Y of
// the cell's boundary (in x' units; +inf for none), rewritten per row, and the cell's info word,
// written once by setup() (#{boundaries below the cell} | int8 value of that code << 8 | of the
// next << 16 | slot of its boundary, kNB for none, << 24), so an element's code is
// below + (x' >= Y) after one table read.
template <int kOut>
struct CodeCtx {
    static constexpr bool k4 = kOut == kRowCode4 || kOut == kRowLut4;
    static constexpr bool k2 = kOut == kRowCode2 || kOut == kRowLut2;
    static constexpr bool k3 = kOut == kRowCode3 || kOut == kRowLut3;
    static constexpr bool k6 = kOut == kRowLut6;
    static constexpr bool kLut = kOut == kRowLut4 || kOut == kRowLut2 || kOut == kRowLut3 || kOut == kRowLut6;
    static constexpr bool kGrid = k4 || k3 || k6;   // boundary grid for 8, 16 and 64 levels
    static constexpr int kBits = k4 ? 4 : (k2 ? 2 : (k3 ? 3 : (k6 ? 6 : 8)));
    static constexpr int kNB = (1 << kBits) - 1;
    static constexpr int kCells = k6 ? 256 : 64;
    static constexpr int kHalfSpan = k6 ? 100 : 20;          // cells per tmax
    static constexpr int kPer = kCells / 64;                 // cells per lane
    // LDS per wave for the table: rows of the wave x kCells x 8 bytes (up to 8 rows of 64 cells when
    // rows are shorter than a wave; one row when a row spans waves)
    static constexpr int kTabBytes = kGrid ? 4096 : 0;
    static constexpr int kTabBytesRow = kGrid ? kCells * 8 : 0;
    int lane_base = 0;
    int kidx = 0;                 // my threshold slot
    float my_t = __builtin_inff();
    float tb[3] = {0.0f, 0.0f, 0.0f};
    float grid_k = 0.0f;
    bool use_grid = false;        // per lane here: the caller makes it uniform over the workgroup
    bool use_bsearch = false;     // 64 levels without the grid: binary search over lane-held thresholds

    // ctab0: the first wave's table region; the workgroup computes the cell info words once, into
    // its first row (fill() then copies them into every wave's rows, after a barrier)
    __device__ __forceinline__ void setup(const float* __restrict__ bounds, const float* __restrict__ cent,
                                          int log2nb, int lane, uint2* ctab0) {
        const int row_lanes = (1 << log2nb) < 64 ? (1 << log2nb) : 64;   // lanes of my row in my wave
        lane_base = lane & ~(row_lanes - 1);
        kidx = lane - lane_base;
        constexpr int L = 1 << kBits;
        if (k2) {
#pragma unroll
            for (int k = 0; k < 3; ++k) tb[k] = bounds[k];
        }
        if (kGrid && kidx < kNB) my_t = bounds[kidx];
        if (k6) use_bsearch = row_lanes == 64;
        if (kGrid) {
            const float vs = kLut ? codebook_int8_scale(cent, L) : 0.0f;
            const float tmax = fmaxf(fabsf(bounds[0]), fabsf(bounds[kNB - 1]));
            use_grid = row_lanes >= kNB + 1 && tmax > 0.0f;
            if (use_grid) {
                grid_k = static_cast<float>(kHalfSpan) / tmax;   // cell units per unit of u
                const float slack = 1.0f / 1024.0f;              // in cell units: covers every rounding error
                static_assert(kCells <= kThreads, "one cell per thread");
                for (int j = static_cast<int>(threadIdx.x); j < kCells; j += kThreads) {   // cell index
                    const float lo = (j == 0) ? -__builtin_inff() : (static_cast<float>(j - kCells / 2) - slack) / grid_k;
                    const float hi = (j == kCells - 1) ? __builtin_inff()
                                                       : (static_cast<float>(j - kCells / 2 + 1) + slack) / grid_k;
                    int below = 0, inside = 0, kin = kNB;
                    for (int k = 0; k < kNB; ++k) {
                        const float t = bounds[k];
                        if (t < lo) ++below;
                        else if (t < hi) { ++inside; kin = k; }
                    }
                    if (inside > 1) use_grid = false;
                    uint32_t v = 0u;
                    if (kLut) {
                        v = (static_cast<uint32_t>(codebook_int8_value(cent, below, vs)) & 0xffu) << 8;
                        if (below + 1 < L) v |= (static_cast<uint32_t>(codebook_int8_value(cent, below + 1, vs)) & 0xffu) << 16;
                    }
                    ctab0[j].y = static_cast<uint32_t>(below) | v | (static_cast<uint32_t>(kin) << 24);
                }
            }
        }
    }

    // After setup() and a barrier (with use_grid made uniform): the info words into every row of
    // this wave's table (the first wave's first row already holds them).
    __device__ __forceinline__ void fill(int log2nb, int lane, uint2* ctab, const uint2* ctab0) const {
        if (!kGrid || !use_grid) return;
        const int row_lanes = (1 << log2nb) < 64 ? (1 << log2nb) : 64;
        const bool first = ctab == ctab0;
#pragma unroll
        for (int p = 0; p < kPer; ++p) {
            const uint32_t ci = ctab0[lane + 64 * p].y;
            for (int r = first ? 1 : 0; r < 64 / row_lanes; ++r) ctab[r * kCells + lane + 64 * p].y = ci;
        }
    }
};

// A lane's quantised block: its code words (INT8 and int8 codebook values: 16 words of 4 bytes;
// packed 4-bit codes: 8 words; 2-bit: 4) and its row's scale or norm.
struct BlockOut {
    uint32_t w[kH / 4];
    float s;
    int32_t z;      // asymmetric INT8: the row's zero point
    int32_t sum;    // asymmetric INT8: the row's code sum
};

// Extra per-row outputs of asymmetric INT8 rows (null otherwise).
struct RowExtra {
    int32_t* zero;
    int32_t* sum;
    unsigned long long* clear;   // words the first workgroup zeroes (the next product's split counters)
    int nclear;
    int tiled;                   // INT8 codes in the product's tiled layout
};

// The first workgroup zeroes the words the launch was asked to clear.
__device__ __forceinline__ void clear_words(const RowExtra& ex) {
    if (blockIdx.x == 0)
        for (int i = static_cast<int>(threadIdx.x); i < ex.nclear; i += static_cast<int>(blockDim.x)) ex.clear[i] = 0ull;
}

// Bytes per output element (8 codes per 64 bits for 4-bit codes etc., in bits).
template <int kOut>
constexpr int out_bits() {
    return kOut == kRowCode4 ? 4 : (kOut == kRowCode2 ? 2 : (kOut == kRowCode3 ? 3 : 8));
}

// Quantise a lane's rotated block (acc = 8 x' in fp64: the lane's 64 outputs of its row) with the
// row's scale or norm, reduced over the row's lanes.  Every lane of the workgroup calls this
// together when rows span several waves (log2nb > 6).  ctab: this wave's LDS region for the
// boundary-grid table (CodeCtx::kTabBytes).
template <int kOut>
__device__ __forceinline__ void quantize_block(double (&acc)[kH], const unsigned char* block, int log2nb,
                                               double* red, uint2* ctab, const CodeCtx<kOut>& cc,
                                               const float* __restrict__ bounds, const float* __restrict__ cent,
                                               float eps, int scale_bf16, BlockOut& res) {
    constexpr bool k4 = CodeCtx<kOut>::k4;
    constexpr bool k2 = CodeCtx<kOut>::k2;
    constexpr bool k3 = CodeCtx<kOut>::k3;
    constexpr bool k6 = CodeCtx<kOut>::k6;
    constexpr bool kLut = CodeCtx<kOut>::kLut;
    constexpr int kBits = CodeCtx<kOut>::kBits;
    constexpr int kNB = CodeCtx<kOut>::kNB;
    uint32_t* w = res.w;
    if constexpr (kOut == kRowInt8Asym) {
        // lo = min(min x', 0), hi = max(max x', 0): fl32(extremes of 8x' / 8) (rounding is monotone),
        // reduced over the row; s = fl32(fl32(hi - lo) / 255) (then bf16 when stored so), and with
        // the stored s: z = clamp(-128 - rne(fl32(lo / s)), -128, 127), q = clamp(rne(fl32(x'/s)) + z)
        double mx4[kH / 4], mn4[kH / 4];
#pragma unroll
        for (int k = 0; k < kH / 4; ++k) {
            mx4[k] = fmax(fmax(acc[4 * k], acc[4 * k + 1]), fmax(acc[4 * k + 2], acc[4 * k + 3]));
            mn4[k] = fmin(fmin(acc[4 * k], acc[4 * k + 1]), fmin(acc[4 * k + 2], acc[4 * k + 3]));
        }
#pragma unroll
        for (int k = 0; k < kH / 16; ++k) {
            mx4[k] = fmax(fmax(mx4[4 * k], mx4[4 * k + 1]), fmax(mx4[4 * k + 2], mx4[4 * k + 3]));
            mn4[k] = fmin(fmin(mn4[4 * k], mn4[4 * k + 1]), fmin(mn4[4 * k + 2], mn4[4 * k + 3]));
        }
        const double bmx = fmax(fmax(fmax(mx4[0], mx4[1]), fmax(mx4[2], mx4[3])), 0.0);
        const double bmn = fmin(fmin(fmin(mn4[0], mn4[1]), fmin(mn4[2], mn4[3])), 0.0);
        // three row reductions back to back: each crosses waves (d > 4096) through its own part of
        // the reduction scratch (floats 0-3, floats 4-7, doubles 4-7), so none overwrites another's
        // values while they are read
        float* red_hi = reinterpret_cast<float*>(red);
        float* red_lo = red ? reinterpret_cast<float*>(red) + 4 : nullptr;
        double* red_sum = red ? red + 4 : nullptr;
        const float hi = row_max(static_cast<float>(bmx * 0.125), log2nb, red_hi);
        const float lo = -row_max(static_cast<float>(-bmn * 0.125), log2nb, red_lo);
        float s = (hi - lo) / 255.0f;
        if (scale_bf16) s = bf16_to_f32(f32_to_bf16(s));
        int z = 0;
        if (s != 0.0f) z = static_cast<int>(fminf(fmaxf(-128.0f - rintf(lo / s), -128.0f), 127.0f));
        // the quotient as in the symmetric path (Markstein's correction step, then 1.5*2^23 rounds
        // it half-to-even into the low mantissa bits); here the whole integer is taken, z added and
        // the sum clamped
        const float s8 = s * 8.0f;
        const float r8 = 1.0f / s8;
        constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
        const int zoff = z - 0x4B400000;       // bits of kMagic, subtracted back out
        int csum = 0;
#pragma unroll
        for (int q = 0; q < kH / 4; ++q) {
            int c[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float y = static_cast<float>(acc[4 * q + p]);
                const float q0 = y * r8;
                const float q1 = fmaf(fmaf(-q0, s8, y), r8, q0);
                c[p] = min(max(__float_as_int(q1 + kMagic) + zoff, -128), 127);
                csum += c[p];
            }
            w[q] = (static_cast<uint32_t>(c[0]) & 0xffu) | ((static_cast<uint32_t>(c[1]) & 0xffu) << 8) |
                   ((static_cast<uint32_t>(c[2]) & 0xffu) << 16) | (static_cast<uint32_t>(c[3]) << 24);
        }
        // fl32(8x')/(8s) equals x'/s while x' is normal; with hi - lo >= 2^-100 a subnormal x' has
        // |x'/s| < 2^-17 and rounds to 0 either way.  Tinier rows take the exact path.
        if (!(hi - lo >= 0x1p-100f)) {
            csum = 0;
#pragma unroll
            for (int q = 0; q < kH / 4; ++q) w[q] = 0u;
            if (s != 0.0f) {
                double a2[kH];
                load_block_fwht(block, a2);
                for (int b = 0; b < kH; ++b) {
                    const float xr = static_cast<float>(a2[b] * 0.125);
                    const int code = static_cast<int>(fminf(fmaxf(rintf(xr / s) + static_cast<float>(z), -128.0f), 127.0f));
                    csum += code;
                    w[b >> 2] |= (static_cast<uint32_t>(code) & 0xffu) << ((b & 3) * 8);
                }
            }
        }
        res.s = s;
        res.z = z;
        res.sum = static_cast<int32_t>(row_sum(static_cast<double>(csum), log2nb, red_sum));
    } else if constexpr (kOut == kRowInt8) {
        // amax = max |x'| = fl32(max |8x'| / 8) exactly (rounding is monotone), reduced over the row;
        // the block maximum as a tree (no serial chain of 64 dependent maxima)
        double m4[kH / 4];
#pragma unroll
        for (int k = 0; k < kH / 4; ++k)
            m4[k] = fmax(fmax(fabs(acc[4 * k]), fabs(acc[4 * k + 1])), fmax(fabs(acc[4 * k + 2]), fabs(acc[4 * k + 3])));
#pragma unroll
        for (int k = 0; k < kH / 16; ++k)
            m4[k] = fmax(fmax(m4[4 * k], m4[4 * k + 1]), fmax(m4[4 * k + 2], m4[4 * k + 3]));
        const double m = fmax(fmax(m4[0], m4[1]), fmax(m4[2], m4[3]));
        const float amax = row_max(static_cast<float>(m * 0.125), log2nb, reinterpret_cast<float*>(red));
        float s = amax / 127.0f;
        if (scale_bf16) s = bf16_to_f32(f32_to_bf16(s));
        // q = rne(fl32(x'/s)) with x'/s = y/(8s), y = fl32(8x'), and no division per element:
        // r = RN(1/(8s)), q0 = RN(y*r), e = y - q0*(8s) (exact by fma), q1 = RN(q0 + e*r) is
        // the correctly rounded quotient (Markstein's correction step), and adding 1.5*2^23
        // rounds q1 half-to-even into the low mantissa bits, whose low byte is the code.
        const float s8 = s * 8.0f;
        const float r8 = 1.0f / s8;
        constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
#pragma unroll
        for (int q = 0; q < kH / 4; ++q) {
            float t[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float y = static_cast<float>(acc[4 * q + p]);
                const float q0 = y * r8;
                const float q1 = fmaf(fmaf(-q0, s8, y), r8, q0);
                t[p] = q1 + kMagic;
            }
            const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(t[1]), __float_as_uint(t[0]), 0x0c0c0400u);
            const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(t[3]), __float_as_uint(t[2]), 0x04000c0cu);
            w[q] = lo | hi;
        }
        // fl32(8x')/(8s) equals x'/s while x' is normal; with amax >= 2^-103 a subnormal x' gives
        // code 0 either way.  Tinier rows (and all-zero rows) take the exact path.
        const bool fast = amax >= 0x1p-103f;
        if (!fast) {
            // exact: q = rne(fl32(x'/s)), x' = fl32(8x' / 8); transform again from LDS (still intact)
#pragma unroll
            for (int q = 0; q < kH / 4; ++q) w[q] = 0u;
            if (s != 0.0f) {
                double a2[kH];
                load_block_fwht(block, a2);
                for (int b = 0; b < kH; ++b) {
                    const float xr = static_cast<float>(a2[b] * 0.125);
                    float r = rintf(xr / s);
                    r = fminf(fmaxf(r, -127.0f), 127.0f);
                    w[b >> 2] |= (static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xffu) << ((b & 3) * 8);
                }
            }
        }
        res.s = s;
    } else {
        // x' = fl32(8x' / 8): the oracle's rotated value (fp64 sums of bf16 inputs are exact while a
        // block's magnitudes span at most 2^39)
        float xr[kH];
        double ss4[4] = {0.0, 0.0, 0.0, 0.0};   // four interleaved partial sums: short dependency chains
#pragma unroll
        for (int b = 0; b < kH; ++b) {
            xr[b] = static_cast<float>(acc[b] * 0.125);
            const double f = static_cast<double>(xr[b]);
            ss4[b & 3] = fma(f, f, ss4[b & 3]);
        }
        double ss = row_sum((ss4[0] + ss4[1]) + (ss4[2] + ss4[3]), log2nb, red);
        const float s = static_cast<float>(sqrt(ss));
        float den = (eps == 0.0f) ? s : s + eps;
        // A row with a tiny norm (a weight row, eps = 0) is scaled by 2^64, x' and den alike: exact
        // (|x'| <= den), and fl32(x'/den) is unchanged, while the thresholds t_k * den and the
        // grid's cells per unit of x' (grid_k / den) stay in the normal fp32 range.
        if (den != 0.0f && den < 0x1p-60f) {
            den *= 0x1p64f;
#pragma unroll
            for (int b = 0; b < kH; ++b) xr[b] *= 0x1p64f;
        }
        // codes as one LSB-first bit stream of kSlot-bit fields: packed codes (2, 3, 4 bits), or one
        // byte per code (kRowLut*: its int8 value; the grid table holds the values, the other paths
        // look codes up afterwards, or as they are found for 6-bit codes)
        constexpr int kSlot = kLut ? 8 : kBits;
        constexpr int kWords = kH * kSlot / 32;
        auto put_bits = [&](int b, uint32_t v) {
            const int p = b * kSlot, q = p >> 5, sh = p & 31;
            w[q] |= v << sh;
            if (sh + kSlot > 32) w[q + 1] |= v >> (32 - sh);
        };
        // 64 levels off the grid: lane k holds the int8 value of code k
        const int lutv = k6 && !cc.use_grid ? codebook_int8_value(cent, threadIdx.x & 63, codebook_int8_scale(cent, 64)) : 0;
        auto put = [&](int b, uint32_t code) {
            if constexpr (k6) code = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(static_cast<int>(4 * code), lutv)) & 0xffu;
            put_bits(b, code);
        };
        bool values_done = false;   // the words already hold int8 values
#pragma unroll
        for (int q = 0; q < kWords; ++q) w[q] = 0u;
        // u = fl32(x'/den); code = #{k : t_k < u} = #{k : x' >= Y_k}, Y_k exact per row
        if (CodeCtx<kOut>::kGrid && cc.use_grid) {
            // Every lane of the wave takes part (table entries of one row are written by lanes
            // of every row, and cross-lane reads see only active lanes), so a row with
            // den = 0 runs here too, with den = 1: its x' are all zero, and x' = 0 against the
            // thresholds for den = 1 gives #{k : t_k < 0}, the code of u = 0.
            const float dn = den != 0.0f ? den : 1.0f;
            // my slot holds Y_kidx; the wave's table gets one entry per (row of the wave, cell)
            const float myY = cc.kidx < kNB ? exact_threshold(cc.my_t, dn) : __builtin_inff();
            constexpr int kCells = CodeCtx<kOut>::kCells;
            const int row_lanes = log2nb < 6 ? 1 << log2nb : 64;
            for (int r = 0; r < 64 / row_lanes; ++r) {
#pragma unroll
                for (int p = 0; p < CodeCtx<kOut>::kPer; ++p) {
                    uint2* ent = ctab + r * kCells + 64 * p + (threadIdx.x & 63);
                    const int slot = static_cast<int>(ent->y >> 24);
                    const float y = __int_as_float(__builtin_amdgcn_ds_bpermute(
                        4 * (r * row_lanes + (slot < kNB ? slot : 0)), __float_as_int(myY)));
                    ent->x = __float_as_uint(slot < kNB ? y : __builtin_inff());
                }
            }
            // (the wave's LDS accesses execute in order: its reads below see these writes)
            const uint2* rt = ctab + (cc.lane_base / row_lanes) * kCells;
            const float ka = cc.grid_k / dn;              // cells per unit of x'
            constexpr float kMid = 0.5f * kCells, kTop = kCells - 0.125f;
#pragma unroll
            for (int b = 0; b < kH; ++b) {
                const int a = static_cast<int>(__builtin_amdgcn_fmed3f(fmaf(xr[b], ka, kMid), 0.0f, kTop));
                const uint2 e = rt[a];
                const bool ge = xr[b] >= __uint_as_float(e.x);
                if constexpr (kLut)
                    put_bits(b, (e.y >> (ge ? 16 : 8)) & 0xffu);
                else
                    put_bits(b, (e.y & 0xffu) + (ge ? 1u : 0u));
            }
            values_done = kLut;
        } else if (den != 0.0f) {
            if (k2) {
                float Y[3];
#pragma unroll
                for (int k = 0; k < 3; ++k) Y[k] = exact_threshold(cc.tb[k], den);
#pragma unroll
                for (int b = 0; b < kH; ++b) {
                    const uint32_t code = (xr[b] >= Y[0] ? 1u : 0u) + (xr[b] >= Y[1] ? 1u : 0u) + (xr[b] >= Y[2] ? 1u : 0u);
                    put(b, code);
                }
            } else if (k6 && cc.use_bsearch) {
                // my lane holds Y_kidx (lane 63: +inf); code = #{k : x' >= Y_k} by binary search
                const float myY = cc.kidx < kNB ? exact_threshold(cc.my_t, den) : __builtin_inff();
#pragma unroll
                for (int b = 0; b < kH; ++b) {
                    int lo = 0;
#pragma unroll
                    for (int step = 32; step >= 1; step >>= 1) {
                        const float t = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (lo + step - 1), __float_as_int(myY)));
                        lo += xr[b] >= t ? step : 0;
                    }
                    put(b, static_cast<uint32_t>(lo));
                }
            } else {
                // a general codebook, or too few lanes per row for the slot table: divide and count
#pragma unroll
                for (int b = 0; b < kH; ++b) {
                    const float u = xr[b] / den;
                    uint32_t code = 0;
                    for (int k = 0; k < kNB; ++k) code += (bounds[k] < u) ? 1u : 0u;
                    put(b, code);
                }
            }
        } else {
            // zero row with eps = 0: u = 0 for every element
            uint32_t code = 0;
            for (int k = 0; k < kNB; ++k) code += (bounds[k] < 0.0f) ? 1u : 0u;
#pragma unroll
            for (int b = 0; b < kH; ++b) put(b, code);
        }
        if (kLut && !k6 && !values_done) {
            uint32_t lut[4];
            codebook_int8_table(cent, 1 << kBits, codebook_int8_scale(cent, 1 << kBits), lut);
#pragma unroll
            for (int q = 0; q < kWords; ++q)
                w[q] = k4 ? lut16_x4(lut, w[q]) : (k3 ? lut8_x4(lut, w[q]) : lut4_x4(lut, w[q]));
        }
        res.s = s;
    }
}

// Store a lane's quantised block (block `blk` of row `row`) and, from the row's first block, its scale.
template <int kOut>
__device__ __forceinline__ void store_block(const BlockOut& res, void* __restrict__ out, void* __restrict__ scale_out,
                                            int scale_bf16, RowExtra ex, int64_t row, int blk, int d) {
    constexpr int kWords = kH * out_bits<kOut>() / 32;
    if (ex.tiled) {
        if constexpr (out_bits<kOut>() == 8) {   // int8 codes or values: a 64-byte slot, chunks swizzled
            int8_t* o = static_cast<int8_t*>(out) + tiled_slot_offset(row, blk, d);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<uint4*>(o + 16 * tiled_chunk(row, q)) =
                    make_uint4(res.w[4 * q], res.w[4 * q + 1], res.w[4 * q + 2], res.w[4 * q + 3]);
        } else if constexpr (kWords % 4 == 0) {   // packed codes: the block's 8 * bits bytes, contiguous
            uint4* o = reinterpret_cast<uint4*>(static_cast<uint8_t*>(out) + tiled_code_offset(row, blk, d, out_bits<kOut>()));
#pragma unroll
            for (int q = 0; q < kWords / 4; ++q) o[q] = make_uint4(res.w[4 * q], res.w[4 * q + 1], res.w[4 * q + 2], res.w[4 * q + 3]);
        } else {
            uint2* o = reinterpret_cast<uint2*>(static_cast<uint8_t*>(out) + tiled_code_offset(row, blk, d, out_bits<kOut>()));
#pragma unroll
            for (int q = 0; q < kWords / 2; ++q) o[q] = make_uint2(res.w[2 * q], res.w[2 * q + 1]);
        }
    } else if constexpr (kWords % 4 == 0) {
        uint4* o = reinterpret_cast<uint4*>(static_cast<uint8_t*>(out) + (row * d + blk * kH) * out_bits<kOut>() / 8);
#pragma unroll
        for (int q = 0; q < kWords / 4; ++q) o[q] = make_uint4(res.w[4 * q], res.w[4 * q + 1], res.w[4 * q + 2], res.w[4 * q + 3]);
    } else {   // 3-bit codes: 24 bytes per block, 8-byte aligned
        uint2* o = reinterpret_cast<uint2*>(static_cast<uint8_t*>(out) + (row * d + blk * kH) * out_bits<kOut>() / 8);
#pragma unroll
        for (int q = 0; q < kWords / 2; ++q) o[q] = make_uint2(res.w[2 * q], res.w[2 * q + 1]);
    }
    if (blk == 0) {
        if (scale_bf16)
            static_cast<uint16_t*>(scale_out)[row] = static_cast<uint16_t>(f32_to_bf16(res.s));
        else
            static_cast<float*>(scale_out)[row] = res.s;
        if constexpr (kOut == kRowInt8Asym) {
            ex.zero[row] = res.z;
            ex.sum[row] = res.sum;
        }
    }
}

// kNC: distinct 16-byte chunk columns a thread stages per group = max(1, d / 2048).
template <int kNC, int kOut>
__global__ void __launch_bounds__(kThreads, 2)
rpbh_quant_bf16_kernel(const uint16_t* __restrict__ x, int64_t rows, int d, int log2d, int log2nb,
                       const int32_t* __restrict__ perm, const int8_t* __restrict__ signs, void* __restrict__ out,
                       void* __restrict__ scale_out, int scale_bf16, const float* __restrict__ bounds, float eps,
                       const float* __restrict__ cent, RowExtra ex) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    clear_words(ex);
    // LDS: [row buffer(s) | prologue scratch overlaid][sign masks, d x u16 (kNC >= 4)][reduction]
    // d <= 4096: two row buffers, so staging group g+1 never waits for readers of group g
    // (one barrier per group).  d >= 8192: one buffer plus the persistent sign-mask table.
    constexpr bool kMaskInLds = kNC >= 4;
    constexpr int kBufs = kMaskInLds ? 1 : 2;
    uint16_t* sg = reinterpret_cast<uint16_t*>(smem + (kMaskInLds ? kRowBuf : 2 * d));
    double* red = reinterpret_cast<double*>(smem + kBufs * kRowBuf + (kMaskInLds ? 2 * d : 0));
    // behind the reduction scratch: each wave's boundary-grid table (codebook kinds)
    uint2* ctab0 = reinterpret_cast<uint2*>(smem + kBufs * kRowBuf + (kMaskInLds ? 2 * d : 0) + 64);
    uint2* ctab = ctab0 + (threadIdx.x >> 6) * (CodeCtx<kOut>::kTabBytesRow / 8);   // a row spans waves: one row each

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int rpg = kThreads >> log2nb;
    const int rg = tid >> log2nb;
    const int blk = tid & ((1 << log2nb) - 1);
    const uint32_t dmask = static_cast<uint32_t>(d - 1);

    // ---- once per workgroup: inverse permutation and source-side signs.  All loads are issued
    //      before any LDS store so their latencies overlap.
    // d = 16384: a thread's 64 scatter addresses would take 32 registers even as 16-bit pairs (and
    // spill); there the table entry of a source column holds its slot's offset / 2 (15 bits) and
    // its sign (bit 15), read with the chunk.  d <= 8192: addresses in registers, signs in LDS.
    constexpr bool kTabAddr = kNC >= 8;
    uint32_t addr[kTabAddr ? 1 : kNC * 8];
    uint4 msk[kMaskInLds ? 1 : kNC];
    if constexpr (kTabAddr) {
        // batches of 8 loads per thread (16 at d = 16384), issued before their LDS stores
        constexpr int kBatch = 8;
        for (int j0 = 4 * tid; j0 < d; j0 += 4 * kThreads * kBatch) {
            int4 pv[kBatch];
            uint32_t sv[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i) {
                const int j = j0 + i * 4 * kThreads;
                if (j < d) {
                    pv[i] = *reinterpret_cast<const int4*>(perm + j);
                    sv[i] = *reinterpret_cast<const uint32_t*>(signs + j);
                }
            }
#pragma unroll
            for (int i = 0; i < kBatch; ++i) {
                const int j = j0 + i * 4 * kThreads;
                if (j < d) {
                    const int pj[4] = {pv[i].x, pv[i].y, pv[i].z, pv[i].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t c = static_cast<uint32_t>(pj[e]) & dmask;
                        const uint32_t jj = static_cast<uint32_t>(j + e);
                        sg[c] = static_cast<uint16_t>(((jj >> 6) * (kBlockPitch / 2) + (jj & 63u)) |
                                                      ((sv[i] >> (8 * e + 7)) & 1u ? 0x8000u : 0u));
                    }
                }
            }
        }
    } else {
        uint16_t* inv = reinterpret_cast<uint16_t*>(smem);     // overlays the row buffer
        constexpr int kPer = kMaxD / 4 / kThreads;             // int4 perm loads per thread at d = 16384
        int4 pv[kPer];
        uint32_t sv[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int j = 4 * (tid + i * kThreads);
            if (j < d) {
                pv[i] = *reinterpret_cast<const int4*>(perm + j);
                sv[i] = *reinterpret_cast<const uint32_t*>(signs + j);
            }
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int j = 4 * (tid + i * kThreads);
            if (j < d) {
                const int pj[4] = {pv[i].x, pv[i].y, pv[i].z, pv[i].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t p = static_cast<uint32_t>(pj[e]) & dmask;
                    inv[p] = static_cast<uint16_t>(j + e);
                    sg[p] = (sv[i] >> (8 * e + 7)) & 1u ? 0x8000u : 0u;
                }
            }
        }
        __syncthreads();
        // For kNC == 1 (d <= 2048) a thread's chunks sit 2048/d rows apart: its first row goes into
        // the address, the per-chunk row step is an immediate.
        const uint32_t row_base = kNC == 1 ? ((8u * tid) >> log2d) * static_cast<uint32_t>((d >> 6) * kBlockPitch) : 0u;
#pragma unroll
        for (int c = 0; c < kNC; ++c) {
            const uint32_t col = (8u * tid + 2048u * c) & dmask;
            const uint4 iv = *reinterpret_cast<const uint4*>(inv + col);
            const uint32_t iw[4] = {iv.x, iv.y, iv.z, iv.w};
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t j = (k & 1) ? (iw[k >> 1] >> 16) : (iw[k >> 1] & 0xffffu);
                addr[c * 8 + k] = row_base + (j >> 6) * kBlockPitch + (j & 63u) * 2u;
            }
            if (!kMaskInLds) msk[c] = *reinterpret_cast<const uint4*>(sg + col);
        }
    }

    // ---- codebook set-up
    CodeCtx<kOut> cc;
    cc.setup(bounds, cent, log2nb, lane, ctab0);
    if (CodeCtx<kOut>::kGrid) cc.use_grid = __syncthreads_and(cc.use_grid ? 1 : 0) != 0;
    cc.fill(log2nb, lane, ctab, ctab0);

    // This workgroup's rows: an even share [r_begin, r_end) of all rows, taken rpg rows per group
    // (the last group of the share may be partial), so every workgroup does the same work.
    const int64_t share = (rows + gridDim.x - 1) / gridDim.x;
    const int64_t r_begin = min<int64_t>(rows, static_cast<int64_t>(blockIdx.x) * share);
    const int64_t r_end = min<int64_t>(rows, r_begin + share);
    const int64_t end_elems = r_end * d;

    // 8 chunks of 16 bytes per thread per group: chunk i covers group elements 8*tid + 2048*i.
    uint4 pre[8];
    auto load_group = [&](int64_t r0) {
        const int64_t e0 = r0 * d + 8 * tid;
        if (r0 * d + kGroup <= end_elems) {
#pragma unroll
            for (int i = 0; i < 8; ++i) pre[i] = *reinterpret_cast<const uint4*>(x + e0 + 2048 * i);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int64_t e = e0 + 2048 * i;
                pre[i] = e < end_elems ? *reinterpret_cast<const uint4*>(x + e) : make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };

    int64_t r0 = r_begin;
    if (r0 < r_end) load_group(r0);
    __syncthreads();  // inverse-permutation scratch consumed by every thread

    for (int it = 0; r0 < r_end; r0 += rpg, ++it) {
        unsigned char* buf = smem + (kBufs == 2 ? (it & 1) * kRowBuf : 0);
        // ---- stage: signs, then scatter each element to its rotated block slot
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint4 m;
            if (kMaskInLds) {
                const uint32_t col = (8u * tid + 2048u * (i % kNC)) & dmask;
                m = *reinterpret_cast<const uint4*>(sg + col);
            } else {
                m = msk[i % kNC];
            }
            const uint32_t mw[4] = {m.x, m.y, m.z, m.w};
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) w[q] = (&pre[i].x)[q] ^ (kTabAddr ? (mw[q] & 0x80008000u) : mw[q]);
            unsigned char* base = buf + (i - (i % kNC)) * kChunkStride;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint16_t h = static_cast<uint16_t>((k & 1) ? (w[k >> 1] >> 16) : (w[k >> 1] & 0xffffu));
                const uint32_t a = kTabAddr ? ((k & 1) ? (mw[k >> 1] >> 15) & 0xfffeu : (mw[k >> 1] << 1) & 0xfffeu)
                                            : addr[(i % kNC) * 8 + k];
                *reinterpret_cast<uint16_t*>(base + a) = h;
            }
        }
        if (r0 + rpg < r_end) load_group(r0 + rpg);
        __syncthreads();

        // A wave whose rows all lie past this workgroup's share (the partial last group) has nothing
        // to compute; with rows spanning several waves (d > 4096) every wave joins the reductions.
        const bool wave_busy = log2nb > 6 || r0 + ((64 * (tid >> 6)) >> log2nb) < r_end;
        if (wave_busy) {
        double acc[kH];
        load_block_fwht(buf + tid * kBlockPitch, acc);

        const int64_t row = r0 + rg;
        const bool valid = row < r_end;

        BlockOut res;
        quantize_block<kOut>(acc, buf + tid * kBlockPitch, log2nb, red, ctab, cc, bounds, cent, eps, scale_bf16, res);
        if (valid) store_block<kOut>(res, out, scale_out, scale_bf16, ex, row, blk, d);
        }
        if (kBufs == 1) __syncthreads();  // every lane has read its block before the buffer is restaged
    }
}

// ---- d <= 4096: one wave per unit of 4096 consecutive elements (4096 / d whole rows, 64
//      blocks, one per lane).  A row never spans waves, so the waves of a workgroup share only the
//      permutation tables and never synchronise after the prologue: each wave stages its unit into
//      its own LDS buffer (LDS operations of one wave execute in order, so its reads see its
//      writes), transforms, quantises and stores, while its next unit's loads are in flight.
constexpr int kUnit = 4096;
constexpr int kWaveBuf = 64 * kBlockPitch;

// LDS addresses as 32-bit integers: a store through an LDS-space pointer formed from the integer
// takes a constant addend into the instruction's offset field.
typedef __attribute__((address_space(3))) uint16_t lds_u16_t;
typedef __attribute__((address_space(3))) unsigned char lds_u8_t;
__device__ __forceinline__ uint32_t lds_address(unsigned char* p) {
    return static_cast<uint32_t>(reinterpret_cast<size_t>((lds_u8_t*)p));
}
__device__ __forceinline__ void lds_store_u16(uint32_t addr, uint16_t v) { *(lds_u16_t*)(size_t)addr = v; }
constexpr int kWaveMaxD = 4096;

template <int kOut>
__global__ void __launch_bounds__(kThreads, 2)
rpbh_wave_bf16_kernel(const uint16_t* __restrict__ x, int64_t rows, int d, int log2d,
                      const int32_t* __restrict__ perm, const int8_t* __restrict__ signs, void* __restrict__ out,
                      void* __restrict__ scale_out, int scale_bf16, const float* __restrict__ bounds, float eps,
                      const float* __restrict__ cent, RowExtra ex) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    clear_words(ex);
    // LDS: [one buffer per wave][scatter offset of each source column, u32[d]][its sign mask,
    // u16[d]][code tables].  The wave buffers come first, at offsets known when compiling, so the
    // d = 4096 staging below folds a wave's buffer base into each store's offset field.
    constexpr int kWaves = kThreads / 64;
    uint32_t* tab_off = reinterpret_cast<uint32_t*>(smem + kWaves * kWaveBuf);
    uint16_t* tab_sgn = reinterpret_cast<uint16_t*>(smem + kWaves * kWaveBuf + 4 * d);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    unsigned char* buf = smem + wave * kWaveBuf;
    uint2* ctab0 = reinterpret_cast<uint2*>(smem + kWaves * kWaveBuf + 6 * d);
    uint2* ctab = ctab0 + wave * (CodeCtx<kOut>::kTabBytes / 8);
    const int log2nb = log2d - 6;
    const uint32_t dmask = static_cast<uint32_t>(d - 1);

    // Destination position j (block j / 64, slot j % 64) takes source column perm[j] with sign
    // signs[j]: the table entry of that column holds j's LDS address within wave 0's buffer (the
    // LDS address of smem plus its offset there) and sign bit.
    const uint32_t lds0 = lds_address(smem);
    // all of this thread's descriptor loads first (d <= 4096: at most 4 each), then the scatter, so
    // their latencies overlap instead of adding up
    constexpr int kTabIters = kWaveMaxD / (4 * kThreads);
    int4 pv[kTabIters];
    uint32_t sv[kTabIters];
#pragma unroll
    for (int it = 0; it < kTabIters; ++it) {
        const int j = 4 * tid + it * 4 * kThreads;
        if (j < d) {
            pv[it] = *reinterpret_cast<const int4*>(perm + j);
            sv[it] = *reinterpret_cast<const uint32_t*>(signs + j);
        }
    }
#pragma unroll
    for (int it = 0; it < kTabIters; ++it) {
        const int j = 4 * tid + it * 4 * kThreads;
        if (j < d) {
            const int pj[4] = {pv[it].x, pv[it].y, pv[it].z, pv[it].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t c = static_cast<uint32_t>(pj[e]) & dmask;
                const uint32_t jj = static_cast<uint32_t>(j + e);
                tab_off[c] = lds0 + (jj >> 6) * kBlockPitch + (jj & 63u) * 2u;
                tab_sgn[c] = (sv[it] >> (8 * e + 7)) & 1u ? 0x8000u : 0u;
            }
        }
    }
    CodeCtx<kOut> cc;
    cc.setup(bounds, cent, log2nb, lane, ctab0);
    if (CodeCtx<kOut>::kGrid) cc.use_grid = __syncthreads_and(cc.use_grid ? 1 : 0) != 0;
    cc.fill(log2nb, lane, ctab, ctab0);
    __syncthreads();   // tables complete

    const int64_t total = rows * static_cast<int64_t>(d);
    const int64_t units = (total + kUnit - 1) / kUnit;
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (kThreads / 64);
    int64_t u = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + wave;

    // chunk i of a unit, for this lane: 8 elements at unit offset 512 i + 8 lane
    uint4 pre[8];
    auto load_unit = [&](int64_t uu) {
        const int64_t e0 = uu * kUnit + 8 * lane;
        if (uu * kUnit + kUnit <= total) {
#pragma unroll
            for (int i = 0; i < 8; ++i) pre[i] = *reinterpret_cast<const uint4*>(x + e0 + 512 * i);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int64_t e = e0 + 512 * i;
                pre[i] = e < total ? *reinterpret_cast<const uint4*>(x + e) : make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };
    if (u < units) load_unit(u);
    const uint32_t row_bytes = static_cast<uint32_t>((d >> 6) * kBlockPitch);
    // A unit's codes are stored after the next unit is staged and its successor's loads issued, so
    // waiting for those loads never waits for the stores as well.
    BlockOut res;
    int64_t res_row = -1;
    const int blk = lane & ((1 << log2nb) - 1);
    // ---- stage: signs, then scatter each element to its rotated block slot (chunk i of the
    // unit lies in row pos >> log2d of the unit, whose blocks start at rb)
    auto stage_chunk = [&](int i, uint32_t rb, uint32_t col) {
        const uint4 m = *reinterpret_cast<const uint4*>(tab_sgn + col);
        const uint4 o0 = *reinterpret_cast<const uint4*>(tab_off + col);
        const uint4 o1 = *reinterpret_cast<const uint4*>(tab_off + col + 4);
        const uint32_t w[4] = {pre[i].x ^ m.x, pre[i].y ^ m.y, pre[i].z ^ m.z, pre[i].w ^ m.w};
        const uint32_t off[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
#pragma unroll
        for (int k = 0; k < 8; ++k)
            lds_store_u16(off[k] + rb, static_cast<uint16_t>((k & 1) ? (w[k >> 1] >> 16) : (w[k >> 1] & 0xffffu)));
    };
    // d = 4096: one row per unit, the wave's buffer at a constant distance from wave 0's, which the
    // compiler folds into each store's offset field
    auto stage_row = [&](uint32_t rb) {
#pragma unroll
        for (int i = 0; i < 8; ++i) stage_chunk(i, rb, 512u * i + 8u * lane);
    };
    for (; u < units; u += nwaves) {
        if (d == kUnit) {
            static_assert(kWaves == 4, "one staging case per wave");
            switch (wave) {
                case 0: stage_row(0u * kWaveBuf); break;
                case 1: stage_row(1u * kWaveBuf); break;
                case 2: stage_row(2u * kWaveBuf); break;
                default: stage_row(3u * kWaveBuf); break;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t pos = 512u * i + 8u * lane;
                stage_chunk(i, static_cast<uint32_t>(wave) * kWaveBuf + (pos >> log2d) * row_bytes, pos & dmask);
            }
        }
        if (res_row >= 0 && res_row < rows) store_block<kOut>(res, out, scale_out, scale_bf16, ex, res_row, blk, d);
        if (u + nwaves < units) load_unit(u + nwaves);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the unit is staged (this wave's LDS writes)

        double acc[kH];
        load_block_fwht(buf + lane * kBlockPitch, acc);
        quantize_block<kOut>(acc, buf + lane * kBlockPitch, log2nb, nullptr, ctab, cc, bounds, cent, eps, scale_bf16, res);
        res_row = u * (kUnit >> log2d) + (lane >> log2nb);
        asm volatile("" ::: "memory");   // this unit's block reads precede the next unit's staging
    }
    if (res_row >= 0 && res_row < rows) store_block<kOut>(res, out, scale_out, scale_bf16, ex, res_row, blk, d);
}

template <int kOut>
hipError_t launch_wave(const RowArgs& a, int log2d, hipStream_t stream) {
    auto kernel = rpbh_wave_bf16_kernel<kOut>;
    const size_t lds = 6 * static_cast<size_t>(a.d) +
                       static_cast<size_t>(kThreads / 64) * (kWaveBuf + CodeCtx<kOut>::kTabBytes);
    int per_cu = 0;
    const hipError_t e = kernel_blocks_per_cu(reinterpret_cast<const void*>(kernel), kThreads, lds, &per_cu);
    if (e != hipSuccess) return e;
    const int64_t cap = static_cast<int64_t>(per_cu) * device_cu_count();
    const int64_t units = (a.rows * a.d + kUnit - 1) / kUnit;
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(cap, (units + kThreads / 64 - 1) / (kThreads / 64)));
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), lds, stream,
                       static_cast<const uint16_t*>(a.x), a.rows, a.d, log2d, a.perm, a.signs, a.out, a.scale,
                       a.scale_bf16 ? 1 : 0, a.bounds, a.eps, a.centroids, RowExtra{a.zero, a.sum, a.clear, a.nclear, a.tiled ? 1 : 0});
    return hipGetLastError();
}

template <int kNC, int kOut>
hipError_t launch_t(const RowArgs& a, int log2d, hipStream_t stream) {
    auto kernel = rpbh_quant_bf16_kernel<kNC, kOut>;
    const int log2nb = log2d - 6;
    const int64_t rpg = kThreads >> log2nb;
    const int64_t ngroups = (a.rows + rpg - 1) / rpg;
    const size_t lds = (kNC >= 4 ? static_cast<size_t>(kRowBuf) + 2 * static_cast<size_t>(a.d) + 64
                                 : 2 * static_cast<size_t>(kRowBuf) + 64) +
                       static_cast<size_t>(kThreads / 64) * CodeCtx<kOut>::kTabBytesRow;
    int per_cu = 0;
    const hipError_t e = kernel_blocks_per_cu(reinterpret_cast<const void*>(kernel), kThreads, lds, &per_cu);
    if (e != hipSuccess) return e;
    const int64_t cap = static_cast<int64_t>(per_cu) * device_cu_count();
    // the fewest workgroups that keep every group count per workgroup at the minimum possible in
    // one resident wave (measured faster than filling every slot with partial last groups)
    const int64_t per_wg = (ngroups + cap - 1) / cap;
    const int grid = static_cast<int>((ngroups + per_wg - 1) / per_wg);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), lds, stream, static_cast<const uint16_t*>(a.x), a.rows,
                       a.d, log2d, log2nb, a.perm, a.signs, a.out, a.scale, a.scale_bf16 ? 1 : 0, a.bounds, a.eps,
                       a.centroids, RowExtra{a.zero, a.sum, a.clear, a.nclear, a.tiled ? 1 : 0});
    return hipGetLastError();
}

template <int kOut>
hipError_t launch_nc(const RowArgs& a, int log2d, hipStream_t stream) {
    if (a.d <= kWaveMaxD) return launch_wave<kOut>(a, log2d, stream);
    switch (a.d / 2048) {
        case 4: return launch_t<4, kOut>(a, log2d, stream);
        case 8: return launch_t<8, kOut>(a, log2d, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool rpbh_quant_bf16_supported(const RowArgs& a) {
    return a.x_bf16 && a.perm != nullptr &&
           (a.out_kind == kRowInt8 || a.out_kind == kRowInt8Asym || a.out_kind == kRowCode4 || a.out_kind == kRowCode2 ||
            a.out_kind == kRowLut4 || a.out_kind == kRowLut2 || a.out_kind == kRowCode3 ||
            a.out_kind == kRowLut3 || a.out_kind == kRowLut6) && a.d >= 64 &&
           a.d <= kMaxD;
}

hipError_t launch_rpbh_quant_bf16(const RowArgs& a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    int log2d = 0;
    while ((1 << log2d) < a.d) ++log2d;
    switch (a.out_kind) {
        case kRowInt8: return launch_nc<kRowInt8>(a, log2d, stream);
        case kRowInt8Asym: return launch_nc<kRowInt8Asym>(a, log2d, stream);
        case kRowCode4: return launch_nc<kRowCode4>(a, log2d, stream);
        case kRowCode2: return launch_nc<kRowCode2>(a, log2d, stream);
        case kRowLut4: return launch_nc<kRowLut4>(a, log2d, stream);
        case kRowLut2: return launch_nc<kRowLut2>(a, log2d, stream);
        case kRowCode3: return launch_nc<kRowCode3>(a, log2d, stream);
        case kRowLut3: return launch_nc<kRowLut3>(a, log2d, stream);
        case kRowLut6: return launch_nc<kRowLut6>(a, log2d, stream);
        default: break;
    }
    return hipErrorInvalidValue;
}

}  // namespace rtq
