// codebook_int8.h -- Lloyd-Max codebooks as int8 values for the INT8 matrix cores.
//
// A codebook c_0 < ... < c_{L-1} (the quantiser's reconstruction points, OrbitQuant article, 2.1
// and 4.2) is used in the product as v_k = rint(c_k * S) with S = 127 / max_k |c_k|: the largest
// centroid maps to +-127 and every product carries a factor 1/S, applied with the row scales.
// Both the activation quantiser (which writes v_k per element) and the GEMM (which decodes packed
// weight codes to v_k) derive the table from the same device centroids with these same fp32
// operations, so they agree bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rtq {

// S for a codebook of L centroids (device pointer; every lane reads the same values).
__device__ __forceinline__ float codebook_int8_scale(const float* c, int L) {
    float m = 0.0f;
    for (int k = 0; k < L; ++k) m = fmaxf(m, fabsf(c[k]));
    return 127.0f / m;
}

// The value v_k of one entry (any L, e.g. the 64 of a 6-bit codebook held one per lane).
__device__ __forceinline__ int codebook_int8_value(const float* c, int k, float s) {
    return static_cast<int>(rintf(c[k] * s));
}

// The L <= 16 values v_k as bytes: entry k in byte k % 4 of word k / 4.
__device__ __forceinline__ void codebook_int8_table(const float* c, int L, float s, uint32_t (&lut)[4]) {
    lut[0] = lut[1] = lut[2] = lut[3] = 0u;
    for (int k = 0; k < L; ++k) {
        const uint32_t v = static_cast<uint32_t>(codebook_int8_value(c, k, s)) & 0xffu;
        lut[k >> 2] |= v << (8 * (k & 3));
    }
}

// 4 codes (one per byte, 0..15) -> their 4 int8 values.  v_perm_b32 picks bytes 0-7 of a table
// pair; selector byte 12 gives 0x00 and 13 gives 0xFF, which builds the select mask for codes >= 8.
__device__ __forceinline__ uint32_t lut16_x4(const uint32_t (&lut)[4], uint32_t b) {
    const uint32_t lo = __builtin_amdgcn_perm(lut[1], lut[0], b);
    const uint32_t hi = __builtin_amdgcn_perm(lut[3], lut[2], b & 0x07070707u);
    const uint32_t m = __builtin_amdgcn_perm(0u, 0u, ((b >> 3) & 0x01010101u) | 0x0C0C0C0Cu);
    return (hi & m) | (lo & ~m);
}

// 4 codes (one per byte, 0..7) -> their 4 int8 values (table in lut[0..1]).
__device__ __forceinline__ uint32_t lut8_x4(const uint32_t (&lut)[4], uint32_t b) {
    return __builtin_amdgcn_perm(lut[1], lut[0], b);
}

// 4 codes (one per byte, 0..3) -> their 4 int8 values (table in lut[0]).
__device__ __forceinline__ uint32_t lut4_x4(const uint32_t (&lut)[4], uint32_t b) {
    return __builtin_amdgcn_perm(lut[0], lut[0], b);
}

}  // namespace rtq
