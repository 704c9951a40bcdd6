// rtq_host.h -- host-only helpers of librtq (descriptor generator, Lloyd-Max codebook).
#pragma once
#include <cstdint>

namespace rtq {
void make_rpbh(uint64_t seed, int32_t d, int32_t* perm, int8_t* signs);
int lloyd_max(int32_t d, int32_t bits, float* centroids, float* boundaries);
}  // namespace rtq
