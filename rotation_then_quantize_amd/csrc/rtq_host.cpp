// rtq_host.cpp -- host-only helpers of librtq: the seeded RPBH descriptor and the Lloyd-Max codebook.
#include <cmath>
#include <cstdint>
#include <utility>
#include <vector>

#include "rtq_host.h"

namespace rtq {

// SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): a Weyl sequence with step 0x9E3779B97F4A7C15
// pushed through the 64-bit variant-13 finaliser.
namespace {
struct SplitMix64 {
    uint64_t state;
    uint64_t next() {
        state += 0x9E3779B97F4A7C15ULL;
        uint64_t z = state;
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
        return z ^ (z >> 31);
    }
};
}  // namespace

// The descriptor of Pi_d = blkdiag(H D_1..H D_{d/h}) P_pi (OrbitQuant article, 2.3), drawn from one
// stream so every platform rebuilds the same rotation from the seed (OrbitQuant article, 6.3).
void make_rpbh(uint64_t seed, int32_t d, int32_t* perm, int8_t* signs) {
    SplitMix64 g{seed};
    for (int32_t i = 0; i < d; ++i) perm[i] = i;
    for (int32_t i = d - 1; i > 0; --i) {
        const uint64_t j = g.next() % static_cast<uint64_t>(i + 1);
        std::swap(perm[i], perm[j]);
    }
    for (int32_t k = 0; k < d; ++k) signs[k] = static_cast<int8_t>((g.next() >> 63) ? -1 : 1);
}

// Lloyd-Max quantiser for N(0,1), computed on the positive half-line and mirrored (the density is
// symmetric and log-concave, so the optimum is symmetric and unique).  Positive levels m_0 < ... <
// m_{L/2-1}; cell edges e_0 = 0, e_k = (m_{k-1} + m_k)/2, e_{L/2} = +inf; each level moves to its
// cell's conditional mean (phi(a) - phi(b)) / (Q(a) - Q(b)), Q the upper tail, until no level moves
// by 1e-15.  Then scaled to N(0, 1/d) (OrbitQuant article, 1 and 4.2) and rounded to fp32.
namespace {
double pdf(double x) { return std::exp(-0.5 * x * x) * 0.39894228040143267794; }
double upper(double x) { return std::isinf(x) ? 0.0 : 0.5 * std::erfc(x * 0.70710678118654752440); }
}  // namespace

int lloyd_max(int32_t d, int32_t bits, float* centroids, float* boundaries) {
    const int L = 1 << bits;
    const int H = L / 2;
    std::vector<double> m(H), e(H + 1);
    for (int k = 0; k < H; ++k) m[k] = 3.0 * (k + 0.5) / H;  // any increasing start converges
    int it = 0;
    for (; it < 4000000; ++it) {
        e[0] = 0.0;
        for (int k = 1; k < H; ++k) e[k] = 0.5 * (m[k - 1] + m[k]);
        e[H] = INFINITY;
        double moved = 0.0;
        for (int k = 0; k < H; ++k) {
            const double a = e[k], b = e[k + 1];
            const double num = pdf(a) - (std::isinf(b) ? 0.0 : pdf(b));
            const double nm = num / (upper(a) - upper(b));
            moved = std::fmax(moved, std::fabs(nm - m[k]));
            m[k] = nm;
        }
        if (moved < 1e-15) break;
    }
    std::vector<double> c(L);
    for (int k = 0; k < H; ++k) {
        c[H + k] = m[k];
        c[H - 1 - k] = -m[k];
    }
    const double inv = 1.0 / std::sqrt(static_cast<double>(d));
    for (int k = 0; k < L; ++k) centroids[k] = static_cast<float>(c[k] * inv);
    for (int k = 0; k + 1 < L; ++k) boundaries[k] = static_cast<float>(0.5 * (c[k] * inv + c[k + 1] * inv));
    return it;
}

}  // namespace rtq
