/*
 * oracle.c -- the plain, slow CPU oracle for the rotated low-bit linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file.  Only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or constant
 * generator with the HIP implementation.
 *
 * Every step is written the obvious way: an explicit dense rotation matrix,
 * a row-by-column product accumulated in double precision, IEEE fp32 division
 * and round-half-to-even where the method turns a real number into a code,
 * a counting search against codebook boundaries, and a naive triple-loop GEMM.
 * No FWHT, no SIMD intrinsics, no BLAS, no fast-math.  OpenMP only splits
 * independent rows across threads (for timing); it never changes an
 * accumulation order.
 *
 * Citations name the pages this method is described on:
 *   [OQ]  the OrbitQuant article (hotelren.com/news/3376620), sections 1-6;
 *   [CR1] "INT8旋转量化是什么？图像生成模型轻量化全解" (cloud.baidu.com/article/9430339);
 *   [CR2] "量化旋转主模型是什么？一文读懂低比特图像生成模型" (cloud.baidu.com/article/9432521).
 *
 * Readings taken where the pages are silent (each is listed with its reason
 * in the project's design notes): Walsh-Hadamard blocks in natural
 * (Sylvester) order, scaled by 1/sqrt(h); P_pi acts as a gather,
 * (P_pi x)_j = x[perm[j]]; signs are applied before the Hadamard block;
 * the RPBH seed expands through SplitMix64 + Fisher-Yates; INT8 is
 * symmetric absmax/127 with round-half-to-even using the stored scale;
 * codes index centroids in ascending order, ties go to the lower cell;
 * b-bit codes pack LSB-first.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------ */
/* SplitMix64: Steele, Lea & Flood, "Fast splittable pseudorandom number
 * generators" (OOPSLA 2014); the 64-bit finaliser is the one in Vigna's
 * public-domain reference.  [OQ] section 6.3 asks for a standardised RNG for
 * the permutation; this is the generator this implementation standardises. */
static uint64_t orc_sm64(uint64_t *state)
{
    uint64_t z;
    *state += 0x9E3779B97F4A7C15ULL;
    z = *state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

ORC_API void orc_splitmix64_stream(uint64_t seed, int64_t n, uint64_t *out)
{
    uint64_t s = seed;
    for (int64_t i = 0; i < n; ++i) out[i] = orc_sm64(&s);
}

/* RPBH descriptor ([OQ] section 2.3): a uniformly drawn permutation pi of
 * {0..d-1} (Fisher-Yates, from the top index down) and d Rademacher signs,
 * all drawn from one SplitMix64 stream. */
ORC_API int orc_rpbh_descriptor(uint64_t seed, int32_t d, int32_t *perm, int8_t *signs)
{
    uint64_t s = seed;
    if (d <= 0) return -1;
    for (int32_t i = 0; i < d; ++i) perm[i] = i;
    for (int32_t i = d - 1; i >= 1; --i) {
        uint64_t j = orc_sm64(&s) % (uint64_t)(i + 1);
        int32_t tmp = perm[i];
        perm[i] = perm[j];
        perm[j] = tmp;
    }
    for (int32_t k = 0; k < d; ++k) signs[k] = (orc_sm64(&s) >> 63) ? (int8_t)-1 : (int8_t)1;
    return 0;
}

/* Entry (a, b) of the h x h Walsh-Hadamard matrix in natural order. */
static int orc_hadamard_entry(int a, int b)
{
    unsigned v = (unsigned)(a & b);
    int parity = 0;
    while (v) {
        parity ^= 1;
        v &= v - 1;
    }
    return parity ? -1 : 1;
}

/* Dense Pi_d = blkdiag(H_h D_1, ..., H_h D_{d/h}) . P_pi  ([OQ] section 2.3),
 * with H_h normalised by 1/sqrt(h) so that Pi is orthogonal.
 * Row i*h+a of block i has, in column perm[i*h+b], the value
 * H[a][b] * sign[i*h+b] / sqrt(h).  Pi is written row-major, d x d doubles. */
ORC_API int orc_rpbh_dense(int32_t d, int32_t h, const int32_t *perm, const int8_t *signs, double *pi)
{
    if (d <= 0 || h <= 0 || d % h != 0) return -1;
    double norm = 1.0 / sqrt((double)h);
    memset(pi, 0, sizeof(double) * (size_t)d * (size_t)d);
    for (int32_t blk = 0; blk < d / h; ++blk)
        for (int32_t a = 0; a < h; ++a)
            for (int32_t b = 0; b < h; ++b) {
                int32_t row = blk * h + a;
                int32_t col = perm[blk * h + b];
                pi[(size_t)row * d + col] = (double)orc_hadamard_entry(a, b) * (double)signs[blk * h + b] * norm;
            }
    return 0;
}

/* out_r = Pi x_r (or Pi^T x_r when transpose != 0) for every row r of x,
 * summed in double over all d columns, zeros included, then rounded once to
 * fp32.  [OQ] section 2.2 (online x' = Pi x) and section 2.1 (offline
 * W' = W Pi^T, whose row n is Pi w_n). */
ORC_API void orc_rotate_rows(const double *pi, int32_t d, const float *x, int64_t rows, int transpose,
                             double *out64, float *out32)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = x + (size_t)r * d;
        for (int32_t i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int32_t j = 0; j < d; ++j) {
                double p = transpose ? pi[(size_t)j * d + i] : pi[(size_t)i * d + j];
                acc += p * (double)xr[j];
            }
            if (out64) out64[(size_t)r * d + i] = acc;
            if (out32) out32[(size_t)r * d + i] = (float)acc;
        }
    }
}

/* ------------------------------------------------------------------ */
/* bfloat16: the top 16 bits of an IEEE binary32, rounded to nearest-even.
 * [OQ] section 2.1 keeps row norms in BF16.  Rounding is done in one step
 * from double: find the binade, scale so one bf16 ulp is 1.0, round half to
 * even, scale back.  Subnormal bf16 values have a fixed ulp of 2^-133. */
static uint16_t orc_double_to_bf16(double x)
{
    if (isnan(x)) return (uint16_t)0x7FC0;
    if (x == 0.0) return signbit(x) ? (uint16_t)0x8000 : (uint16_t)0x0000;
    if (isinf(x)) return x > 0 ? (uint16_t)0x7F80 : (uint16_t)0xFF80;
    int e;
    (void)frexp(x, &e);          /* |x| = m * 2^e with 0.5 <= m < 1 */
    int ulp_exp = e - 8;         /* 8 significant bits in bf16 */
    if (ulp_exp < -133) ulp_exp = -133;
    double r = nearbyint(ldexp(x, -ulp_exp)); /* default mode: ties to even */
    double y = ldexp(r, ulp_exp);
    float yf = (float)y;          /* exact unless it overflows */
    uint32_t bits;
    memcpy(&bits, &yf, sizeof bits);
    if (isinf(yf)) return (uint16_t)(bits >> 16);
    return (uint16_t)(bits >> 16);
}

static float orc_bf16_value(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

ORC_API void orc_to_bf16(const double *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_double_to_bf16(x[i]);
}

/* ------------------------------------------------------------------ */
/* Symmetric per-row INT8 ([CR2] section 4: q = round(R W / s); [CR1]
 * section 3 stores one scale per channel).  s = max_j |v_j| / 127 in fp32;
 * the scale is stored (fp32, or bf16 when scale_is_bf16) and the STORED
 * value divides; q = round-half-even(v / s), clamped to [-127, 127].
 * A zero row gets s = 0 and q = 0.  pre (optional) receives v / s, the fp32
 * value that round-half-even turns into the code. */
ORC_API void orc_quant_int8_rows(const float *v, int64_t rows, int32_t d, int scale_is_bf16, int8_t *q,
                                 float *scale_out, float *pre)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float *vr = v + (size_t)r * d;
        float amax = 0.0f;
        for (int32_t j = 0; j < d; ++j) {
            float a = fabsf(vr[j]);
            if (a > amax) amax = a;
        }
        float s = amax / 127.0f;
        if (scale_is_bf16) s = orc_bf16_value(orc_double_to_bf16((double)s));
        scale_out[r] = s;
        for (int32_t j = 0; j < d; ++j) {
            int code = 0;
            float t = 0.0f;
            if (s != 0.0f) {
                t = vr[j] / s;
                float rq = nearbyintf(t);
                if (rq > 127.0f) rq = 127.0f;
                if (rq < -127.0f) rq = -127.0f;
                code = (int)rq;
            }
            q[(size_t)r * d + j] = (int8_t)code;
            if (pre) pre[(size_t)r * d + j] = t;
        }
    }
}

/* Asymmetric INT8 rows: the scale-and-zero-point form of INT8 ([CR1] section 3 lists per-channel
 * scales and zero points; [CR3] computes a scale and a zero-point offset), per row.  The range is
 * widened to contain 0 so that 0 is an exact code: lo = min(min_j v_j, 0), hi = max(max_j v_j, 0),
 * s = fl32(fl32(hi - lo) / 255), stored as bf16 for weights; with the STORED s,
 * z = clamp(-128 - rne(fl32(lo / s)), -128, 127) and q_j = clamp(rne(fl32(v_j / s)) + z, -128, 127),
 * so v_j ~ s (q_j - z).  s == 0 (an all-zero row) gives q = 0 and z = 0.  Outputs also the row's
 * code sum and (optional) the pre-rounding fl32(v_j / s). */
ORC_API void orc_quant_int8_asym_rows(const float *v, int64_t rows, int32_t d, int scale_is_bf16, int8_t *q,
                                      float *scale_out, int32_t *zero_out, int64_t *sum_out, float *pre)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float *vr = v + (size_t)r * d;
        float lo = 0.0f, hi = 0.0f;
        for (int32_t j = 0; j < d; ++j) {
            if (vr[j] < lo) lo = vr[j];
            if (vr[j] > hi) hi = vr[j];
        }
        float s = (hi - lo) / 255.0f;
        if (scale_is_bf16) s = orc_bf16_value(orc_double_to_bf16((double)s));
        int z = 0;
        if (s != 0.0f) {
            float zr = -128.0f - nearbyintf(lo / s);
            if (zr > 127.0f) zr = 127.0f;
            if (zr < -128.0f) zr = -128.0f;
            z = (int)zr;
        }
        scale_out[r] = s;
        zero_out[r] = z;
        int64_t sum = 0;
        for (int32_t j = 0; j < d; ++j) {
            int code = 0;
            float t = 0.0f;
            if (s != 0.0f) {
                t = vr[j] / s;
                float rq = nearbyintf(t) + (float)z;
                if (rq > 127.0f) rq = 127.0f;
                if (rq < -128.0f) rq = -128.0f;
                code = (int)rq;
            }
            q[(size_t)r * d + j] = (int8_t)code;
            sum += code;
            if (pre) pre[(size_t)r * d + j] = t;
        }
        sum_out[r] = sum;
    }
}

/* The product of asymmetric codes, from its definition: acc[t][n] = sum_j (qa - za_t)(qw - zw_n),
 * a naive int64 triple loop. */
ORC_API void orc_gemm_int8_asym(const int8_t *qa, const int32_t *za, const int8_t *qw, const int32_t *zw,
                                int64_t T, int64_t N, int32_t d, int64_t *acc)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < N; ++n) {
            int64_t a = 0;
            for (int32_t j = 0; j < d; ++j)
                a += ((int64_t)qa[(size_t)t * d + j] - za[t]) * ((int64_t)qw[(size_t)n * d + j] - zw[n]);
            acc[(size_t)t * N + n] = a;
        }
}

/* Codebook rows ([OQ] section 2.1 steps 2-3 for weights, section 2.2 steps
 * 2-4 for activations).  The row's L2 norm is summed in double and rounded
 * once to fp32.  Weights (is_weight != 0): direction u = v / r in fp32
 * (r = 0 gives u = 0) and the stored norm is bf16(r).  Activations:
 * u = v / (s + eps) in fp32 and the stored norm is s in fp32.
 * code_j = number of boundaries t_k with t_k < u_j (ascending centroids,
 * ties fall to the lower cell).  codes are one byte per element here;
 * orc_pack packs them.  u_out (optional) receives u. */
ORC_API void orc_quant_codebook_rows(const float *v, int64_t rows, int32_t d, int is_weight, float eps,
                                     int32_t nbound, const float *bounds, uint8_t *codes, float *norm_out,
                                     float *u_out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float *vr = v + (size_t)r * d;
        double ss = 0.0;
        for (int32_t j = 0; j < d; ++j) ss += (double)vr[j] * (double)vr[j];
        float nrm = (float)sqrt(ss);
        float denom;
        if (is_weight) {
            denom = nrm;
            norm_out[r] = orc_bf16_value(orc_double_to_bf16((double)nrm));
        } else {
            denom = nrm + eps;
            norm_out[r] = nrm;
        }
        for (int32_t j = 0; j < d; ++j) {
            float u = (denom == 0.0f) ? 0.0f : vr[j] / denom;
            int code = 0;
            for (int32_t k = 0; k < nbound; ++k)
                if (bounds[k] < u) ++code;
            codes[(size_t)r * d + j] = (uint8_t)code;
            if (u_out) u_out[(size_t)r * d + j] = u;
        }
    }
}

/* b-bit packing, least-significant bits first: the codes of a row form one little-endian bit
 * stream, element j in bits [j*b, j*b + b).  For b = 2 and 4 this is byte j*b/8 at bit offset
 * (j mod 8/b)*b; for b = 3 and 6 a code may straddle two bytes (8 3-bit codes per 3 bytes, 4
 * 6-bit codes per 3 bytes).  bits is 2, 3, 4, 6 or 8 (8 is a copy); d*b must be a multiple of 8. */
static int pack_bits_ok(int32_t d, int32_t bits)
{
    if (bits != 2 && bits != 3 && bits != 4 && bits != 6 && bits != 8) return 0;
    return ((int64_t)d * bits) % 8 == 0;
}

ORC_API int orc_pack(const uint8_t *codes, int64_t rows, int32_t d, int32_t bits, uint8_t *packed)
{
    if (!pack_bits_ok(d, bits)) return -1;
    int64_t row_bytes = (int64_t)d * bits / 8;
    memset(packed, 0, (size_t)(rows * row_bytes));
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t j = 0; j < d; ++j) {
            unsigned c = codes[(size_t)r * d + j] & ((1u << bits) - 1u);
            for (int b = 0; b < bits; ++b) {
                int64_t bit = (int64_t)j * bits + b;
                if ((c >> b) & 1u) packed[(size_t)(r * row_bytes + bit / 8)] |= (uint8_t)(1u << (bit % 8));
            }
        }
    return 0;
}

ORC_API int orc_unpack(const uint8_t *packed, int64_t rows, int32_t d, int32_t bits, uint8_t *codes)
{
    if (!pack_bits_ok(d, bits)) return -1;
    int64_t row_bytes = (int64_t)d * bits / 8;
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t j = 0; j < d; ++j) {
            unsigned c = 0;
            for (int b = 0; b < bits; ++b) {
                int64_t bit = (int64_t)j * bits + b;
                c |= (unsigned)((packed[(size_t)(r * row_bytes + bit / 8)] >> (bit % 8)) & 1u) << b;
            }
            codes[(size_t)r * d + j] = (uint8_t)c;
        }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Lloyd-Max codebook for N(0, 1/d) ([OQ] section 1 and section 4.2: one
 * codebook per input dimension d, precomputed offline).  The iteration runs
 * on N(0,1): boundaries are midpoints of neighbouring centroids, centroids
 * are conditional means of the cell, E[X | a < X < b] =
 * (phi(a) - phi(b)) / (Phi(b) - Phi(a)).  It starts from L evenly spaced
 * points on [-2, 2] and stops when no centroid moves by 1e-15 or more.
 * The result is made exactly symmetric, scaled by 1/sqrt(d), and rounded to
 * fp32; each fp32 boundary is the midpoint of the scaled double centroids. */
static double orc_phi(double x) { return exp(-0.5 * x * x) / sqrt(2.0 * M_PI); }
static double orc_upper_tail(double x) { return 0.5 * erfc(x / sqrt(2.0)); }  /* P(X > x) */
static double orc_lower_tail(double x) { return 0.5 * erfc(-x / sqrt(2.0)); } /* P(X < x) */

static double orc_cell_mass(double a, double b) /* P(a < X < b), a < b, infinities allowed */
{
    if (a >= 0.0) return orc_upper_tail(a) - orc_upper_tail(b);
    if (b <= 0.0) return orc_lower_tail(b) - orc_lower_tail(a);
    return 1.0 - orc_lower_tail(a) - orc_upper_tail(b);
}

static double orc_cell_mean(double a, double b)
{
    double pa = isinf(a) ? 0.0 : orc_phi(a);
    double pb = isinf(b) ? 0.0 : orc_phi(b);
    return (pa - pb) / orc_cell_mass(a, b);
}

ORC_API int orc_lloyd_max(int32_t bits, int32_t d, double *c_unit, double *t_unit, float *c32, float *t32)
{
    if (bits < 1 || bits > 8 || d <= 0) return -1;
    int L = 1 << bits;
    double *c = (double *)malloc(sizeof(double) * L);
    double *t = (double *)malloc(sizeof(double) * (L + 1));
    for (int k = 0; k < L; ++k) c[k] = -2.0 + 4.0 * (double)k / (double)(L - 1);
    int iters = 0;
    for (;;) {
        t[0] = -INFINITY;
        t[L] = INFINITY;
        for (int k = 1; k < L; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
        double moved = 0.0;
        for (int k = 0; k < L; ++k) {
            double nc = orc_cell_mean(t[k], t[k + 1]);
            double dlt = fabs(nc - c[k]);
            if (dlt > moved) moved = dlt;
            c[k] = nc;
        }
        ++iters;
        if (moved < 1e-15 || iters >= 2000000) break;
    }
    for (int k = 0; k < L / 2; ++k) {
        double m = 0.5 * (c[L - 1 - k] - c[k]);
        c[k] = -m;
        c[L - 1 - k] = m;
    }
    double inv_sqrt_d = 1.0 / sqrt((double)d);
    for (int k = 0; k < L; ++k) {
        if (c_unit) c_unit[k] = c[k];
        if (c32) c32[k] = (float)(c[k] * inv_sqrt_d);
    }
    for (int k = 0; k + 1 < L; ++k) {
        double tu = 0.5 * (c[k] + c[k + 1]);
        if (t_unit) t_unit[k] = tu;
        if (t32) t32[k] = (float)(0.5 * (c[k] * inv_sqrt_d + c[k + 1] * inv_sqrt_d));
    }
    free(c);
    free(t);
    return iters;
}

/* ------------------------------------------------------------------ */
/* INT8 x INT8 product by the definition: acc[t][n] = sum_j a[t][j] * w[n][j]
 * in 64-bit integers ([OQ] section 2.2: the rotation cancels inside W'x'). */
ORC_API void orc_gemm_int8(const int8_t *a, const int8_t *w, int64_t T, int64_t N, int32_t d, int64_t *acc)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int32_t j = 0; j < d; ++j) s += (int64_t)a[(size_t)t * d + j] * (int64_t)w[(size_t)n * d + j];
            acc[(size_t)t * N + n] = s;
        }
}

/* y[t][n] = acc[t][n] * a_scale[t] * w_scale[n], in double ([CR2] section 4:
 * the dequantised value is s * q; both operands carry their own scale). */
ORC_API void orc_rescale_int8(const int64_t *acc, const float *a_scale, const float *w_scale, int64_t T,
                              int64_t N, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < N; ++n)
            y[(size_t)t * N + n] = (double)acc[(size_t)t * N + n] * (double)a_scale[t] * (double)w_scale[n];
}

/* Codebook product ([OQ] sections 2.1-2.2): x_hat = s * c_a[code], w_hat =
 * r * c_w[code], y[t][n] = r[n] * s[t] * sum_j c_w[qw[n][j]] * c_a[qa[t][j]],
 * summed in double.  Codes are one byte per element (unpacked). */
ORC_API void orc_gemm_codebook(const uint8_t *qa, const uint8_t *qw, const float *ca, const float *cw,
                               const float *s_a, const float *r_w, int64_t T, int64_t N, int32_t d, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int32_t j = 0; j < d; ++j)
                s += (double)cw[qw[(size_t)n * d + j]] * (double)ca[qa[(size_t)t * d + j]];
            y[(size_t)t * N + n] = (double)r_w[n] * (double)s_a[t] * s;
        }
}

/* Reference product of the unquantised layer, y = W x in double. */
ORC_API void orc_matmul_f64(const float *x, const float *w, int64_t T, int64_t N, int32_t d, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int32_t j = 0; j < d; ++j) s += (double)w[(size_t)n * d + j] * (double)x[(size_t)t * d + j];
            y[(size_t)t * N + n] = s;
        }
}

ORC_API int orc_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
