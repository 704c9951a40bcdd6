/*
 * rtq.h -- C ABI of librtq: rotate-then-quantize linear layers on AMD MI355X (gfx950).
 *
 * The method (OrbitQuant article, hotelren.com/news/3376620, sections 2.1-2.3):
 *   offline   W' = W Pi_d^T; each row of W' is quantised (INT8 with a per-row scale, or a bf16
 *             row norm r' plus Lloyd-Max codes of the direction w'/r');
 *   online    x' = Pi_d x; per token the scale (INT8) or norm s = ||x'|| (codebook) is taken,
 *             x' is quantised, and the quantised product W'x' is formed; Pi^T Pi = I cancels,
 *             so no inverse rotation runs at inference time;
 *   Pi_d      = blkdiag(H_64 D_1, ..., H_64 D_{d/64}) P_pi  (random-permutation block Hadamard,
 *             RPBH), with H_64 the natural-order Walsh-Hadamard matrix scaled by 1/8, D_i
 *             Rademacher sign matrices and P_pi a permutation acting as a gather,
 *             (P_pi x)_j = x[perm[j]].
 * The uniform INT8 variant (q = round(v/s), s = max|v|/127, symmetric) follows
 * "量化旋转主模型是什么？一文读懂低比特图像生成模型" (cloud.baidu.com/article/9432521), section 4.
 *
 * Conventions shared by every call
 *   - Row-major storage.  x is [rows][d]; weights are [N][d] as in y = W x; y is [T][N].
 *   - Device pointers are allocated and freed by the caller; the library allocates no device
 *     memory and keeps no state besides a thread-local error string and per-device kernel
 *     attributes.  Device pointers must be 16-byte aligned (else RTQ_ERR_MISALIGNED).
 *   - Device calls are asynchronous on `stream` (a hipStream_t passed as void*, NULL = the
 *     default stream).  Arguments are checked on the host before anything is enqueued; on any
 *     non-OK status nothing was enqueued and rtq_last_error() describes the problem.  Faults
 *     during execution surface at the caller's next synchronisation.
 *   - d must be a multiple of 64 with d/64 a power of two, 64 <= d <= 16384 (the block size h is
 *     64); other shapes return RTQ_ERR_UNSUPPORTED.
 *   - Inputs are finite.  perm must be a permutation of 0..d-1 and signs must be +1/-1; other
 *     values give unspecified results (never an out-of-bounds access).
 */
#ifndef RTQ_H
#define RTQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RTQ_OK = 0,
    RTQ_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, inconsistent arguments    */
    RTQ_ERR_UNSUPPORTED = -2, /* valid but not implemented: d shape, dtype combination, bits */
    RTQ_ERR_MISALIGNED = -3,  /* a device pointer is not 16-byte aligned                     */
    RTQ_ERR_HIP = -4          /* the HIP runtime refused a call (message from hipGetErrorString) */
} rtq_status;

typedef enum {
    RTQ_F32 = 0,  /* IEEE binary32                                               */
    RTQ_BF16 = 1, /* bfloat16 bit patterns (uint16), rounded to nearest-even      */
    RTQ_I32 = 2   /* int32 accumulators: rtq_qgemm output (INT8, CODEBOOK_I8)   */
} rtq_dtype;

typedef enum {
    RTQ_INT8 = 0,     /* symmetric INT8, scale = max|v|/127, codes in [-127, 127]       */
    RTQ_CODEBOOK = 1, /* L2 norm + Lloyd-Max direction codes of `bits` bits, packed     */
    RTQ_CODEBOOK_I8 = 2, /* the same Lloyd-Max codes, multiplied on the INT8 matrix cores:
                         * each codebook enters the product as v_k = rint(c_k * S),
                         * S = 127 / max_k |c_k| (largest centroid -> +-127), and y is
                         * rescaled by 1/(S_a S_w).  Activations are then stored as their
                         * int8 values v[code] (1 byte per element, not packed); weights
                         * stay packed codes.  Relative Frobenius error of y against the
                         * exact-centroid product: ~0.9% (W4A4) / ~0.5% (W2A4) on the DiT
                         * synthetic shapes, inside the 2e-2 bound for bf16 outputs.    */
    RTQ_INT8_TILED = 3, /* RTQ_INT8 codes and scales, with the codes stored in the product's tiled
                         * layout: rows in tiles of 256 (padded to a multiple of 256; padding rows
                         * are neither written nor read as results), K in slices of 64 bytes;
                         * block (tile, slice) is 16 KB contiguous at
                         * ((row / 256) * (d / 64) + j / 64) * 16384, holding [256 rows][64 bytes],
                         * and within a row's 64 bytes the 16-byte chunk c (bytes j = 16c .. of
                         * the slice) sits at chunk c ^ ((row >> 2) & 3).  It is the image of one
                         * LDS stage of the INT8 product, whose operand loads then read whole 1 KB
                         * runs (about 7% faster products at the DiT shapes than row-major codes).
                         * A codes buffer holds ceil(rows / 256) * 256 * d bytes.            */
    RTQ_CODEBOOK_TILED = 4, /* RTQ_CODEBOOK codes and norms (weights: packed 2-, 3- or 4-bit
                         * codes), with the codes stored in the tiled code layout: the same tiles
                         * of 256 rows (padded; padding rows neither written nor read as results)
                         * and K slices of 64 elements; block (tile, slice) is contiguous at
                         * ((row / 256) * (d / 64) + j / 64) * 256 * 8 * bits bytes and holds
                         * [256 rows][8 * bits bytes], a row's bytes being exactly its packed
                         * codes of elements 64 * (j / 64) .. +64 as in the row-major bit stream.
                         * It is the image of one raw code slot of the product.  Written by
                         * rtq_quantize_rows; multiplied in RTQ_CODEBOOK_I8_TILED.  A codes
                         * buffer holds ceil(rows / 256) * 256 * d * bits / 8 bytes.          */
    RTQ_CODEBOOK_I8_TILED = 5 /* RTQ_CODEBOOK_I8 with both operands tiled: activations' int8
                         * codebook values in RTQ_INT8_TILED's layout (rtq_quantize_rows in this
                         * mode; ceil(rows / 256) * 256 * d bytes), weight codes in
                         * RTQ_CODEBOOK_TILED's.  Products equal RTQ_CODEBOOK_I8's bit for bit
                         * and are 7-10% faster at the DiT shapes.                           */
} rtq_qmode;

/* RPBH descriptor (OrbitQuant article, section 2.3).  perm (int32[d]) and signs (int8[d], +-1)
 * are DEVICE pointers; h must be 64.  The same descriptor must rotate a layer's weights offline
 * and its activations online (section 2.2: the two rotations cancel only if they are equal). */
typedef struct {
    int32_t d;
    int32_t h;
    const int32_t* perm;
    const int8_t* signs;
} rtq_rpbh;

/* Lloyd-Max codebook for N(0, 1/d) (OrbitQuant article, sections 1 and 4.2).  centroids holds
 * 2^bits ascending fp32 values, boundaries the 2^bits - 1 fp32 cell edges; DEVICE pointers.
 * Code k stands for centroids[k]; a value u gets code #{k : boundaries[k] < u}. */
typedef struct {
    int32_t bits;
    const float* centroids;
    const float* boundaries;
} rtq_codebook;

/* ---------------------------------------------------------------- host-only helpers */

/* Build an RPBH descriptor from a seed (OrbitQuant article, section 6.3 asks for a standardised
 * generator).  SplitMix64 stream from `seed`; perm starts as the identity and is shuffled by
 * Fisher-Yates from index d-1 down to 1 (j = next() mod (i+1)); then signs[k] = -1 if the top bit
 * of next() is set, else +1.  perm_out (int32[d]) and signs_out (int8[d]) are HOST pointers.
 * Errors: RTQ_ERR_INVALID_ARG for null pointers or d <= 0 or d % h != 0; h must be 64. */
rtq_status rtq_rpbh_make(uint64_t seed, int32_t d, int32_t h, int32_t* perm_out, int8_t* signs_out);

/* Lloyd-Max codebook for N(0, 1/d) with 2^bits levels (OrbitQuant article, section 4.2: one
 * codebook per input dimension, computed offline).  Computed in double on N(0,1), made exactly
 * symmetric, scaled by 1/sqrt(d) and rounded to fp32; each boundary is the fp32 rounding of the
 * midpoint of the two neighbouring scaled centroids.  centroids_out (float[2^bits]) and
 * boundaries_out (float[2^bits - 1]) are HOST pointers.  bits in 1..8. */
rtq_status rtq_lloyd_max(int32_t d, int32_t bits, float* centroids_out, float* boundaries_out);

/* ---------------------------------------------------------------- device calls */

/* y = Pi x for each row (inverse = 0), or x = Pi^T y (inverse = 1): the RPBH rotation alone
 * (OrbitQuant article, sections 2.2-2.3).  x: [rows][R->d] of xt (F32 or BF16); y: [rows][R->d] of
 * yt (F32 or BF16).  The transform is evaluated exactly in double and rounded once to fp32; a
 * BF16 output is that fp32 value rounded to nearest-even.  rows == 0 is a no-op. */
rtq_status rtq_rpbh_rotate(const void* x, rtq_dtype xt, void* y, rtq_dtype yt, int64_t rows,
                           const rtq_rpbh* R, int32_t inverse, void* stream);

/* Rotate (when R != NULL) and quantise rows (OrbitQuant article, section 2.1 steps 1-3 for weights,
 * section 2.2 steps 1-4 for activations; the INT8 rule of cloud.baidu.com/article/9432521, section 4).
 *   x      [rows][d] of xt (F32 or BF16).  R == NULL: x is already rotated.  R != NULL: R->d == d.
 *   INT8:      s = max_j |x'_j| / 127 in fp32, stored as scale_t (F32 or BF16); the STORED value
 *              divides: q_j = round-half-even(x'_j / s), clamped to [-127, 127]; s == 0 gives q = 0.
 *              codes: int8[rows][d].  cb must be NULL.  eps is ignored.
 *   INT8_TILED: the same codes and scales, codes written in the tiled layout (RTQ_INT8_TILED).
 *   CODEBOOK_TILED, CODEBOOK_I8_TILED: the CODEBOOK / CODEBOOK_I8 codes and norms below, codes
 *              written in the tiled layouts (see the modes); the same kernels and bits.
 *   CODEBOOK:  s = ||x'||_2 (summed in double, rounded to fp32); u_j = x'_j / (s + eps) in fp32
 *              (0 when s + eps == 0); code_j = #{k : boundaries[k] < u_j}.  The norm s is stored as
 *              scale_t: BF16 for weights (eps = 0), F32 for activations (eps > 0, e.g. 1e-8).
 *              codes: uint8[rows][d * bits / 8], the row's codes as one little-endian bit stream,
 *              element j in bits [j*bits, j*bits + bits) (least significant first; for 2 and 4
 *              bits: byte j*bits/8, bit (j mod 8/bits)*bits).  cb->bits 2, 3 or 4 (the 3-bit codes
 *              of the W3A3 variant, OrbitQuant article 3.2-3.3, need BF16 x and R != NULL).
 *   CODEBOOK_I8: the CODEBOOK codes, written as their int8 codebook values v[code] (see
 *              RTQ_CODEBOOK_I8): codes int8[rows][d].  cb needs centroids and boundaries;
 *              cb->bits 2, 3, 4 or 6 (3 and 6, as for W3A3 / W4A6 activations, need BF16 x and
 *              R != NULL; 6-bit codes are searched among the row's exact thresholds for d >= 4096,
 *              and counted boundary by boundary below that).
 *   scale  [rows] of scale_t.
 * rows == 0 is a no-op. */
rtq_status rtq_quantize_rows(const void* x, rtq_dtype xt, int64_t rows, int32_t d, const rtq_rpbh* R,
                             rtq_qmode mode, const rtq_codebook* cb, float eps, void* codes, void* scale,
                             rtq_dtype scale_t, void* stream);

/* The quantised product in which the rotation has cancelled (OrbitQuant article, section 2.2:
 * W'x' = W Pi^T Pi x).
 *   a_codes [T][d] (INT8) or [T][d*bits_a/8] packed (CODEBOOK), a_scale fp32[T] (INT8 scale or
 *   token norm); w_codes [N][d] or [N][d*bits_w/8], w_scale [N] of w_scale_t (F32 or BF16).
 *   INT8, INT8_TILED (both operands' codes in the tiled layout):
 *              acc[t][n] = sum_j a[t][j] w[n][j] exactly in int32 (|acc| <= 127^2 d);
 *              y = acc * a_scale[t] * w_scale[n] (fp32 arithmetic), stored as yt (F32 or BF16);
 *              yt == RTQ_I32 stores acc itself.  cb_a and cb_w must be NULL.  N <= 2^22 for BF16
 *              output, N <= 2^21 for F32 and I32 (else RTQ_ERR_UNSUPPORTED).
 *   CODEBOOK:  y = w_scale[n] * a_scale[t] * sum_j cb_w->centroids[qw] * cb_a->centroids[qa],
 *              accumulated in fp32 from fp16 copies of the centroids; yt must be BF16.
 *              cb_a->bits must be 4; cb_w->bits 2 or 4.
 *   CODEBOOK_I8: a_codes int8[T][d] holds the activations' int8 codebook values (rtq_quantize_rows
 *              in this mode), w_codes packed codes [N][d*bits_w/8]; acc = sum_j a[t][j] v_w[qw]
 *              exactly in int32, y = acc * a_scale[t] * w_scale[n] / (S_a S_w) in fp32; yt BF16,
 *              or RTQ_I32 for acc itself.  cb_a (centroids, bits 2, 3, 4 or 6) gives S_a; cb_w
 *              (centroids, bits 2, 3 or 4) the weight values.  N <= 2^22 (BF16), 2^21 (I32).
 *   CODEBOOK_I8_TILED: CODEBOOK_I8 with a_codes in RTQ_INT8_TILED's layout and w_codes in
 *              RTQ_CODEBOOK_TILED's (each buffer padded to a multiple of 256 rows); same results.
 *   CODEBOOK_TILED is a weight-code layout only: rtq_qgemm returns RTQ_ERR_UNSUPPORTED for it.
 *   The codebook modes give bf16 output (yt == RTQ_F32 returns RTQ_ERR_UNSUPPORTED): their
 *   centroid rounding (fp16 copies, or int8 values) is sized for the bf16 output bound, not for
 *   an fp32 one.
 * T == 0 is a no-op. */
rtq_status rtq_qgemm(const void* a_codes, const float* a_scale, int64_t T, const void* w_codes,
                     const void* w_scale, rtq_dtype w_scale_t, int64_t N, int32_t d, rtq_qmode mode,
                     const rtq_codebook* cb_a, const rtq_codebook* cb_w, void* y, rtq_dtype yt, void* stream);

/* rtq_qgemm with a workspace for the INT8-core modes (RTQ_INT8, RTQ_CODEBOOK_I8 and their tiled
 * forms): a partial last
 * round of 256 x 256 output tiles is shared along d, so no compute unit idles behind it.  After
 * at least one full round, the last full round and the remainder are dealt out as equal runs of
 * K stages that cross tile edges (stream-K); with fewer tiles than compute units, each tile is
 * cut into equal K ranges.  A piece that holds only part of a tile stores an int32 partial tile
 * in the workspace, and the last piece of the tile to finish adds the others (exact int32 sums, so
 * results equal rtq_qgemm's bit for bit).
 *   workspace: device memory of at least rtq_qgemm_workspace() bytes, 16-byte aligned, zero-filled
 *   once before its first use: it ends with one 8-byte arrival counter per shared tile (the last
 *   16 bytes per compute unit), which must start at zero; the block that finishes a shared tile
 *   sets its counter back to zero, so every call that completes leaves the workspace reusable as
 *   is (the partial tiles before the counters may hold anything).  Launches that share a
 *   workspace must not run concurrently.  A smaller or NULL workspace, or the RTQ_CODEBOOK mode,
 *   gives exactly rtq_qgemm. */
rtq_status rtq_qgemm_ws(const void* a_codes, const float* a_scale, int64_t T, const void* w_codes,
                        const void* w_scale, rtq_dtype w_scale_t, int64_t N, int32_t d, rtq_qmode mode,
                        const rtq_codebook* cb_a, const rtq_codebook* cb_w, void* y, rtq_dtype yt,
                        void* workspace, size_t ws_bytes, void* stream);

/* Bytes of workspace rtq_qgemm_ws uses on the current device: two 256 KB int32 partial tiles per
 * compute unit, then two 8-byte counters per compute unit (128 MB on a 256-CU MI355X). */
size_t rtq_qgemm_workspace(void);

/* The online layer: rtq_quantize_rows(x, R, mode, cb_a, eps = 1e-8 (CODEBOOK) ...) into `workspace`
 * followed by rtq_qgemm on the same stream (OrbitQuant article, section 2.2, steps 1-5 and the
 * cancellation).  Weights come from rtq_quantize_rows with the SAME descriptor R (RTQ_INT8_TILED:
 * weight codes written in that mode, and the activation codes go to the workspace tiled too;
 * RTQ_CODEBOOK_I8_TILED: weight codes written in RTQ_CODEBOOK_TILED, activation values tiled).
 *   workspace: device memory of at least rtq_rotated_qlinear_workspace(T, R->d, mode, bits_a) bytes,
 *   16-byte aligned, any contents (the quantiser launch zeroes the product's split counters); on
 *   return it starts with the activation codes and scales.  Calls sharing a workspace must not
 *   overlap.  yt: F32 or BF16 for RTQ_INT8, BF16 for the codebook modes. */
rtq_status rtq_rotated_qlinear(const void* x, rtq_dtype xt, int64_t T, const rtq_rpbh* R, const void* w_codes,
                               const void* w_scale, rtq_dtype w_scale_t, int64_t N, rtq_qmode mode,
                               const rtq_codebook* cb_a, const rtq_codebook* cb_w, void* y, rtq_dtype yt,
                               void* workspace, size_t ws_bytes, void* stream);

/* Bytes of workspace rtq_rotated_qlinear uses: the codes and fp32 scales (each 256-byte aligned;
 * the codes take T*d bytes for RTQ_INT8 and RTQ_CODEBOOK_I8, ceil(T/256)*256*d for RTQ_INT8_TILED
 * and RTQ_CODEBOOK_I8_TILED,
 * T*d*bits_a/8 for RTQ_CODEBOOK), then,
 * for the INT8-core modes, rtq_qgemm_workspace() bytes for the product's K-split.  A workspace
 * that holds only the codes and scales is accepted (the product then runs without the split).
 * bits_a is ignored for RTQ_INT8.  Returns 0 for invalid arguments. */
size_t rtq_rotated_qlinear_workspace(int64_t T, int32_t d, rtq_qmode mode, int32_t bits_a);

/* The online layer with no workspace and no allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * rtq_rotated_qlinear with the activation codes and fp32 token scales held in a static device
 * array of RTQ_NOALLOC_SCRATCH_BYTES bytes inside the library (one per GPU, kept until the
 * process ends) instead of a caller's workspace.  Arguments and results as rtq_rotated_qlinear;
 * the product runs without the K-split of a partial last round (it has no split region).
 * Limit: rtq_rotated_qlinear_workspace's codes and scales, i.e. align256(T*d) + align256(4*T)
 * bytes (T*d*bits_a/8 codes for RTQ_CODEBOOK), at most RTQ_NOALLOC_SCRATCH_BYTES; larger inputs
 * return RTQ_ERR_INVALID_ARG before anything is enqueued.  Calls and graph replays on one GPU
 * share the array: calls that overlap on a GPU (other streams, other threads) race, so order
 * them on one stream.  The first call on a device looks up its copy with hipGetSymbolAddress. */
#define RTQ_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
rtq_status rtq_rotated_qlinear_noalloc(const void* x, rtq_dtype xt, int64_t T, const rtq_rpbh* R,
                                       const void* w_codes, const void* w_scale, rtq_dtype w_scale_t, int64_t N,
                                       rtq_qmode mode, const rtq_codebook* cb_a, const rtq_codebook* cb_w,
                                       void* y, rtq_dtype yt, void* stream);

/* ---- Asymmetric INT8: a scale and a zero point per row (the scale-and-zero-point INT8 the pages
 * name: "INT8旋转量化是什么" section 3 lists per-channel scales and zero points; the int8
 * image-model page computes a scale and a zero-point offset).  With the range widened to contain 0,
 * lo = min(min_j x'_j, 0), hi = max(max_j x'_j, 0): s = fl32(fl32(hi - lo) / 255) (stored as
 * scale_t; the STORED value divides), z = clamp(-128 - rne(fl32(lo / s)), -128, 127),
 * q_j = clamp(rne(fl32(x'_j / s)) + z, -128, 127), so x'_j ~ s (q_j - z); s == 0 gives q = 0, z = 0.
 *   x [rows][d] BF16 (F32 rows are not supported: RTQ_ERR_UNSUPPORTED); R required (the rotation
 *   as in rtq_quantize_rows).  codes int8[rows][d]; scale [rows] of scale_t (F32 or BF16);
 *   zero int32[rows]; code_sum int32[rows] = sum_j q_j (the product's zero-point correction needs
 *   it).  All DEVICE pointers, caller-owned; rows == 0 is a no-op. */
rtq_status rtq_quantize_rows_asym(const void* x, rtq_dtype xt, int64_t rows, int32_t d, const rtq_rpbh* R,
                                  int8_t* codes, void* scale, rtq_dtype scale_t, int32_t* zero, int32_t* code_sum,
                                  void* stream);

/* The product of asymmetric codes: acc[t][n] = sum_j (qa[t][j] - za[t]) (qw[n][j] - zw[n]), exact in
 * int32 (evaluated as acc' - zw sum(qa) - za (sum(qw) - d zw) from the int8 products acc'), then
 * y = acc * a_scale[t] * w_scale[n] in fp32, stored as yt (F32, BF16, or RTQ_I32 for acc itself).
 * a_codes int8[T][d], a_scale fp32[T], a_zero/a_sum int32[T]; w_codes int8[N][d], w_scale [N] of
 * w_scale_t, w_zero/w_sum int32[N]; workspace as for rtq_qgemm_ws (zero-filled once; may be NULL). */
rtq_status rtq_qgemm_asym(const int8_t* a_codes, const float* a_scale, const int32_t* a_zero, const int32_t* a_sum,
                          int64_t T, const int8_t* w_codes, const void* w_scale, rtq_dtype w_scale_t,
                          const int32_t* w_zero, const int32_t* w_sum, int64_t N, int32_t d, void* y, rtq_dtype yt,
                          void* workspace, size_t ws_bytes, void* stream);

/* The online asymmetric layer: rtq_quantize_rows_asym of x (fp32 token scales) into `workspace`, then
 * rtq_qgemm_asym on the same stream.  workspace: at least rtq_rotated_qlinear_asym_workspace(T, R->d)
 * bytes (codes, scales, zero points and code sums, each 256-byte aligned, then the product's
 * K-split region; a workspace without that region is accepted and the product is not split). */
rtq_status rtq_rotated_qlinear_asym(const void* x, rtq_dtype xt, int64_t T, const rtq_rpbh* R, const int8_t* w_codes,
                                    const void* w_scale, rtq_dtype w_scale_t, const int32_t* w_zero,
                                    const int32_t* w_sum, int64_t N, void* y, rtq_dtype yt, void* workspace,
                                    size_t ws_bytes, void* stream);
size_t rtq_rotated_qlinear_asym_workspace(int64_t T, int32_t d);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* rtq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RTQ_H */
