// rtq_internal.h -- launchers shared between the C-ABI layer and the HIP kernels of librtq.
// Not part of the public interface (include/rtq.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rtq {

// What the RPBH row kernel writes for each row.
enum RowOut : int {
    kRowRotF32 = 0,   // rotated row, fp32
    kRowRotBF16 = 1,  // rotated row, bf16 (RNE of the fp32 value)
    kRowInt8 = 2,     // symmetric INT8 codes + per-row scale
    kRowCode4 = 3,    // 4-bit Lloyd-Max codes (packed) + row norm
    kRowCode2 = 4,    // 2-bit Lloyd-Max codes (packed) + row norm
    kRowLut4 = 5,     // 4-bit Lloyd-Max codes written as their int8 codebook values (1 byte each) + norm
    kRowLut2 = 6,     // 2-bit Lloyd-Max codes written as their int8 codebook values + norm
    kRowCode3 = 7,    // 3-bit Lloyd-Max codes (packed bit stream, 8 codes per 3 bytes) + row norm
    kRowLut3 = 8,     // 3-bit codes written as their int8 codebook values + norm
    kRowLut6 = 9,     // 6-bit codes written as their int8 codebook values + norm
    kRowInt8Asym = 10,  // asymmetric INT8 codes + per-row scale, zero point and code sum
};

// The tiled layout of INT8 operands (RTQ_INT8_TILED): rows are grouped in tiles of 256 and the K
// dimension in slices of 64 bytes; block (tile, slice) is 16 KB, contiguous, [256 rows][64 bytes],
// and within a row's 64 bytes the 16-byte chunk c sits at chunk c ^ ((row >> 2) & 3).  This is the
// image of one LDS stage of the INT8 product, so its loads copy whole 1 KB runs.  Rows are padded
// to a multiple of 256 (padding rows are neither written nor used).
constexpr int kTileRows = 256;
constexpr int kTileK = 64;
__host__ __device__ constexpr int64_t tiled_rows(int64_t rows) { return (rows + kTileRows - 1) / kTileRows * kTileRows; }
// Byte offset of the 64-byte slot of row `row`, K slice `blk` (bytes blk*64 .. +64 of the row).
__host__ __device__ inline int64_t tiled_slot_offset(int64_t row, int blk, int d) {
    return ((row / kTileRows) * (d / kTileK) + blk) * (kTileRows * kTileK) + (row % kTileRows) * kTileK;
}
// Position (in 16-byte chunks) of chunk c of a row inside its 64-byte slot.
__host__ __device__ inline int tiled_chunk(int64_t row, int c) { return c ^ static_cast<int>((row >> 2) & 3); }
// The tiled layout of packed codebook codes (RTQ_CODEBOOK_TILED): the same tiles of 256 rows and K
// slices of 64 elements; block (tile, slice) is [256 rows][8 * bits bytes], contiguous, and a row's
// 8 * bits bytes are its packed codes of elements 64 * slice .. +64, as in the row-major bit stream.
// It is the image of one raw code slot of the product.  Byte offset of row `row`, slice `blk`:
__host__ __device__ inline int64_t tiled_code_offset(int64_t row, int blk, int d, int bits) {
    return (((row / kTileRows) * (d / kTileK) + blk) * kTileRows + (row % kTileRows)) * (8 * bits);
}

struct RowArgs {
    const void* x;          // [rows][d] fp32 or bf16
    bool x_bf16;
    int64_t rows;
    int d;
    const int32_t* perm;    // nullptr: rows are already rotated
    const int8_t* signs;
    RowOut out_kind;
    void* out;              // rotated rows or codes
    void* scale;            // [rows] fp32 or bf16 (quantising kinds only)
    bool scale_bf16;
    const float* bounds;    // codebook boundaries (device), 2^bits - 1 entries
    float eps;
    const float* centroids = nullptr;   // codebook centroids (device), 2^bits entries (kRowLut*)
    int32_t* zero = nullptr;            // kRowInt8Asym: per-row zero point
    int32_t* sum = nullptr;             // kRowInt8Asym: per-row sum of the codes
    bool tiled = false;                 // codes in a tiled layout (int8 values: the INT8 one; packed: the code one)
    // words zeroed by the launch (the K-split counters of the product that follows on the stream)
    unsigned long long* clear = nullptr;
    int nclear = 0;
};

hipError_t launch_rpbh_rows(const RowArgs& a, hipStream_t stream);

// Per-device launch facts, queried once per process and device (the queries can synchronise, so
// they must stay off the per-launch path): compute units, and for a kernel with a given dynamic
// LDS size the resident workgroups per CU (after raising its dynamic-LDS limit).
int device_cu_count();
hipError_t kernel_blocks_per_cu(const void* kernel, int threads, size_t lds, int* per_cu);

// The throughput kernel for bf16 rows with the rotation and a quantising output (rpbh_quant.hip).
bool rpbh_quant_bf16_supported(const RowArgs& a);
hipError_t launch_rpbh_quant_bf16(const RowArgs& a, hipStream_t stream);

// x = Pi^T y for each row (rotation inverse), fp32/bf16 in and out.
hipError_t launch_rpbh_inverse(const void* y, bool y_bf16, void* x, bool x_bf16, int64_t rows, int d,
                               const int32_t* perm, const int8_t* signs, hipStream_t stream);

struct GemmI8Args {
    const int8_t* a;        // [T][d] int8 operand (INT8 codes, or int8 codebook values)
    const float* a_scale;   // [T]
    const int8_t* w;        // [N][d] int8 codes (w_bits 8), or [N][d*w_bits/8] packed codebook codes
    const void* w_scale;    // [N] fp32 or bf16
    bool w_scale_bf16;
    int64_t T, N;
    int d;
    void* y;                // [T][N]
    int y_kind;             // 0 fp32, 1 bf16, 2 raw int32
    bool tiled = false;     // both operands tiled: A (int8) in the INT8 layout, W in the INT8 or packed-code one
    // codebook operands on the INT8 matrix cores (w_bits 4 or 2): both codebooks are rounded to
    // int8 as v_k = rint(c_k * S), S = 127 / max_k |c_k|; the product is rescaled by 1/(S_a S_w)
    int w_bits = 8;
    const float* cent_a = nullptr;   // activation codebook centroids (device), 2^a_bits
    int a_bits = 0;
    const float* cent_w = nullptr;   // weight codebook centroids (device), 2^w_bits
    // asymmetric INT8 (int8 weights): zero points and code sums of both operands, all or none
    const int32_t* a_zero = nullptr;
    const int32_t* a_sum = nullptr;
    const int32_t* w_zero = nullptr;
    const int32_t* w_sum = nullptr;
    // optional workspace (gemm_i8_workspace_bytes()): lets a partial last round of tiles be shared
    // along K (stream-K runs, or equal K ranges per tile)
    void* workspace = nullptr;
    size_t ws_bytes = 0;
};

hipError_t launch_gemm_i8(const GemmI8Args& g, hipStream_t stream);
// Workspace bytes for the K-split of launch_gemm_i8 on the current device (two partial int32
// tiles and two counters per CU slot).
size_t gemm_i8_workspace_bytes();
// The split counters inside a workspace of ws_bytes (nullptr and *n = 0 if it has no split region).
unsigned long long* gemm_i8_split_counters(void* workspace, size_t ws_bytes, int* n);
// Zero n counter words on the stream (a fill kernel: safe under graph capture).
hipError_t launch_split_clear(unsigned long long* counters, int n, hipStream_t stream);
// Largest N the INT8-core product takes for an output kind (0 fp32, 1 bf16, 2 int32).
int64_t gemm_i8_max_n(int y_kind);

struct GemmLutArgs {
    const uint8_t* a;         // [T][d*bits_a/8] packed codes
    const float* a_scale;     // [T] token norms
    const uint8_t* w;         // [N][d*bits_w/8] packed codes
    const void* w_scale;      // [N] fp32 or bf16 row norms
    bool w_scale_bf16;
    const float* ca;          // activation centroids (device), 2^bits_a
    const float* cw;          // weight centroids (device), 2^bits_w
    int bits_a, bits_w;
    int64_t T, N;
    int d;
    void* y;                  // [T][N]
    int y_kind;               // 0 fp32, 1 bf16
};

hipError_t launch_gemm_lut(const GemmLutArgs& g, hipStream_t stream);

}  // namespace rtq
