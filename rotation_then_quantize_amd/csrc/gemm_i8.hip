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
// Tiling.  A workgroup owns a 256 x 256 output tile, split over 2 x kWavesN waves; each wave
// computes a 128 x (256 / kWavesN) block as 32 x 32 MFMA tiles.  kWavesN = 2: four waves (one per
// SIMD), 128 x 128 per wave, 8 KB of LDS fragment reads per 16 MFMAs.  kWavesN = 4: eight waves
// (two per SIMD), 128 x 64 per wave, 6 KB per 8 MFMAs.
//
// Pipeline.  K advances in stages of 64 bytes through a ring of 4 LDS stages (32 KB each: the A
// and W tile rows for that K range).  Stages are filled by buffer loads that write LDS directly
// (no staging registers), two stages ahead of the one being multiplied.  Inside a stage, the
// fragments of the next K step are read while the MFMAs of the current one run (two fragment
// register sets, reads interleaved one per MFMA).  The waits on the LDS-writing loads are explicit
// (the compiler does not track them).
//
// LDS layout.  A stage block holds 256 rows x 64 bytes per operand; 16-byte chunk c of row r sits
// at slot c ^ ((r >> 2) & 3).  A fragment read (16 lanes = 16 consecutive rows, one chunk, per LDS
// cycle) then touches 16 distinct 16-byte bank groups, and every load instruction writes a
// contiguous 1 KB (16 rows), with the permutation applied to which global chunk each lane fetches.
// Operands in the tiled layouts are stored as these stage blocks (int8 operands) or as the raw code
// slots below (packed weight codes), so each load instruction also reads contiguous bytes.
//
// Schedule.  One workgroup per CU runs persistently over tiles.  The tiles are split into 8
// contiguous ranges, one per XCD (block b runs on XCD b % 8, and each XCD has its own L2); the
// blocks of an XCD walk their range in bands of 8 N-tiles so concurrently running blocks share
// A and W rows in that L2.  The next tile's first two stages are fetched while the current
// tile's epilogue runs.  Y is written with streaming stores of whole cache lines: it is written
// once, and letting it allocate in the caches evicts the operand rows that later tiles re-read.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "codebook_int8.h"
#include "rtq_internal.h"

// The LDS-writing loads set M0 in inline assembly; M0 is otherwise unused by this kernel.
#pragma clang diagnostic ignored "-Winline-asm"

namespace rtq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;                          // K bytes per LDS stage (two MFMA K steps)
constexpr int kStages = 4;                      // LDS ring depth
constexpr int kOpBytes = BM * BK;               // 16 KB: one operand's rows for one stage
constexpr int kStageBytes = 2 * kOpBytes;       // A then W
constexpr int kRingBytes = kStages * kStageBytes;
constexpr int kLds = kRingBytes + (BM + BN) * static_cast<int>(sizeof(float)) + 16;   // ring + scales + flag
constexpr int kWavesM = 2;
constexpr int WM = BM / kWavesM;                // 128 rows per wave
constexpr int kXcds = 8;
constexpr int kBufferWord3 = 0x00020000;        // gfx9 buffer descriptor word 3 (raw, 32-bit dwords)
constexpr int kStoreNT = 2;                     // buffer store cache policy: nontemporal (streaming)
constexpr int kLoadL2 = 1;                      // buffer load cache policy: sc0, served from the L2 (not L1)
constexpr int kDefaultWavesN = 4;               // the configuration the launcher uses

// Two fp32 values -> a bf16 pair (the first in the low half), rounded to nearest even by the
// gfx950 packed conversion instruction: one VALU operation per pair.  It was checked bit-exact
// against the integer form of that rounding on 2^26 inputs (every bf16 upper half with tie,
// near-tie and hashed lower halves, subnormals and infinities included); a NaN stays a NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Raw buffer descriptor over [base, base + bytes): loads at offsets >= bytes return zero.
__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    v4i r;
    r.x = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b)));
    r.y = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b >> 32) & 0xffffu));
    r.z = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
    r.w = kBufferWord3;
    return r;
}

// 16 bytes per lane from buffer offset voff to LDS address lds_addr + 16 * lane.
__device__ __forceinline__ void load_to_lds(v4i rsrc, uint32_t voff, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(static_cast<int>(lds_addr))), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

#define RTQ_BARRIER() asm volatile("s_barrier" ::: "memory")
// every vector memory access of this wave has completed (stores acknowledged by the L2)
#define RTQ_WAIT_ALL_VMEM() asm volatile("s_waitcnt vmcnt(0)" ::: "memory")
// orders a wave's own LDS accesses (executed in order per wave) against compiler reordering
#define RTQ_LDS_FENCE() asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory")

// Wait until at most n vector-memory operations of this wave are outstanding.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n == 0 || n == 2 || n == 3 || n == 4 || n == 5 || n == 8, "add the immediate");
    if constexpr (n == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if constexpr (n == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    if constexpr (n == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    if constexpr (n == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    if constexpr (n == 5) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    if constexpr (n == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
}

// 4 bytes per lane from buffer offset voff to LDS address lds_addr + 4 * lane.
__device__ __forceinline__ void load_to_lds4(v4i rsrc, uint32_t voff, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(static_cast<int>(lds_addr))), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

// 32 packed 4-bit codes (LSB first) -> 32 int8 values in order (8 words)
__device__ __forceinline__ void decode4(const uint32_t (&lut)[4], const uint32_t (&in)[4], uint32_t (&out)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t ev = lut16_x4(lut, in[i] & 0x0F0F0F0Fu);           // codes 0, 2, 4, 6 of the word
        const uint32_t od = lut16_x4(lut, (in[i] >> 4) & 0x0F0F0F0Fu);    // codes 1, 3, 5, 7
        out[2 * i] = __builtin_amdgcn_perm(od, ev, 0x05010400u);
        out[2 * i + 1] = __builtin_amdgcn_perm(od, ev, 0x07030602u);
    }
}

// 32 packed 2-bit codes (LSB first) -> 32 int8 values in order (8 words); lut[0] holds the 4 values
__device__ __forceinline__ void decode2(const uint32_t (&lut)[4], const uint32_t (&in)[2], uint32_t (&out)[8]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        // vj = values of codes j, 4+j, 8+j, 12+j of the word
        const uint32_t v0 = __builtin_amdgcn_perm(lut[0], lut[0], in[i] & 0x03030303u);
        const uint32_t v1 = __builtin_amdgcn_perm(lut[0], lut[0], (in[i] >> 2) & 0x03030303u);
        const uint32_t v2 = __builtin_amdgcn_perm(lut[0], lut[0], (in[i] >> 4) & 0x03030303u);
        const uint32_t v3 = __builtin_amdgcn_perm(lut[0], lut[0], (in[i] >> 6) & 0x03030303u);
        const uint32_t t01l = __builtin_amdgcn_perm(v1, v0, 0x05010400u);
        const uint32_t t01h = __builtin_amdgcn_perm(v1, v0, 0x07030602u);
        const uint32_t t23l = __builtin_amdgcn_perm(v3, v2, 0x05010400u);
        const uint32_t t23h = __builtin_amdgcn_perm(v3, v2, 0x07030602u);
        out[4 * i] = __builtin_amdgcn_perm(t23l, t01l, 0x05040100u);
        out[4 * i + 1] = __builtin_amdgcn_perm(t23l, t01l, 0x07060302u);
        out[4 * i + 2] = __builtin_amdgcn_perm(t23h, t01h, 0x05040100u);
        out[4 * i + 3] = __builtin_amdgcn_perm(t23h, t01h, 0x07060302u);
    }
}

// 32 packed 3-bit codes (one LSB-first bit stream over 3 words) -> 32 int8 values in order (8
// words); lut[0..1] hold the 8 values.  Group g of 4 codes is the 12 bits at 12g: its codes are
// spread into the 4 selector bytes of one v_perm_b32.
__device__ __forceinline__ void decode3(const uint32_t (&lut)[4], const uint32_t (&in)[3], uint32_t (&out)[8]) {
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        const int bit = 12 * g, w = bit >> 5, sh = bit & 31;
        const uint32_t v = sh + 12 <= 32 ? in[w] >> sh : __builtin_amdgcn_alignbit(in[w + 1], in[w], sh);
        const uint32_t sel = (v & 7u) | ((v << 5) & 0x700u) | ((v << 10) & 0x70000u) | ((v << 15) & 0x7000000u);
        out[g] = __builtin_amdgcn_perm(lut[1], lut[0], sel);
    }
}

// Tiles shared along K.  Tiles [0, dp_tiles) run whole, data-parallel; the remaining (shared)
// tiles are cut along K into runs of blocks: either `split` equal K ranges per tile (a last round
// that would leave most blocks idle), or stream-K (split 0: a last full round plus a small
// remainder spread evenly over every block, each run at least one tile long).  Every block whose
// run meets a tile only in part stores its int32 partial tile and arrives on the tile's counter;
// the last to arrive adds the others' partials and runs the epilogue (no block ever waits for
// another; a stream-K tile's second piece to finish skips its own store, see the epilogue).
// The counters are zero when the launch starts (the quantiser launch that precedes the product in
// the layer clears them; a standalone product's workspace is zero-filled once by its owner), and
// the block that finishes a shared tile sets its counter back to zero, so every complete launch
// leaves them zero for the next.
constexpr int kMaxSplit = 8;

struct SplitArgs {
    int dp_tiles;
    int split;                      // 1: no shared tiles; >= 2: equal K ranges per tile; 0: stream-K
    v4i* partials;                  // [block][2][BM * BN / 4] int32 quads (below)
    unsigned long long* counters;   // [shared tile], zero at launch
};

// Workspace per block slot (one block per compute unit): two partial tiles, since a run meets at
// most two tiles in part (its first piece and its last), and two counters, since a stream-K launch
// shares less than two rounds of tiles.
constexpr int64_t partial_slots_cap(int64_t slots) { return 2 * slots; }
constexpr int64_t shared_tiles_cap(int64_t slots) { return 2 * slots; }

// Add `add` to a shared tile's counter (an atomic at the L2 of the XCD that runs every piece of
// the tile); returns the arrivals before this one.
__device__ __forceinline__ unsigned int split_arrive(unsigned long long* c, unsigned int add) {
    return static_cast<unsigned int>(
        __hip_atomic_fetch_add(c, static_cast<unsigned long long>(add), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// The block that finishes a shared tile leaves its counter at zero again, so a launch that completes
// leaves every counter as it found it.
__device__ __forceinline__ void split_reset(unsigned long long* c) {
    __hip_atomic_store(c, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void __launch_bounds__(256) split_clear_kernel(unsigned long long* __restrict__ c, int n) {
    for (int i = static_cast<int>(threadIdx.x); i < n; i += 256) c[i] = 0ull;
}

// Tile index within the XCD-ordered sequence -> (tile_m, tile_n), in bands of 8 N-tiles.
__device__ __forceinline__ void tile_of(int lin, int tiles_m, int tiles_n, int* tm, int* tn) {
    constexpr int kBand = 8;
    const int band = lin / (kBand * tiles_m);
    const int in_band = lin % (kBand * tiles_m);
    const int band_w = min(kBand, tiles_n - band * kBand);
    *tm = in_band / band_w;
    *tn = band * kBand + in_band % band_w;
}

// LDS bytes of one stage of packed weight codes, and the ring of kRawSlots of them behind the
// scales (codebook weights only).
constexpr int raw_stage_bytes(int w_bits) { return w_bits < 8 ? BN * BK * w_bits / 8 : 0; }
constexpr int kRawSlots = 3;
constexpr int lds_bytes(int w_bits) { return kLds + kRawSlots * raw_stage_bytes(w_bits); }
// Asymmetric INT8 (int8 weights only): zero points and code sums of the tile's rows and columns,
// two int32 arrays of BM + BN behind the scales (where coded weights keep their raw slots).
constexpr int kAsymBytes = 2 * (BM + BN) * static_cast<int>(sizeof(int32_t));

// Zero points and code sums of asymmetric INT8 operands (all null: symmetric codes).
struct AsymArgs {
    const int32_t* a_zero;   // [T]
    const int32_t* a_sum;    // [T]  sum_j qa[t][j]
    const int32_t* w_zero;   // [N]
    const int32_t* w_sum;    // [N]  sum_j qw[n][j]
};

template <int kWavesN, int kYKind, bool kWScaleBF16, bool kVec, int kWBits, bool kAsym, bool kTiled>
__global__ void __launch_bounds__(64 * kWavesM * kWavesN, 1)
gemm_i8_kernel(const int8_t* __restrict__ A, const float* __restrict__ a_scale, const int8_t* __restrict__ W,
               const void* __restrict__ w_scale, int64_t T, int64_t N, int d, void* __restrict__ Y,
               int tiles_m, int tiles_n, const float* __restrict__ cent_a, int a_bits,
               const float* __restrict__ cent_w, SplitArgs sp, AsymArgs za) {
    constexpr int kWaves = kWavesM * kWavesN;
    // kWBits < 8: W holds packed codebook codes; they are loaded into a ring of raw LDS slots two
    // stages ahead and decoded to int8 codebook values into the stage ring one stage ahead.
    constexpr bool kCoded = kWBits < 8;
    constexpr int kRawStage = raw_stage_bytes(kWBits);
    constexpr int kCodeLoads = kWBits == 4 ? 1 : (kWBits == 3 ? 3 : 2);   // LDS-writing loads per thread per code stage
    constexpr int kThreads = 64 * kWaves;
    constexpr int WN = BN / kWavesN;                           // columns per wave
    constexpr int TM = WM / 32, TN = WN / 32;                  // MFMA tiles per wave
    constexpr int kLoadsPerOp = BM * BK / (kThreads * 16);     // 16-byte loads per thread per operand
    constexpr int kLoadsPerStage = (kCoded ? 1 : 2) * kLoadsPerOp;   // A (and W when int8)
    constexpr int kScalesPerThread = (BM + BN) / kThreads;

    extern __shared__ __attribute__((aligned(16))) int8_t lds[];   // ring of stages, then scales

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / kWavesN, wn = wave % kWavesN;

    // Whole tiles [0, dp): split into 8 contiguous ranges, one per XCD (block b runs on XCD b % 8),
    // taken round-robin by that XCD's blocks.
    const int total = tiles_m * tiles_n;
    const int xcd = blockIdx.x % kXcds;
    const int stride = gridDim.x / kXcds;
    const int local = static_cast<int>(blockIdx.x / kXcds);
    const int dp = sp.dp_tiles;
    const int per = (dp + kXcds - 1) / kXcds;
    const int lin_end = min((xcd + 1) * per, dp);
    const int nk_all = d / BK;
    // Shared tiles [dp, total): shared tile st is tile dp + st and runs on XCD st % 8, so all its K
    // ranges meet in one L2 (and the shared tiles' partial traffic spreads over every XCD).  The
    // XCD's tiles_x shared tiles form one tile-major sequence of tiles_x * nk_all K stages, cut into
    // equal runs [g_run, g_end), one per block: blocks_x = tiles_x * split runs (split equal K ranges
    // per tile), or, with split 0 (stream-K), a run for each of the XCD's blocks; those runs are at
    // least one tile long, so a tile meets at most two of them.
    const int shared = total - dp;
    const int tiles_x = shared > xcd ? (shared - xcd + kXcds - 1) / kXcds : 0;
    const int blocks_x = sp.split == 0 ? stride : min(stride, tiles_x * sp.split);
    const int64_t w_x = static_cast<int64_t>(tiles_x) * nk_all;
    int64_t g_run = 0, g_end = 0;
    if (sp.split != 1 && local < blocks_x) {
        g_run = local * w_x / blocks_x;
        g_end = (local + 1) * w_x / blocks_x;
    }
    int lin = xcd * per + local;
    bool in_tail = lin >= lin_end;
    if (in_tail && g_run >= g_end) return;   // no work for this block: before any barrier

    const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
    float* s_as = reinterpret_cast<float*>(lds + kRingBytes);
    float* s_ws = s_as + BM;
    int* s_flag = reinterpret_cast<int*>(s_ws + BN);
    static_assert(!kAsym || !kCoded, "zero points with int8 weights only");
    int* s_z = reinterpret_cast<int*>(lds + kLds);   // kAsym: zero points, rows then columns
    int* s_e = s_z + BM + BN;                        // kAsym: sum_j qa (rows), sum_j qw - d zw (columns)
    int kbeg = 0, nk = nk_all;   // the current work item's K stages
    // The current shared piece: its tile's counter (shared tile index), the first run (XCD-local
    // block) that meets the tile, the number of runs that do (1: no partials) and this block's
    // place among them.
    int ptile = 0, pfirst = 0, pcount = 1, pord = 0;
    // Partial slot of the o-th run meeting a tile whose first run is `first`: slot [1] of block
    // `first` (a stream-K tile's head, the last piece of that run), else slot [0] of block
    // first + o (the first piece of its run; with equal K ranges, a run's only piece).
    auto piece_slot = [&](int first, int o) {
        return 2 * ((first + o) * kXcds + xcd) + ((sp.split == 0 && o == 0) ? 1 : 0);
    };

    // Load geometry: instruction q of wave w fills rows 16 * (q * kWaves + w) .. +16 of an operand
    // block, 1 KB of LDS; lane L writes its 16 bytes at LDS offset 16 L of that KB, which holds row
    // 16 * (q * kWaves + w) + L / 4, chunk (L % 4) ^ ((row >> 2) & 3) = (L % 4) ^ ((L >> 4) & 3).
    // Row-major operands: each lane fetches that chunk of that row (16 rows x 64 bytes per
    // instruction).  kTiled: the operands are stored as the stage blocks themselves (the tiled
    // layout), so a lane fetches bytes 16 L of the KB and each instruction reads 1 KB contiguous.
    uint32_t load_off[kLoadsPerOp];
#pragma unroll
    for (int q = 0; q < kLoadsPerOp; ++q) {
        const int row = 16 * (q * kWaves + wave) + (lane >> 2);
        const int chunk = (lane & 3) ^ ((lane >> 4) & 3);
        load_off[q] = kTiled ? static_cast<uint32_t>((q * kWaves + wave) * 1024 + 16 * lane)
                             : static_cast<uint32_t>(row * d + chunk * 16);
    }
    const uint32_t wave_lds = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(wave * 1024));

    // Fragment geometry: lane reads row (lane % 32) of a 32-row block, chunk 2 * ks + lane / 32.
    const int fr = lane & 31, fh = lane >> 5;
    const int fsw = (fr >> 2) & 3;
    const uint32_t frag_off0 = static_cast<uint32_t>(fr * BK + (((0 + fh) ^ fsw) << 4));
    const uint32_t frag_off1 = static_cast<uint32_t>(fr * BK + (((2 + fh) ^ fsw) << 4));

    int64_t m0 = 0, n0 = 0;
    v4i rsa, rsw;
    auto set_item = [&](bool tail, int l) {
        int tile = l;
        kbeg = 0;
        nk = nk_all;
        if (tail) {   // the next piece of this block's run: up to the end of the run or of the tile
            const int i = static_cast<int>(g_run / nk_all);
            const int64_t t0 = static_cast<int64_t>(i) * nk_all;
            const int64_t t1 = min<int64_t>(g_end, t0 + nk_all);
            kbeg = static_cast<int>(g_run - t0);
            nk = static_cast<int>(t1 - g_run);
            // the run holding stage q is run (blocks_x (q + 1) - 1) / w_x
            const int first = static_cast<int>((blocks_x * (t0 + 1) - 1) / w_x);
            const int last = static_cast<int>((blocks_x * (t0 + nk_all) - 1) / w_x);
            ptile = xcd + kXcds * i;
            pcount = last - first + 1;
            pfirst = first;
            pord = local - first;
            tile = dp + ptile;
            g_run = t1;
        }
        int tm, tn;
        tile_of(tile, tiles_m, tiles_n, &tm, &tn);
        m0 = static_cast<int64_t>(tm) * BM;
        n0 = static_cast<int64_t>(tn) * BN;
        const int rows_a = static_cast<int>(min<int64_t>(BM, T - m0));
        const int rows_w = static_cast<int>(min<int64_t>(BN, N - n0));
        // (tiled operands: the tile's whole panel, padding rows included, is in the buffer)
        rsa = make_rsrc(A + m0 * d, static_cast<uint32_t>((kTiled ? BM : rows_a) * d));
        const int wrow = d * kWBits / 8;                      // bytes per weight row
        rsw = make_rsrc(W + n0 * wrow, static_cast<uint32_t>((kTiled ? BN : rows_w) * wrow));
    };
    auto issue_stage = [&](int st) {
        const uint32_t sb = lds_base + static_cast<uint32_t>((st & (kStages - 1)) * kStageBytes) + wave_lds;
        const uint32_t k0 = static_cast<uint32_t>((kbeg + st) * (kTiled ? BM * BK : BK));   // BM == BN
#pragma unroll
        for (int q = 0; q < kLoadsPerOp; ++q) {
            load_to_lds(rsa, load_off[q] + k0, sb + q * kWaves * 1024);
            if (!kCoded) load_to_lds(rsw, load_off[q] + k0, sb + kOpBytes + q * kWaves * 1024);
        }
    };
    // Packed weight codes of stage st -> raw slot st % kRawSlots, laid out [row][BK * bits / 8].
    // 4-bit: one 16-byte load per thread (thread t: row t / 2, half t % 2 of the row's 32 bytes);
    // 2-bit: two 4-byte loads per thread (load q, thread t: bytes q * 2048 + 4t of the slot);
    // 3-bit: three such loads (rows of 24 bytes).  kTiled: the codes are stored as these slots (the
    // tiled code layout), so every load instruction reads one contiguous run (1 KB, or 256 bytes).
    const uint32_t raw_base = lds_base + static_cast<uint32_t>(kLds);
    auto issue_codes = [&](int st) {
        const uint32_t slot = raw_base + static_cast<uint32_t>((st % kRawSlots) * kRawStage);
        const int wrow = d * kWBits / 8;
        if constexpr (kWBits == 4) {
            const uint32_t off = kTiled ? static_cast<uint32_t>((kbeg + st) * (BN * 32) + 16 * tid)
                                        : static_cast<uint32_t>((tid >> 1) * wrow + (kbeg + st) * 32 + (tid & 1) * 16);
            load_to_lds(rsw, off, slot + wave_lds);
        } else if constexpr (kWBits == 2) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int b = q * 2048 + 4 * tid;                 // byte within the slot
                const uint32_t off = kTiled ? static_cast<uint32_t>((kbeg + st) * (BN * 16) + b)
                                            : static_cast<uint32_t>((b >> 4) * wrow + (kbeg + st) * 16 + (b & 15));
                load_to_lds4(rsw, off, slot + q * 2048 + static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(wave * 256)));
            }
        } else if constexpr (kWBits == 3) {
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                const int b = q * 2048 + 4 * tid;                 // byte within the slot
                const int row = b / 24;
                const uint32_t off = kTiled ? static_cast<uint32_t>((kbeg + st) * (BN * 24) + b)
                                            : static_cast<uint32_t>(row * wrow + (kbeg + st) * 24 + (b - 24 * row));
                load_to_lds4(rsw, off, slot + q * 2048 + static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(wave * 256)));
            }
        }
    };
    // Raw slot of stage st -> int8 values in the W half of stage st's ring slot.  Thread t decodes
    // row t / 2, K bytes 32 * (t % 2) .. +32 (two 16-byte chunks of the swizzled row).  In the main
    // loop the raw codes are read right after the barrier and decoded behind the first K step's
    // MFMAs, so the read's latency is covered (measured 2-3% faster than decoding at the barrier).
    uint32_t lut[4] = {0u, 0u, 0u, 0u};
    struct RawCodes { uint32_t w[4]; };
    auto read_raw = [&](int st) -> RawCodes {
        const int8_t* raw = lds + kLds + (st % kRawSlots) * kRawStage;
        RawCodes r{{0u, 0u, 0u, 0u}};
        if constexpr (kWBits == 4) {
            const v4i x = *reinterpret_cast<const v4i*>(raw + 16 * tid);
            r.w[0] = static_cast<uint32_t>(x.x); r.w[1] = static_cast<uint32_t>(x.y);
            r.w[2] = static_cast<uint32_t>(x.z); r.w[3] = static_cast<uint32_t>(x.w);
        } else if constexpr (kWBits == 2) {
            const uint2 x = *reinterpret_cast<const uint2*>(raw + 8 * tid);
            r.w[0] = x.x; r.w[1] = x.y;
        } else if constexpr (kWBits == 3) {
            const uint32_t* xr = reinterpret_cast<const uint32_t*>(raw + 12 * tid);
            r.w[0] = xr[0]; r.w[1] = xr[1]; r.w[2] = xr[2];
        }
        return r;
    };
    auto decode_write = [&](int st, const RawCodes& r) {
        uint32_t v[8];
        if constexpr (kWBits == 4) {
            const uint32_t in[4] = {r.w[0], r.w[1], r.w[2], r.w[3]};
            decode4(lut, in, v);
        } else if constexpr (kWBits == 2) {
            const uint32_t in[2] = {r.w[0], r.w[1]};
            decode2(lut, in, v);
        } else if constexpr (kWBits == 3) {
            const uint32_t in[3] = {r.w[0], r.w[1], r.w[2]};
            decode3(lut, in, v);
        }
        const int row = tid >> 1, c0 = 2 * (tid & 1), sw = (row >> 2) & 3;
        int8_t* wb = lds + (st & (kStages - 1)) * kStageBytes + kOpBytes + row * BK;
        *reinterpret_cast<v4i*>(wb + (((c0) ^ sw) << 4)) =
            v4i{static_cast<int>(v[0]), static_cast<int>(v[1]), static_cast<int>(v[2]), static_cast<int>(v[3])};
        *reinterpret_cast<v4i*>(wb + (((c0 + 1) ^ sw) << 4)) =
            v4i{static_cast<int>(v[4]), static_cast<int>(v[5]), static_cast<int>(v[6]), static_cast<int>(v[7])};
    };
    auto decode_stage = [&](int st) { decode_write(st, read_raw(st)); };
    // The tile's token scales (entries 0..255) and output-row scales (256..511), one or two per
    // thread, staged in LDS behind the ring for the epilogue.
    float sc[kScalesPerThread];
    int zr[kScalesPerThread], er[kScalesPerThread];
    float alpha = 1.0f;   // codebook operands: 1 / (S_a S_w), folded into the token scales
    auto load_scales = [&]() {
        if constexpr (kAsym) {
#pragma unroll
            for (int r = 0; r < kScalesPerThread; ++r) {
                const int k = tid + r * kThreads;
                zr[r] = 0;
                er[r] = 0;
                if (k < BM) {
                    if (m0 + k < T) {
                        zr[r] = za.a_zero[m0 + k];
                        er[r] = za.a_sum[m0 + k];
                    }
                } else if (n0 + (k - BM) < N) {
                    const int64_t n = n0 + (k - BM);
                    zr[r] = za.w_zero[n];
                    er[r] = za.w_sum[n] - d * zr[r];
                }
            }
        }
        if (kYKind == 2) return;
#pragma unroll
        for (int r = 0; r < kScalesPerThread; ++r) {
            const int k = tid + r * kThreads;
            sc[r] = 0.0f;
            if (k < BM) {
                if (m0 + k < T) sc[r] = kCoded ? a_scale[m0 + k] * alpha : a_scale[m0 + k];
            } else if (n0 + (k - BM) < N) {
                const int64_t n = n0 + (k - BM);
                if (kWScaleBF16)
                    sc[r] = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(w_scale)[n]) << 16);
                else
                    sc[r] = static_cast<const float*>(w_scale)[n];
            }
        }
    };

    v4i fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    auto read_frags = [&](v4i* fa, v4i* fb, int st, uint32_t foff) {
        const int8_t* la = lds + (st & (kStages - 1)) * kStageBytes + foff;
        const int8_t* lb = la + kOpBytes;
        // in the order the MFMAs below first use them: W0, A0, W1, A1, ...
#pragma unroll
        for (int k = 0; k < (TM > TN ? TM : TN); ++k) {
            if (k < TN) fb[k] = *reinterpret_cast<const v4i*>(lb + (wn * WN + k * 32) * BK);
            if (k < TM) fa[k] = *reinterpret_cast<const v4i*>(la + (wm * WM + k * 32) * BK);
        }
    };
    v16i acc[TM][TN];
    auto mfmas = [&](const v4i* fa, const v4i* fb) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[j], fa[i], acc[i][j], 0, 0, 0);
    };

    if constexpr (kCoded) {
        const float sw = codebook_int8_scale(cent_w, 1 << kWBits);
        codebook_int8_table(cent_w, 1 << kWBits, sw, lut);
        alpha = 1.0f / (codebook_int8_scale(cent_a, 1 << a_bits) * sw);
    }

    // Stages 0 and 1 of a tile (and weight codes 0..2) are fetched before the previous tile's
    // epilogue (which stages its output through ring slots 2 and 3), stage 2 after it.  The waits
    // count loads by iteration: in the loop, iteration s issues codes s + 4 and stage s + 3.
    auto prefetch_early = [&]() {
        issue_stage(0);
        if (kCoded) {
            issue_codes(0);
            if (nk > 1) issue_codes(1);
        }
        if (nk > 1) issue_stage(1);
        if (kCoded && nk > 2) issue_codes(2);
    };
    // Partial tiles of split tiles are kept in the accumulators' own register layout, so a partial
    // moves between registers and memory with no staging, each instruction covering a contiguous
    // 1 KB: quad g (int32 elements 4g .. 4g + 3) of lane L's MFMA block (i, j) in wave w sits at
    // byte ((((w * TM + i) * TN + j) * 4 + g) * 64 + L) * 16 of its 256 KB slot (the wave-uniform
    // part of the offset goes in the instructions' scalar offset).
    const int part_lane = 16 * lane;
    const int part_wave = __builtin_amdgcn_readfirstlane(wave * TM * TN * 4 * 1024);
    auto part_soff = [&](int i, int j, int g) { return part_wave + ((i * TN + j) * 4 + g) * 1024; };
    auto part_rsrc = [&](int slot) {
        return __builtin_amdgcn_make_buffer_rsrc(sp.partials + static_cast<size_t>(slot) * (BM * BN / 4), (short)0,
                                                 BM * BN * 4, kBufferWord3);
    };

    set_item(in_tail, lin);
    prefetch_early();
    load_scales();

    for (;;) {
        if (nk > 2) issue_stage(2);
        if (kYKind != 2) {
#pragma unroll
            for (int r = 0; r < kScalesPerThread; ++r) s_as[tid + r * kThreads] = sc[r];   // s_ws follows s_as
        }
        if constexpr (kAsym) {
#pragma unroll
            for (int r = 0; r < kScalesPerThread; ++r) {
                s_z[tid + r * kThreads] = zr[r];
                s_e[tid + r * kThreads] = er[r];
            }
        }
        // stages 0 and 1 (and codes 0..2) have landed, with everything issued before them
        // (e.g. the previous tile's stores); only stage 2 may be in flight
        if (nk > 2)
            wait_vmcnt<kLoadsPerStage>();
        else
            wait_vmcnt<0>();
        if constexpr (kCoded) {
            RTQ_BARRIER();   // every wave's code loads have landed (2-bit rows are loaded by other waves)
            decode_stage(0);
            if (nk > 1) decode_stage(1);
        }
        RTQ_BARRIER();   // ... in every wave; the scales and decoded stages are visible
        if (kCoded && nk > 3) issue_codes(3);   // raw slot 0: decoded above, in every wave

#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = v16i{};
        read_frags(fa0, fb0, 0, frag_off0);

        // One K stage.  kSteady (s + 4 < nk): every load and decode below is issued, so the stage is
        // one basic block and the compiler can place the decode's VALU work among the MFMAs (with
        // the checks, each conditional load or decode was a block of its own between two MFMA
        // groups); the last four stages take the checked form.
        auto kstep = [&](int s, auto steady_tag) {
            constexpr bool kSteady = decltype(steady_tag)::value;
            // stage s + 1 (and codes s + 2) must have landed; what iteration s - 1 issued (stage
            // s + 2, codes s + 3) may still be in flight
            if constexpr (kCoded) {
                if (kSteady || s + 3 < nk)
                    wait_vmcnt<kLoadsPerStage + kCodeLoads>();
                else if (s + 2 < nk)
                    wait_vmcnt<kLoadsPerStage>();
                else
                    wait_vmcnt<0>();
            } else {
                if (kSteady || s + 2 < nk)
                    wait_vmcnt<kLoadsPerStage>();
                else
                    wait_vmcnt<0>();
            }
            RTQ_BARRIER();   // every wave's part of stage s + 1 is in LDS; stage s - 1 is consumed
            RawCodes rc{{0u, 0u, 0u, 0u}};
            if (kCoded) {
                if (kSteady || s + 4 < nk) issue_codes(s + 4);   // raw slot of codes s + 1, decoded last iteration
                if (kSteady || s + 2 < nk) rc = read_raw(s + 2);
            }
            read_frags(fa1, fb1, s, frag_off1);
            mfmas(fa0, fb0);
            if (kCoded && (kSteady || s + 2 < nk)) decode_write(s + 2, rc);   // visible after the next barrier
            // stage s + 3 into stage s - 1's slot, issued behind the first K step's MFMAs (measured
            // 2% faster than right after the barrier)
            if (kSteady || s + 3 < nk) issue_stage(s + 3);
            // (on the last stage this reads an unused slot: unconditional, so the compiler's LDS wait
            // before the next MFMAs does not also cover these reads)
            read_frags(fa0, fb0, s + 1, frag_off0);
            mfmas(fa1, fb1);
            // Issue order: each fragment read sits between two MFMAs of the other register set, so
            // the reads of one K step are in flight while the previous step's MFMAs run.
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int k = 0; k < TM + TN; ++k) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
                }
                __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - (TM + TN), 0);
            }
        };
        int s = 0;
        for (; s + 4 < nk; ++s) kstep(s, std::true_type{});
        for (; s < nk; ++s) kstep(s, std::false_type{});
        RTQ_BARRIER();   // every wave is done reading the ring

        const int64_t cm0 = m0, cn0 = n0;
        const bool ctail = in_tail && pcount > 1;   // a piece of a tile shared with another run
        const int ctile = ptile, cfirst = pfirst, ccount = pcount, cord = pord;
        bool more = false;
        if (!in_tail) {
            if (lin + stride < lin_end) {
                lin += stride;
                more = true;
            } else if (g_run < g_end) {
                in_tail = true;
                more = true;
            }
        } else {
            more = g_run < g_end;
        }
        if (more) {
            set_item(in_tail, lin);
            prefetch_early();
            load_scales();
        }

        // ---- staging: the MFMA computed the transposed tile (W fragment first), so a lane holds
        // D[n][t] at n = 8*(r/4) + 4*(lane/32) + r%4, t = lane % 32: four consecutive output columns
        // of one token row per group r/4.  stage_block(i) copies a wave's raw int32 rows of MFMA
        // block i (32 token rows) into its private LDS region (ring slots 2 and 3; 16-byte chunk c of
        // row r at chunk c ^ (r % 16), against bank conflicts), to be read back row-contiguously.
        constexpr int kPassRows = 32;
        constexpr int kPitch = WN * 4;                             // raw int32 row
        static_assert(kWaves * kPassRows * kPitch <= 2 * kStageBytes, "staging must fit ring slots 2-3");
        int8_t* stg = lds + 2 * kStageBytes + wave * (kPassRows * kPitch);
        auto swz = [](int row, int chunk) { return (chunk ^ (row & 15)) << 4; };   // byte offset in the row
        auto stage_block = [&](int i) {
            int8_t* wrow = stg + fr * kPitch;
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<v4i*>(wrow + swz(fr, 8 * j + 2 * g + fh)) =
                        v4i{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
            RTQ_LDS_FENCE();   // the wave's rows are in LDS before they are read back
        };

        // ---- split tile: publish this K range's partial; the last block of the tile to arrive adds
        // the other partials into its accumulators and runs the epilogue.
        bool epilogue = true;
        // Partial layout: the accumulators' own register layout, so a partial moves between
        // registers and memory with no staging, each instruction covering a contiguous 1 KB: quad
        // g (int32 elements 4g .. 4g + 3) of lane L's MFMA block (i, j) in wave w sits at byte
        // ((((w * TM + i) * TN + j) * 4 + g) * 64 + L) * 16 of the 256 KB slot.
        // Stream-K tiles have two pieces: the tile's head, the last piece of its run, and the tail,
        // the first piece of the next run, which is nearly always done first.  The tail stores its
        // partial and adds 1.  The head first adds 2: if the tail's 1 is there, the head finishes
        // the tile without storing its own partial; otherwise it stores it and adds 4, and whoever
        // then sees both the other's publication (1 or 4) finishes the tile.  Exactly one does,
        // after both partials it reads are stored.
        bool publish = ctail;
        const bool sk = sp.split == 0;
        const bool head = sk && cord == 0;
        if (ctail && head) {
            __syncthreads();
            if (tid == 0) {
                const unsigned int v = split_arrive(sp.counters + ctile, 2u);
                if (v & 1u) split_reset(sp.counters + ctile);   // the tail has arrived: this block finishes
                s_flag[0] = static_cast<int>(v);
            }
            __syncthreads();
            publish = (static_cast<unsigned int>(s_flag[0]) & 1u) == 0u;
        }
        if (publish) {
            const __amdgpu_buffer_rsrc_t rsm = part_rsrc(piece_slot(cfirst, cord));
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        __builtin_amdgcn_raw_buffer_store_b128(
                            v4i{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]}, rsm,
                            part_lane, part_soff(i, j, g), 0);
            // All blocks of a split tile run on one XCD, so its L2 is the point of coherence: the
            // stores have reached it once they are acknowledged, the counter's atomic executes
            // there, and the last block reads the partials with loads that bypass its own L1.
            RTQ_WAIT_ALL_VMEM();
            __syncthreads();
            if (tid == 0) {
                const unsigned int v = split_arrive(sp.counters + ctile, sk ? (head ? 4u : 1u) : 1u);
                const bool last = sk ? (v & (head ? 1u : 4u)) != 0u : v == static_cast<unsigned int>(ccount - 1);
                if (last) split_reset(sp.counters + ctile);    // nobody arrives on this tile again
                s_flag[0] = last;
            }
            __syncthreads();
            epilogue = s_flag[0] != 0;
        }
        // The finishing block adds the other pieces' partials (stored before their arrivals, read
        // from the XCD's L2 past this block's L1) into its accumulators, one 32 x 32 MFMA block (four
        // 1 KB loads per wave) at a time.
        if (epilogue && ctail) {
            for (int o = 0; o < ccount; ++o) {
                if (o == cord) continue;
                const __amdgpu_buffer_rsrc_t rso = part_rsrc(piece_slot(cfirst, o));
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        v4i part[4];
#pragma unroll
                        for (int g = 0; g < 4; ++g)
                            part[g] = __builtin_amdgcn_raw_buffer_load_b128(rso, part_lane, part_soff(i, j, g), kLoadL2);
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            acc[i][j][4 * g] += part[g].x;
                            acc[i][j][4 * g + 1] += part[g].y;
                            acc[i][j][4 * g + 2] += part[g].z;
                            acc[i][j][4 * g + 3] += part[g].w;
                        }
                    }
            }
        }

        // Zero points: sum_j (qa - za)(qw - zw) = acc - zw * sum(qa) - za * (sum(qw) - d zw), exact
        // in int32 (24-bit multiplies: |zero| <= 128, |sums| <= 2^22).
        auto correct = [&](v4i a, int row, int col) -> v4i {
            if constexpr (kAsym) {
                const int A = s_z[row], B = s_e[row];
                const v4i C = *reinterpret_cast<const v4i*>(s_z + BM + col);
                const v4i E = *reinterpret_cast<const v4i*>(s_e + BM + col);
                a.x -= __mul24(C.x, B) + __mul24(A, E.x);
                a.y -= __mul24(C.y, B) + __mul24(A, E.y);
                a.z -= __mul24(C.z, B) + __mul24(A, E.z);
                a.w -= __mul24(C.w, B) + __mul24(A, E.w);
            }
            return a;
        };

        // ---- epilogue.  Each wave stages its raw int32 block one 32-row MFMA block at a time, reads
        // it back row-contiguously, scales and converts, and stores: the
        // lanes of one row write a whole run of the wave's columns (128-512 bytes), so the
        // streaming stores are full cache lines.  Stores go through a descriptor that ends at the
        // tile's last valid row; columns past N are sent past its range.  kVec (N % 8 == 0): an
        // output chunk of 16 bytes is wholly inside or outside [0, N).
        if (epilogue) {
            constexpr int kOutBytes = kYKind == 1 ? 2 : 4;
            constexpr int kPerChunk = 16 / kOutBytes;              // outputs per 16-byte store
            constexpr int kChunksPerRow = WN / kPerChunk;
            constexpr int kChunksPerLane = kPassRows * kChunksPerRow / 64;
            constexpr uint32_t kOob = 0x80000000u;
            // A lane's read-back chunk is column chunk lane % kChunksPerRow of every row it handles
            // (64 is a multiple of kChunksPerRow), so its output-column scales are read once per tile.
            static_assert(64 % kChunksPerRow == 0, "a lane's column chunk is the same in every pass");
            float wsl[kPerChunk];
            if constexpr (kYKind != 2) {
#pragma unroll
                for (int h4 = 0; h4 < kPerChunk / 4; ++h4) {
                    const float4 v = *reinterpret_cast<const float4*>(s_ws + wn * WN + (lane % kChunksPerRow) * kPerChunk + 4 * h4);
                    wsl[4 * h4 + 0] = v.x;
                    wsl[4 * h4 + 1] = v.y;
                    wsl[4 * h4 + 2] = v.z;
                    wsl[4 * h4 + 3] = v.w;
                }
            }
            const int rows_y = static_cast<int>(min<int64_t>(BM, T - cm0));
            const __amdgpu_buffer_rsrc_t rsy = __builtin_amdgcn_make_buffer_rsrc(
                static_cast<int8_t*>(Y) + cm0 * N * kOutBytes, (short)0, static_cast<int>(rows_y * N * kOutBytes),
                kBufferWord3);
            if constexpr (kYKind == 1 && !kAsym) {
                // bf16 output: each lane scales and converts its accumulators where they are (token
                // row fr, columns 8g + 4fh .. +3 of block j), stages them as bf16 rows (half the LDS
                // bytes of int32 staging) and reads back whole 16-byte chunks to store.  The 16-byte
                // chunk k of a staged row r sits at chunk k ^ ((r >> 1) & 7): both the 8-byte writes (32
                // rows at once) and the 16-byte reads (8 rows) then touch every bank equally often.
                // Same arithmetic as below: (float(acc) * a_t) * w_n, rounded to bf16 once.
                constexpr int kRowB = WN * 2;                          // a wave's 64 bf16 outputs of a row
                static_assert(kPassRows * kRowB <= kPassRows * kPitch, "fits the wave's staging region");
                float4 wsv[TN][4];
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        wsv[j][g] = *reinterpret_cast<const float4*>(s_ws + wn * WN + j * 32 + 8 * g + 4 * fh);
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const float as = s_as[wm * WM + i * 32 + fr];
                    int8_t* wrow = stg + fr * kRowB;
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const float y0 = static_cast<float>(acc[i][j][4 * g]) * as * wsv[j][g].x;
                            const float y1 = static_cast<float>(acc[i][j][4 * g + 1]) * as * wsv[j][g].y;
                            const float y2 = static_cast<float>(acc[i][j][4 * g + 2]) * as * wsv[j][g].z;
                            const float y3 = static_cast<float>(acc[i][j][4 * g + 3]) * as * wsv[j][g].w;
                            *reinterpret_cast<uint2*>(wrow + ((((4 * j + g) ^ ((fr >> 1) & 7)) << 4) + 8 * fh)) =
                                make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
                        }
                    RTQ_LDS_FENCE();   // the wave's rows are in LDS before they are read back
#pragma unroll 1
                    for (int p = 0; p < kChunksPerLane; ++p) {
                        const int q = p * 64 + lane;
                        const int r = q / kChunksPerRow, c = q % kChunksPerRow;
                        const int trow = wm * WM + i * 32 + r;
                        const int col = wn * WN + c * kPerChunk;
                        const v4i out = *reinterpret_cast<const v4i*>(stg + r * kRowB + ((c ^ ((r >> 1) & 7)) << 4));
                        const int64_t n = cn0 + col;
                        const uint32_t off = (static_cast<uint32_t>(trow) * static_cast<uint32_t>(N) +
                                              static_cast<uint32_t>(n)) * kOutBytes;
                        if (kVec) {
                            __builtin_amdgcn_raw_buffer_store_b128(out, rsy, static_cast<int>(n < N ? off : kOob), 0,
                                                                   kStoreNT);
                        } else {
                            const uint32_t w[4] = {static_cast<uint32_t>(out.x), static_cast<uint32_t>(out.y),
                                                   static_cast<uint32_t>(out.z), static_cast<uint32_t>(out.w)};
#pragma unroll
                            for (int e = 0; e < kPerChunk; ++e) {
                                const int o = static_cast<int>(n + e < N ? off + e * kOutBytes : kOob);
                                __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1))),
                                                                      rsy, o, 0, kStoreNT);
                            }
                        }
                    }
                    RTQ_LDS_FENCE();   // read back before the next block overwrites the region
                }
            } else {
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    stage_block(i);
#pragma unroll 1
                    for (int p = 0; p < kChunksPerLane; ++p) {
                        const int q = p * 64 + lane;
                        const int r = q / kChunksPerRow, c = q % kChunksPerRow;
                        const int trow = wm * WM + i * 32 + r;              // row within the tile
                        const int col = wn * WN + c * kPerChunk;            // column within the tile
                        const int8_t* src = stg + r * kPitch;
                        constexpr int kQuads = kPerChunk / 4;               // 16-byte int32 chunks per output chunk
                        v4i out;
                        if (kYKind == 2) {
                            out = correct(*reinterpret_cast<const v4i*>(src + swz(r, c)), trow, col);
                        } else {
                            const float as = s_as[trow];
                            float y[kPerChunk];
#pragma unroll
                            for (int h4 = 0; h4 < kPerChunk / 4; ++h4) {
                                const v4i a = correct(*reinterpret_cast<const v4i*>(src + swz(r, kQuads * c + h4)),
                                                      trow, col + 4 * h4);
                                y[4 * h4 + 0] = static_cast<float>(a.x) * as * wsl[4 * h4 + 0];
                                y[4 * h4 + 1] = static_cast<float>(a.y) * as * wsl[4 * h4 + 1];
                                y[4 * h4 + 2] = static_cast<float>(a.z) * as * wsl[4 * h4 + 2];
                                y[4 * h4 + 3] = static_cast<float>(a.w) * as * wsl[4 * h4 + 3];
                            }
                            if (kYKind == 0) {
                                out = v4i{static_cast<int>(__float_as_uint(y[0])), static_cast<int>(__float_as_uint(y[1])),
                                          static_cast<int>(__float_as_uint(y[2])), static_cast<int>(__float_as_uint(y[3]))};
                            } else {
                                uint32_t w[4];
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    w[e] = pack_bf16x2(y[2 * e], y[2 * e + 1]);
                                out = v4i{static_cast<int>(w[0]), static_cast<int>(w[1]), static_cast<int>(w[2]),
                                          static_cast<int>(w[3])};
                            }
                        }
                        const int64_t n = cn0 + col;
                        const uint32_t off = (static_cast<uint32_t>(trow) * static_cast<uint32_t>(N) +
                                              static_cast<uint32_t>(n)) * kOutBytes;
                        if (kVec) {
                            __builtin_amdgcn_raw_buffer_store_b128(out, rsy, static_cast<int>(n < N ? off : kOob), 0,
                                                                   kStoreNT);
                        } else {
                            const uint32_t w[4] = {static_cast<uint32_t>(out.x), static_cast<uint32_t>(out.y),
                                                   static_cast<uint32_t>(out.z), static_cast<uint32_t>(out.w)};
#pragma unroll
                            for (int e = 0; e < kPerChunk; ++e) {
                                const int o = static_cast<int>(n + e < N ? off + e * kOutBytes : kOob);
                                if (kOutBytes == 4)
                                    __builtin_amdgcn_raw_buffer_store_b32(w[e], rsy, o, 0, kStoreNT);
                                else
                                    __builtin_amdgcn_raw_buffer_store_b16(
                                        static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1))), rsy, o, 0, kStoreNT);
                            }
                        }
                    }
                    RTQ_LDS_FENCE();   // read back before the next pass overwrites the region
                }
            }
        }
        RTQ_BARRIER();   // every wave is done with the staging slots and the scales
        if (!more) break;
    }
}

template <int kWavesN, int kWBits, bool kAsym, bool kTiled = false>
hipError_t launch_config(const GemmI8Args& g, hipStream_t stream) {
    static_assert(!kTiled || !kAsym, "the tiled layouts hold symmetric codes");
    using KernelFn = void (*)(const int8_t*, const float*, const int8_t*, const void*, int64_t, int64_t, int,
                              void*, int, int, const float*, int, const float*, SplitArgs, AsymArgs);
    constexpr int kYKinds = 3;   // fp32, bf16, raw int32 accumulators
    constexpr int kLdsBytes = lds_bytes(kWBits) + (kAsym ? kAsymBytes : 0);
    static_assert(kLdsBytes <= 160 * 1024, "LDS");
    // [w_scale bf16][N % 8 == 0][y kind]
    static const KernelFn kernels[2][2][3] = {
        {{gemm_i8_kernel<kWavesN, 0, false, false, kWBits, kAsym, kTiled>, gemm_i8_kernel<kWavesN, 1, false, false, kWBits, kAsym, kTiled>,
          kYKinds > 2 ? gemm_i8_kernel<kWavesN, kYKinds - 1, false, false, kWBits, kAsym, kTiled> : nullptr},
         {gemm_i8_kernel<kWavesN, 0, false, true, kWBits, kAsym, kTiled>, gemm_i8_kernel<kWavesN, 1, false, true, kWBits, kAsym, kTiled>,
          kYKinds > 2 ? gemm_i8_kernel<kWavesN, kYKinds - 1, false, true, kWBits, kAsym, kTiled> : nullptr}},
        {{gemm_i8_kernel<kWavesN, 0, true, false, kWBits, kAsym, kTiled>, gemm_i8_kernel<kWavesN, 1, true, false, kWBits, kAsym, kTiled>,
          kYKinds > 2 ? gemm_i8_kernel<kWavesN, kYKinds - 1, true, false, kWBits, kAsym, kTiled> : nullptr},
         {gemm_i8_kernel<kWavesN, 0, true, true, kWBits, kAsym, kTiled>, gemm_i8_kernel<kWavesN, 1, true, true, kWBits, kAsym, kTiled>,
          kYKinds > 2 ? gemm_i8_kernel<kWavesN, kYKinds - 1, true, true, kWBits, kAsym, kTiled> : nullptr}}};
    static const hipError_t attr_err = [] {
        hipError_t e = hipSuccess;
        for (auto& a : kernels)
            for (auto& b : a)
                for (KernelFn k : b) {
                    if (k == nullptr) continue;
                    const hipError_t r = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                                             hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
                    if (r != hipSuccess) e = r;
                }
        return e;
    }();
    if (attr_err != hipSuccess) return attr_err;
    if (g.y_kind < 0 || g.y_kind >= kYKinds) return hipErrorInvalidValue;
    const int64_t tiles_m = (g.T + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
    const int64_t total = tiles_m * tiles_n;
    if (total > (int64_t(1) << 30)) return hipErrorInvalidValue;
    // persistent grid: one block per compute unit (the LDS allows one), a multiple of the XCD count,
    // and no more blocks than tiles (rounded up to that multiple)
    const int cus = device_cu_count();
    if (cus <= 0) return hipErrorInvalidDevice;
    const int64_t slots = std::max<int64_t>(kXcds, cus / kXcds * kXcds);
    int64_t grid = std::min<int64_t>(slots, (total + kXcds - 1) / kXcds * kXcds);
    SplitArgs sp{static_cast<int>(total), 1, nullptr, nullptr};
    // With a workspace, a partial last round is shared along K (tiles of at least 16 stages):
    //  * after at least one full round: stream-K over the last full round and the remainder, so
    //    every block runs the same number of K stages (measured up to 3% faster than leaving half
    //    the blocks idle in a last half round, 8-11% at 1.125 rounds);
    //  * with no full round, when the tiles would leave at least 3/4 of the slots idle: each of the
    //    `rem` tiles in min(slots / rem, K stages / 16, kMaxSplit) equal ranges.
    if (g.workspace != nullptr && g.ws_bytes >= gemm_i8_workspace_bytes()) {
        const int64_t whole = total / slots * slots;
        const int64_t rem = total - whole;
        const int64_t nk = g.d / BK;
        int64_t dp = total, split = 1;
        if (rem > 0 && nk >= 16) {
            if (whole >= slots) {
                dp = whole - slots;
                split = 0;
            } else if (4 * rem <= slots) {
                split = std::min<int64_t>(std::min<int64_t>(slots / rem, nk / 16),
                                          std::min<int64_t>(slots / kXcds, kMaxSplit));
                // a power of two: the blocks per XCD are a multiple of it, so a tile's ranges share an XCD
                while (split & (split - 1)) split &= split - 1;
                if ((slots / kXcds) % split != 0) split = 1;
                dp = split >= 2 ? whole : total;
            }
        }
        if (dp < total) {
            unsigned char* ws = static_cast<unsigned char*>(g.workspace);
            sp = SplitArgs{static_cast<int>(dp), static_cast<int>(split), reinterpret_cast<v4i*>(ws),
                           reinterpret_cast<unsigned long long*>(
                               ws + static_cast<size_t>(partial_slots_cap(slots)) * BM * BN * 4)};
            grid = slots;
        }
    }
    const KernelFn k = kernels[g.w_scale_bf16 ? 1 : 0][(g.N % 8) == 0 ? 1 : 0][g.y_kind];
    hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(grid)), dim3(64 * kWavesM * kWavesN), kLdsBytes, stream, g.a,
                       g.a_scale, g.w, g.w_scale, g.T, g.N, g.d, g.y, static_cast<int>(tiles_m),
                       static_cast<int>(tiles_n), g.cent_a, g.a_bits, g.cent_w, sp,
                       AsymArgs{g.a_zero, g.a_sum, g.w_zero, g.w_sum});
    return hipGetLastError();
}

}  // namespace

size_t gemm_i8_workspace_bytes() {
    const int cus = device_cu_count();
    const int64_t slots = std::max<int64_t>(kXcds, cus / kXcds * kXcds);
    // partial tiles (int32) and one counter per shared tile
    return static_cast<size_t>(partial_slots_cap(slots)) * BM * BN * 4 +
           static_cast<size_t>(shared_tiles_cap(slots)) * sizeof(unsigned long long);
}

unsigned long long* gemm_i8_split_counters(void* workspace, size_t ws_bytes, int* n) {
    *n = 0;
    if (workspace == nullptr || ws_bytes < gemm_i8_workspace_bytes()) return nullptr;
    const int cus = device_cu_count();
    const int64_t slots = std::max<int64_t>(kXcds, cus / kXcds * kXcds);
    *n = static_cast<int>(shared_tiles_cap(slots));
    return reinterpret_cast<unsigned long long*>(static_cast<unsigned char*>(workspace) +
                                                 static_cast<size_t>(partial_slots_cap(slots)) * BM * BN * 4);
}

hipError_t launch_split_clear(unsigned long long* counters, int n, hipStream_t stream) {
    if (counters == nullptr || n <= 0) return hipSuccess;
    hipLaunchKernelGGL(split_clear_kernel, dim3(1), dim3(256), 0, stream, counters, n);
    return hipGetLastError();
}

int64_t gemm_i8_max_n(int y_kind) { return y_kind == 1 ? (int64_t(1) << 22) : (int64_t(1) << 21); }

hipError_t launch_gemm_i8(const GemmI8Args& g, hipStream_t stream) {
    if (g.T <= 0 || g.N <= 0) return hipSuccess;
    if (g.d % BK != 0 || g.d > 16384) return hipErrorInvalidValue;
    // the epilogue's store descriptor spans one 256-row block of Y (at most 2^31 bytes, so its
    // byte offsets and the out-of-range sentinel 2^31 fit its 32-bit range)
    if (g.N > gemm_i8_max_n(g.y_kind)) return hipErrorInvalidValue;
    const bool asym = g.a_zero != nullptr;
    if (asym != (g.a_sum != nullptr) || asym != (g.w_zero != nullptr) || asym != (g.w_sum != nullptr))
        return hipErrorInvalidValue;
    if (asym) return g.w_bits == 8 && !g.tiled ? launch_config<kDefaultWavesN, 8, true>(g, stream) : hipErrorInvalidValue;
    const bool coded = g.w_bits != 8;
    if (coded && (g.cent_a == nullptr || g.cent_w == nullptr || g.a_bits < 1 || g.a_bits > 6)) return hipErrorInvalidValue;
    if (g.tiled) {
        switch (g.w_bits) {
            case 8: return launch_config<kDefaultWavesN, 8, false, true>(g, stream);
            case 4: return launch_config<kDefaultWavesN, 4, false, true>(g, stream);
            case 3: return launch_config<kDefaultWavesN, 3, false, true>(g, stream);
            case 2: return launch_config<kDefaultWavesN, 2, false, true>(g, stream);
        }
        return hipErrorInvalidValue;
    }
    switch (g.w_bits) {
        case 8: return launch_config<kDefaultWavesN, 8, false>(g, stream);
        case 4: return launch_config<kDefaultWavesN, 4, false>(g, stream);
        case 3: return launch_config<kDefaultWavesN, 3, false>(g, stream);
        case 2: return launch_config<kDefaultWavesN, 2, false>(g, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace rtq
