// rtq_api.cpp -- the C ABI of librtq: argument checks, error reporting, and kernel dispatch.
// Every check runs on the host before anything is enqueued; a non-OK status means no work was
// queued.  Kernel launches go to the caller's stream and never allocate device memory.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>

#include "../../include/rtq.h"
#include "rtq_host.h"
#include "rtq_internal.h"

namespace {

thread_local std::string g_err;

rtq_status fail(rtq_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

rtq_status ok() {
    g_err.clear();
    return RTQ_OK;
}

rtq_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(RTQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define RTQ_TRY(expr)                     \
    do {                                  \
        rtq_status _s = (expr);           \
        if (_s != RTQ_OK) return _s;      \
    } while (0)

rtq_status check_ptr(const void* p, const char* name) {
    if (p == nullptr) return fail(RTQ_ERR_INVALID_ARG, "%s is NULL", name);
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return fail(RTQ_ERR_MISALIGNED, "%s is not 16-byte aligned", name);
    return RTQ_OK;
}

// d: a multiple of 64 whose block count d/64 is a power of two, 64..16384.
rtq_status check_d(int64_t d) {
    if (d <= 0) return fail(RTQ_ERR_INVALID_ARG, "d must be positive (got %lld)", static_cast<long long>(d));
    if (d % 64 != 0) return fail(RTQ_ERR_INVALID_ARG, "d must be a multiple of the block size 64 (got %lld)",
                                 static_cast<long long>(d));
    const int64_t nb = d / 64;
    if ((nb & (nb - 1)) != 0 || d > 16384)
        return fail(RTQ_ERR_UNSUPPORTED, "d/64 must be a power of two and d <= 16384 (got d=%lld)",
                    static_cast<long long>(d));
    return RTQ_OK;
}

rtq_status check_rpbh(const rtq_rpbh* R, int64_t d) {
    if (R == nullptr) return fail(RTQ_ERR_INVALID_ARG, "rpbh descriptor is NULL");
    if (R->h != 64) return fail(RTQ_ERR_UNSUPPORTED, "only h = 64 is supported (got %d)", R->h);
    if (R->d != d) return fail(RTQ_ERR_INVALID_ARG, "descriptor d=%d does not match d=%lld", R->d,
                               static_cast<long long>(d));
    RTQ_TRY(check_d(d));
    RTQ_TRY(check_ptr(R->perm, "rpbh.perm"));
    RTQ_TRY(check_ptr(R->signs, "rpbh.signs"));
    return RTQ_OK;
}

rtq_status check_float_dtype(rtq_dtype t, const char* name) {
    if (t != RTQ_F32 && t != RTQ_BF16) return fail(RTQ_ERR_UNSUPPORTED, "%s must be RTQ_F32 or RTQ_BF16", name);
    return RTQ_OK;
}

rtq_status check_codebook(const rtq_codebook* cb, const char* name, bool need_centroids, bool need_bounds) {
    if (cb == nullptr) return fail(RTQ_ERR_INVALID_ARG, "%s is NULL", name);
    if (cb->bits != 2 && cb->bits != 3 && cb->bits != 4 && cb->bits != 6)
        return fail(RTQ_ERR_UNSUPPORTED, "%s.bits must be 2, 3, 4 or 6 (got %d)", name, cb->bits);
    if (need_centroids && cb->centroids == nullptr) return fail(RTQ_ERR_INVALID_ARG, "%s.centroids is NULL", name);
    if (need_bounds && cb->boundaries == nullptr) return fail(RTQ_ERR_INVALID_ARG, "%s.boundaries is NULL", name);
    return RTQ_OK;
}

rtq_status plan_quantize(const void* x, rtq_dtype xt, int64_t rows, int32_t d, const rtq_rpbh* R, rtq_qmode mode,
                         const rtq_codebook* cb, float eps, void* codes, void* scale, rtq_dtype scale_t,
                         rtq::RowArgs* out) {
    if (rows < 0) return fail(RTQ_ERR_INVALID_ARG, "rows must be >= 0");
    RTQ_TRY(check_d(d));
    if (R != nullptr) RTQ_TRY(check_rpbh(R, d));
    RTQ_TRY(check_float_dtype(xt, "xt"));
    RTQ_TRY(check_float_dtype(scale_t, "scale_t"));
    RTQ_TRY(check_ptr(x, "x"));
    RTQ_TRY(check_ptr(codes, "codes"));
    if (scale == nullptr) return fail(RTQ_ERR_INVALID_ARG, "scale is NULL");
    if (reinterpret_cast<uintptr_t>(scale) % 4 != 0) return fail(RTQ_ERR_MISALIGNED, "scale is not 4-byte aligned");
    rtq::RowArgs a{};
    a.x = x;
    a.x_bf16 = xt == RTQ_BF16;
    a.rows = rows;
    a.d = d;
    a.perm = R ? R->perm : nullptr;
    a.signs = R ? R->signs : nullptr;
    a.out = codes;
    a.scale = scale;
    a.scale_bf16 = scale_t == RTQ_BF16;
    a.eps = eps;
    if (mode == RTQ_INT8 || mode == RTQ_INT8_TILED) {
        if (cb != nullptr) return fail(RTQ_ERR_INVALID_ARG, "cb must be NULL for RTQ_INT8 and RTQ_INT8_TILED");
        a.out_kind = rtq::kRowInt8;
        a.bounds = nullptr;
        a.tiled = mode == RTQ_INT8_TILED;
    } else if (mode == RTQ_CODEBOOK || mode == RTQ_CODEBOOK_TILED) {
        RTQ_TRY(check_codebook(cb, "cb", false, true));
        if (!(eps >= 0.0f) || std::isinf(eps)) return fail(RTQ_ERR_INVALID_ARG, "eps must be finite and >= 0");
        if (cb->bits == 6) return fail(RTQ_ERR_UNSUPPORTED, "packed 6-bit codes are not supported (use RTQ_CODEBOOK_I8)");
        a.out_kind = cb->bits == 4 ? rtq::kRowCode4 : (cb->bits == 3 ? rtq::kRowCode3 : rtq::kRowCode2);
        a.bounds = cb->boundaries;
        a.tiled = mode == RTQ_CODEBOOK_TILED;
    } else if (mode == RTQ_CODEBOOK_I8 || mode == RTQ_CODEBOOK_I8_TILED) {
        RTQ_TRY(check_codebook(cb, "cb", true, true));
        if (!(eps >= 0.0f) || std::isinf(eps)) return fail(RTQ_ERR_INVALID_ARG, "eps must be finite and >= 0");
        a.out_kind = cb->bits == 4 ? rtq::kRowLut4
                     : cb->bits == 3 ? rtq::kRowLut3
                     : cb->bits == 6 ? rtq::kRowLut6
                                     : rtq::kRowLut2;
        a.bounds = cb->boundaries;
        a.centroids = cb->centroids;
        a.tiled = mode == RTQ_CODEBOOK_I8_TILED;
    } else {
        return fail(RTQ_ERR_INVALID_ARG, "unknown mode %d", static_cast<int>(mode));
    }
    if ((a.out_kind == rtq::kRowCode3 || a.out_kind == rtq::kRowLut3 || a.out_kind == rtq::kRowLut6) &&
        (!a.x_bf16 || a.perm == nullptr))
        return fail(RTQ_ERR_UNSUPPORTED, "3- and 6-bit codes need bf16 rows and a rotation descriptor");
    *out = a;
    return RTQ_OK;
}

struct GemmPlan {
    bool lut;
    rtq::GemmI8Args i8;
    rtq::GemmLutArgs cb;
};

rtq_status plan_gemm(const void* a_codes, const float* a_scale, int64_t T, const void* w_codes, const void* w_scale,
                     rtq_dtype w_scale_t, int64_t N, int32_t d, rtq_qmode mode, const rtq_codebook* cb_a,
                     const rtq_codebook* cb_w, void* y, rtq_dtype yt, GemmPlan* out) {
    if (T < 0) return fail(RTQ_ERR_INVALID_ARG, "T must be >= 0");
    if (N <= 0) return fail(RTQ_ERR_INVALID_ARG, "N must be positive");
    RTQ_TRY(check_d(d));
    RTQ_TRY(check_ptr(a_codes, "a_codes"));
    RTQ_TRY(check_ptr(w_codes, "w_codes"));
    RTQ_TRY(check_ptr(y, "y"));
    if (a_scale == nullptr || w_scale == nullptr) return fail(RTQ_ERR_INVALID_ARG, "scale pointer is NULL");
    if (reinterpret_cast<uintptr_t>(a_scale) % 4 != 0) return fail(RTQ_ERR_MISALIGNED, "a_scale is not 4-byte aligned");
    if (reinterpret_cast<uintptr_t>(w_scale) % 2 != 0) return fail(RTQ_ERR_MISALIGNED, "w_scale is not 2-byte aligned");
    RTQ_TRY(check_float_dtype(w_scale_t, "w_scale_t"));
    if (w_scale_t == RTQ_F32 && reinterpret_cast<uintptr_t>(w_scale) % 4 != 0)
        return fail(RTQ_ERR_MISALIGNED, "w_scale is not 4-byte aligned");
    if ((T + 127) / 128 > 65535) return fail(RTQ_ERR_UNSUPPORTED, "T too large (max %d)", 65535 * 128);
    GemmPlan p{};
    if (mode == RTQ_INT8 || mode == RTQ_INT8_TILED) {
        if (cb_a != nullptr || cb_w != nullptr)
            return fail(RTQ_ERR_INVALID_ARG, "codebooks must be NULL for RTQ_INT8 and RTQ_INT8_TILED");
        if (yt != RTQ_F32 && yt != RTQ_BF16 && yt != RTQ_I32) return fail(RTQ_ERR_UNSUPPORTED, "bad yt");
        const int y_kind = yt == RTQ_F32 ? 0 : (yt == RTQ_BF16 ? 1 : 2);
        if (N > rtq::gemm_i8_max_n(y_kind))
            return fail(RTQ_ERR_UNSUPPORTED, "N too large for this output type (max %lld)",
                        static_cast<long long>(rtq::gemm_i8_max_n(y_kind)));
        p.lut = false;
        p.i8 = rtq::GemmI8Args{static_cast<const int8_t*>(a_codes), a_scale, static_cast<const int8_t*>(w_codes),
                               w_scale, w_scale_t == RTQ_BF16, T, N, d, y,
                               yt == RTQ_F32 ? 0 : (yt == RTQ_BF16 ? 1 : 2)};
        p.i8.tiled = mode == RTQ_INT8_TILED;
    } else if (mode == RTQ_CODEBOOK) {
        RTQ_TRY(check_codebook(cb_a, "cb_a", true, false));
        RTQ_TRY(check_codebook(cb_w, "cb_w", true, false));
        if (cb_a->bits != 4) return fail(RTQ_ERR_UNSUPPORTED, "activation codes must be 4-bit (got %d)", cb_a->bits);
        if (cb_w->bits != 2 && cb_w->bits != 4)
            return fail(RTQ_ERR_UNSUPPORTED, "RTQ_CODEBOOK weight codes must be 2- or 4-bit (got %d)", cb_w->bits);
        if (yt != RTQ_BF16) return fail(RTQ_ERR_UNSUPPORTED, "codebook products give bf16 output (yt must be RTQ_BF16)");
        p.lut = true;
        p.cb = rtq::GemmLutArgs{static_cast<const uint8_t*>(a_codes), a_scale, static_cast<const uint8_t*>(w_codes),
                                w_scale, w_scale_t == RTQ_BF16, cb_a->centroids, cb_w->centroids, cb_a->bits,
                                cb_w->bits, T, N, d, y, yt == RTQ_F32 ? 0 : 1};
    } else if (mode == RTQ_CODEBOOK_TILED) {
        return fail(RTQ_ERR_UNSUPPORTED, "RTQ_CODEBOOK_TILED is a weight-code layout: multiply in RTQ_CODEBOOK_I8_TILED");
    } else if (mode == RTQ_CODEBOOK_I8 || mode == RTQ_CODEBOOK_I8_TILED) {
        RTQ_TRY(check_codebook(cb_a, "cb_a", true, false));
        RTQ_TRY(check_codebook(cb_w, "cb_w", true, false));
        if (cb_w->bits == 6) return fail(RTQ_ERR_UNSUPPORTED, "weight codes must be 2-, 3- or 4-bit (got 6)");
        if (yt != RTQ_BF16 && yt != RTQ_I32)
            return fail(RTQ_ERR_UNSUPPORTED, "codebook products give bf16 output (yt must be RTQ_BF16, or RTQ_I32 "
                                             "for the raw int8-value accumulators)");
        const int y_kind = yt == RTQ_BF16 ? 1 : 2;
        if (N > rtq::gemm_i8_max_n(y_kind))
            return fail(RTQ_ERR_UNSUPPORTED, "N too large for this output type (max %lld)",
                        static_cast<long long>(rtq::gemm_i8_max_n(y_kind)));
        p.lut = false;
        p.i8 = rtq::GemmI8Args{static_cast<const int8_t*>(a_codes), a_scale, static_cast<const int8_t*>(w_codes),
                               w_scale, w_scale_t == RTQ_BF16, T, N, d, y, y_kind};
        p.i8.w_bits = cb_w->bits;
        p.i8.cent_a = cb_a->centroids;
        p.i8.a_bits = cb_a->bits;
        p.i8.cent_w = cb_w->centroids;
        p.i8.tiled = mode == RTQ_CODEBOOK_I8_TILED;
    } else {
        return fail(RTQ_ERR_INVALID_ARG, "unknown mode %d", static_cast<int>(mode));
    }
    *out = p;
    return RTQ_OK;
}

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

// Bytes of rtq_rotated_qlinear's workspace: codes and scales (required), then the product's
// K-split region (used when present; see rtq_qgemm_ws).
size_t workspace_bytes(int64_t T, int32_t d, rtq_qmode mode, int32_t bits_a, bool with_split = true) {
    if (T < 0 || d <= 0) return 0;
    size_t code_bytes;
    if (mode == RTQ_INT8_TILED || (mode == RTQ_CODEBOOK_I8_TILED && (bits_a == 2 || bits_a == 3 || bits_a == 4 || bits_a == 6)))
        code_bytes = static_cast<size_t>(rtq::tiled_rows(T)) * static_cast<size_t>(d);
    else if (mode == RTQ_INT8 || (mode == RTQ_CODEBOOK_I8 && (bits_a == 2 || bits_a == 3 || bits_a == 4 || bits_a == 6)))
        code_bytes = static_cast<size_t>(T) * static_cast<size_t>(d);
    else if (mode == RTQ_CODEBOOK && (bits_a == 2 || bits_a == 4))
        code_bytes = static_cast<size_t>(T) * static_cast<size_t>(d) * static_cast<size_t>(bits_a) / 8;
    else
        return 0;
    return align256(code_bytes) + align256(static_cast<size_t>(T) * sizeof(float)) +
           (with_split && mode != RTQ_CODEBOOK ? align256(rtq::gemm_i8_workspace_bytes()) : 0);
}


rtq_status plan_gemm_asym(const int8_t* a_codes, const float* a_scale, const int32_t* a_zero, const int32_t* a_sum,
                          int64_t T, const int8_t* w_codes, const void* w_scale, rtq_dtype w_scale_t,
                          const int32_t* w_zero, const int32_t* w_sum, int64_t N, int32_t d, void* y, rtq_dtype yt,
                          GemmPlan* p) {
    RTQ_TRY(plan_gemm(a_codes, a_scale, T, w_codes, w_scale, w_scale_t, N, d, RTQ_INT8, nullptr, nullptr, y, yt, p));
    const int32_t* ptrs[4] = {a_zero, a_sum, w_zero, w_sum};
    for (const int32_t* q : ptrs) {
        if (q == nullptr) return fail(RTQ_ERR_INVALID_ARG, "zero point or code sum pointer is NULL");
        if (reinterpret_cast<uintptr_t>(q) % 4 != 0) return fail(RTQ_ERR_MISALIGNED, "zero/sum array not 4-byte aligned");
    }
    p->i8.a_zero = a_zero;
    p->i8.a_sum = a_sum;
    p->i8.w_zero = w_zero;
    p->i8.w_sum = w_sum;
    return RTQ_OK;
}

size_t asym_workspace_bytes(int64_t T, int32_t d, bool with_split) {
    if (T < 0 || d <= 0) return 0;
    const size_t rows = static_cast<size_t>(T);
    return align256(rows * static_cast<size_t>(d)) + 3 * align256(rows * 4) +
           (with_split ? align256(rtq::gemm_i8_workspace_bytes()) : 0);
}

// Bytes of activation codes and scales the online layer needs (the workspace's required part).
rtq_status qlinear_need(const rtq_rpbh* R, int64_t T, rtq_qmode mode, const rtq_codebook* cb_a, size_t* need) {
    if (R == nullptr) return fail(RTQ_ERR_INVALID_ARG, "rpbh descriptor is NULL");
    RTQ_TRY(check_d(R->d));
    const bool cbook = mode == RTQ_CODEBOOK || mode == RTQ_CODEBOOK_I8 || mode == RTQ_CODEBOOK_I8_TILED;
    if (cbook && cb_a == nullptr) return fail(RTQ_ERR_INVALID_ARG, "cb_a is NULL");
    const int32_t bits_a = cbook ? cb_a->bits : 8;
    if (mode == RTQ_CODEBOOK && bits_a != 4)
        return fail(RTQ_ERR_UNSUPPORTED, "activation codes must be 4-bit (got %d)", bits_a);
    *need = workspace_bytes(T < 0 ? 0 : T, R->d, mode, bits_a, false);
    if (*need == 0 && T > 0) return fail(RTQ_ERR_INVALID_ARG, "unsupported mode or activation bits");
    return RTQ_OK;
}

// The online layer on a caller's workspace: rotate-quantise into its head, then the product.
rtq_status rotated_qlinear_ws(const void* x, rtq_dtype xt, int64_t T, const rtq_rpbh* R, const void* w_codes,
                              const void* w_scale, rtq_dtype w_scale_t, int64_t N, rtq_qmode mode,
                              const rtq_codebook* cb_a, const rtq_codebook* cb_w, void* y, rtq_dtype yt,
                              void* workspace, size_t ws_bytes, void* stream) {
    size_t need = 0;
    RTQ_TRY(qlinear_need(R, T, mode, cb_a, &need));
    const int32_t d = R->d;
    if (yt == RTQ_I32) return fail(RTQ_ERR_UNSUPPORTED, "rtq_rotated_qlinear produces F32 or BF16 output");
    const bool cbook = mode == RTQ_CODEBOOK || mode == RTQ_CODEBOOK_I8 || mode == RTQ_CODEBOOK_I8_TILED;
    const int32_t bits_a = cbook ? cb_a->bits : 8;
    // (need covers the codes and scales; a larger workspace also carries the product's K-split)
    if (workspace == nullptr) return fail(RTQ_ERR_INVALID_ARG, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return fail(RTQ_ERR_MISALIGNED, "workspace is not 16-byte aligned");
    if (ws_bytes < need) return fail(RTQ_ERR_INVALID_ARG, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    const int64_t rows = T < 0 ? 0 : T;
    const bool tiled = mode == RTQ_INT8_TILED || mode == RTQ_CODEBOOK_I8_TILED;
    const size_t code_bytes = mode == RTQ_CODEBOOK ? static_cast<size_t>(rows) * d * bits_a / 8
                              : tiled              ? static_cast<size_t>(rtq::tiled_rows(rows)) * d
                                                   : static_cast<size_t>(rows) * d;
    void* a_codes = ws;
    float* a_scale = reinterpret_cast<float*>(ws + align256(code_bytes));
    rtq::RowArgs qa{};
    RTQ_TRY(plan_quantize(x, xt, T, d, R, mode, cbook ? cb_a : nullptr, cbook ? 1e-8f : 0.0f, a_codes, a_scale,
                          RTQ_F32, &qa));
    GemmPlan gp{};
    RTQ_TRY(plan_gemm(a_codes, a_scale, T, w_codes, w_scale, w_scale_t, N, d, mode, cb_a, cb_w, y, yt, &gp));
    if (T == 0) return ok();
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t split_off = align256(code_bytes) + align256(static_cast<size_t>(T) * sizeof(float));
    if (!gp.lut) {
        // the quantiser launch zeroes the product's split counters (when the workspace has them)
        gp.i8.workspace = ws + split_off;
        gp.i8.ws_bytes = ws_bytes - split_off;
        qa.clear = rtq::gemm_i8_split_counters(gp.i8.workspace, gp.i8.ws_bytes, &qa.nclear);
    }
    RTQ_TRY(hip_status(rtq::launch_rpbh_rows(qa, s), "rpbh_rows launch"));
    if (gp.lut) return hip_status(rtq::launch_gemm_lut(gp.cb, s), "gemm_lut launch");
    return hip_status(rtq::launch_gemm_i8(gp.i8, s), "gemm_i8 launch");
}

// Device scratch of rtq_rotated_qlinear_noalloc: the activation codes, then the fp32 token scales
// (the head of rtq_rotated_qlinear's workspace, without the product's K-split region).  Each GPU
// the library runs on holds its own copy until the process ends; host code reaches it only
// through the address hipGetSymbolAddress returns on that device (the array's name is a host-side
// stand-in, not a device address).
constexpr size_t kScratchBytes = RTQ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_addr;   // device -> address of its copy of `scratch`

// The current device's copy of `scratch`, looked up once per device (with that device current).
rtq_status scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    auto it = g_scratch_addr.find(dev);
    if (it == g_scratch_addr.end()) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        if (p == nullptr || reinterpret_cast<uintptr_t>(p) % 256 != 0)
            return fail(RTQ_ERR_HIP, "hipGetSymbolAddress(scratch) returned an unaligned address");
        it = g_scratch_addr.emplace(dev, p).first;
    }
    *out = it->second;
    return RTQ_OK;
}

}  // namespace

extern "C" {

rtq_status rtq_rpbh_make(uint64_t seed, int32_t d, int32_t h, int32_t* perm_out, int8_t* signs_out) {
    if (perm_out == nullptr || signs_out == nullptr) return fail(RTQ_ERR_INVALID_ARG, "output pointer is NULL");
    if (h != 64) return fail(RTQ_ERR_UNSUPPORTED, "only h = 64 is supported (got %d)", h);
    if (d <= 0 || d % h != 0) return fail(RTQ_ERR_INVALID_ARG, "d must be a positive multiple of h (got %d)", d);
    rtq::make_rpbh(seed, d, perm_out, signs_out);
    return ok();
}

rtq_status rtq_lloyd_max(int32_t d, int32_t bits, float* centroids_out, float* boundaries_out) {
    if (centroids_out == nullptr || boundaries_out == nullptr) return fail(RTQ_ERR_INVALID_ARG, "output pointer is NULL");
    if (d <= 0) return fail(RTQ_ERR_INVALID_ARG, "d must be positive (got %d)", d);
    if (bits < 1 || bits > 8) return fail(RTQ_ERR_INVALID_ARG, "bits must be in 1..8 (got %d)", bits);
    rtq::lloyd_max(d, bits, centroids_out, boundaries_out);
    return ok();
}

rtq_status rtq_rpbh_rotate(const void* x, rtq_dtype xt, void* y, rtq_dtype yt, int64_t rows, const rtq_rpbh* R,
                           int32_t inverse, void* stream) {
    if (rows < 0) return fail(RTQ_ERR_INVALID_ARG, "rows must be >= 0");
    if (R == nullptr) return fail(RTQ_ERR_INVALID_ARG, "rpbh descriptor is NULL");
    RTQ_TRY(check_rpbh(R, R->d));
    RTQ_TRY(check_float_dtype(xt, "xt"));
    RTQ_TRY(check_float_dtype(yt, "yt"));
    RTQ_TRY(check_ptr(x, "x"));
    RTQ_TRY(check_ptr(y, "y"));
    if (inverse != 0 && inverse != 1) return fail(RTQ_ERR_INVALID_ARG, "inverse must be 0 or 1");
    if (rows == 0) return ok();
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (inverse) {
        return hip_status(rtq::launch_rpbh_inverse(x, xt == RTQ_BF16, y, yt == RTQ_BF16, rows, R->d, R->perm,
                                                   R->signs, s),
                          "rpbh_inverse launch");
    }
    rtq::RowArgs a{};
    a.x = x;
    a.x_bf16 = xt == RTQ_BF16;
    a.rows = rows;
    a.d = R->d;
    a.perm = R->perm;
    a.signs = R->signs;
    a.out_kind = yt == RTQ_BF16 ? rtq::kRowRotBF16 : rtq::kRowRotF32;
    a.out = y;
    return hip_status(rtq::launch_rpbh_rows(a, s), "rpbh_rows launch");
}

rtq_status rtq_quantize_rows(const void* x, rtq_dtype xt, int64_t rows, int32_t d, const rtq_rpbh* R,
                             rtq_qmode mode, const rtq_codebook* cb, float eps, void* codes, void* scale,
                             rtq_dtype scale_t, void* stream) {
    rtq::RowArgs a{};
    RTQ_TRY(plan_quantize(x, xt, rows, d, R, mode, cb, eps, codes, scale, scale_t, &a));
    if (rows == 0) return ok();
    return hip_status(rtq::launch_rpbh_rows(a, static_cast<hipStream_t>(stream)), "rpbh_rows launch");
}

rtq_status rtq_qgemm(const void* a_codes, const float* a_scale, int64_t T, const void* w_codes, const void* w_scale,
                     rtq_dtype w_scale_t, int64_t N, int32_t d, rtq_qmode mode, const rtq_codebook* cb_a,
                     const rtq_codebook* cb_w, void* y, rtq_dtype yt, void* stream) {
    GemmPlan p{};
    RTQ_TRY(plan_gemm(a_codes, a_scale, T, w_codes, w_scale, w_scale_t, N, d, mode, cb_a, cb_w, y, yt, &p));
    if (T == 0) return ok();
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.lut) return hip_status(rtq::launch_gemm_lut(p.cb, s), "gemm_lut launch");
    return hip_status(rtq::launch_gemm_i8(p.i8, s), "gemm_i8 launch");
}

rtq_status rtq_qgemm_ws(const void* a_codes, const float* a_scale, int64_t T, const void* w_codes,
                        const void* w_scale, rtq_dtype w_scale_t, int64_t N, int32_t d, rtq_qmode mode,
                        const rtq_codebook* cb_a, const rtq_codebook* cb_w, void* y, rtq_dtype yt,
                        void* workspace, size_t ws_bytes, void* stream) {
    GemmPlan p{};
    RTQ_TRY(plan_gemm(a_codes, a_scale, T, w_codes, w_scale, w_scale_t, N, d, mode, cb_a, cb_w, y, yt, &p));
    if (workspace != nullptr && reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
        return fail(RTQ_ERR_MISALIGNED, "workspace is not 16-byte aligned");
    if (T == 0) return ok();
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.lut) return hip_status(rtq::launch_gemm_lut(p.cb, s), "gemm_lut launch");
    p.i8.workspace = workspace;
    p.i8.ws_bytes = workspace != nullptr ? ws_bytes : 0;
    return hip_status(rtq::launch_gemm_i8(p.i8, s), "gemm_i8 launch");
}

size_t rtq_qgemm_workspace(void) { return rtq::gemm_i8_workspace_bytes(); }

size_t rtq_rotated_qlinear_workspace(int64_t T, int32_t d, rtq_qmode mode, int32_t bits_a) {
    return workspace_bytes(T, d, mode, bits_a);
}

rtq_status rtq_rotated_qlinear(const void* x, rtq_dtype xt, int64_t T, const rtq_rpbh* R, const void* w_codes,
                               const void* w_scale, rtq_dtype w_scale_t, int64_t N, rtq_qmode mode,
                               const rtq_codebook* cb_a, const rtq_codebook* cb_w, void* y, rtq_dtype yt,
                               void* workspace, size_t ws_bytes, void* stream) {
    return rotated_qlinear_ws(x, xt, T, R, w_codes, w_scale, w_scale_t, N, mode, cb_a, cb_w, y, yt, workspace,
                              ws_bytes, stream);
}

rtq_status rtq_rotated_qlinear_noalloc(const void* x, rtq_dtype xt, int64_t T, const rtq_rpbh* R, const void* w_codes,
                                       const void* w_scale, rtq_dtype w_scale_t, int64_t N, rtq_qmode mode,
                                       const rtq_codebook* cb_a, const rtq_codebook* cb_w, void* y, rtq_dtype yt,
                                       void* stream) {
    size_t need = 0;
    RTQ_TRY(qlinear_need(R, T, mode, cb_a, &need));
    if (need > kScratchBytes)
        return fail(RTQ_ERR_INVALID_ARG,
                    "rtq_rotated_qlinear_noalloc: the activation codes and scales need %zu bytes, more than its "
                    "static scratch of %zu bytes (use rtq_rotated_qlinear with a workspace)", need, kScratchBytes);
    void* ws = nullptr;
    RTQ_TRY(scratch_address(&ws));
    return rotated_qlinear_ws(x, xt, T, R, w_codes, w_scale, w_scale_t, N, mode, cb_a, cb_w, y, yt, ws, need,
                              stream);
}

// ---- asymmetric INT8 (scale + zero point per row)

rtq_status rtq_quantize_rows_asym(const void* x, rtq_dtype xt, int64_t rows, int32_t d, const rtq_rpbh* R,
                                  int8_t* codes, void* scale, rtq_dtype scale_t, int32_t* zero, int32_t* code_sum,
                                  void* stream) {
    rtq::RowArgs a{};
    RTQ_TRY(plan_quantize(x, xt, rows, d, R, RTQ_INT8, nullptr, 0.0f, codes, scale, scale_t, &a));
    if (R == nullptr || xt != RTQ_BF16)
        return fail(RTQ_ERR_UNSUPPORTED, "asymmetric INT8 needs BF16 rows and a rotation descriptor");
    if (zero == nullptr || code_sum == nullptr) return fail(RTQ_ERR_INVALID_ARG, "zero or code_sum is NULL");
    if (reinterpret_cast<uintptr_t>(zero) % 4 != 0 || reinterpret_cast<uintptr_t>(code_sum) % 4 != 0)
        return fail(RTQ_ERR_MISALIGNED, "zero or code_sum is not 4-byte aligned");
    a.out_kind = rtq::kRowInt8Asym;
    a.zero = zero;
    a.sum = code_sum;
    if (rows == 0) return ok();
    return hip_status(rtq::launch_rpbh_rows(a, static_cast<hipStream_t>(stream)), "rpbh_rows launch");
}


rtq_status rtq_qgemm_asym(const int8_t* a_codes, const float* a_scale, const int32_t* a_zero, const int32_t* a_sum,
                          int64_t T, const int8_t* w_codes, const void* w_scale, rtq_dtype w_scale_t,
                          const int32_t* w_zero, const int32_t* w_sum, int64_t N, int32_t d, void* y, rtq_dtype yt,
                          void* workspace, size_t ws_bytes, void* stream) {
    GemmPlan p{};
    RTQ_TRY(plan_gemm_asym(a_codes, a_scale, a_zero, a_sum, T, w_codes, w_scale, w_scale_t, w_zero, w_sum, N, d, y, yt,
                           &p));
    if (workspace != nullptr && reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
        return fail(RTQ_ERR_MISALIGNED, "workspace is not 16-byte aligned");
    if (T == 0) return ok();
    p.i8.workspace = workspace;
    p.i8.ws_bytes = workspace != nullptr ? ws_bytes : 0;
    return hip_status(rtq::launch_gemm_i8(p.i8, static_cast<hipStream_t>(stream)), "gemm_i8 launch");
}

size_t rtq_rotated_qlinear_asym_workspace(int64_t T, int32_t d) { return asym_workspace_bytes(T, d, true); }

rtq_status rtq_rotated_qlinear_asym(const void* x, rtq_dtype xt, int64_t T, const rtq_rpbh* R, const int8_t* w_codes,
                                    const void* w_scale, rtq_dtype w_scale_t, const int32_t* w_zero,
                                    const int32_t* w_sum, int64_t N, void* y, rtq_dtype yt, void* workspace,
                                    size_t ws_bytes, void* stream) {
    if (R == nullptr) return fail(RTQ_ERR_INVALID_ARG, "rpbh descriptor is NULL");
    const int32_t d = R->d;
    RTQ_TRY(check_d(d));
    if (yt == RTQ_I32) return fail(RTQ_ERR_UNSUPPORTED, "rtq_rotated_qlinear_asym produces F32 or BF16 output");
    const size_t need = asym_workspace_bytes(T < 0 ? 0 : T, d, false);
    if (workspace == nullptr) return fail(RTQ_ERR_INVALID_ARG, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return fail(RTQ_ERR_MISALIGNED, "workspace is not 16-byte aligned");
    if (ws_bytes < need) return fail(RTQ_ERR_INVALID_ARG, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    const size_t rows = static_cast<size_t>(T < 0 ? 0 : T);
    int8_t* a_codes = reinterpret_cast<int8_t*>(ws);
    size_t off = align256(rows * static_cast<size_t>(d));
    float* a_scale = reinterpret_cast<float*>(ws + off);
    off += align256(rows * 4);
    int32_t* a_zero = reinterpret_cast<int32_t*>(ws + off);
    off += align256(rows * 4);
    int32_t* a_sum = reinterpret_cast<int32_t*>(ws + off);
    off += align256(rows * 4);
    rtq::RowArgs qa{};
    RTQ_TRY(plan_quantize(x, xt, T, d, R, RTQ_INT8, nullptr, 0.0f, a_codes, a_scale, RTQ_F32, &qa));
    if (xt != RTQ_BF16) return fail(RTQ_ERR_UNSUPPORTED, "asymmetric INT8 needs BF16 rows");
    qa.out_kind = rtq::kRowInt8Asym;
    qa.zero = a_zero;
    qa.sum = a_sum;
    GemmPlan gp{};
    RTQ_TRY(plan_gemm_asym(a_codes, a_scale, a_zero, a_sum, T, w_codes, w_scale, w_scale_t, w_zero, w_sum, N, d, y, yt,
                           &gp));
    if (T == 0) return ok();
    hipStream_t s = static_cast<hipStream_t>(stream);
    gp.i8.workspace = ws + off;
    gp.i8.ws_bytes = ws_bytes - off;
    qa.clear = rtq::gemm_i8_split_counters(gp.i8.workspace, gp.i8.ws_bytes, &qa.nclear);
    RTQ_TRY(hip_status(rtq::launch_rpbh_rows(qa, s), "rpbh_rows launch"));
    return hip_status(rtq::launch_gemm_i8(gp.i8, s), "gemm_i8 launch");
}

const char* rtq_last_error(void) { return g_err.c_str(); }

}  // extern "C"
