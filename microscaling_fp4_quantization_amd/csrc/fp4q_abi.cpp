// fp4q_abi.cpp -- the extern "C" entry points declared in include/fp4q.h.
//
// Every entry point validates its arguments completely before anything is
// launched, so an error status means nothing was enqueued and no output was
// touched.  Launching is delegated to fp4q_kernels.hip.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/fp4q.h"
#include "fp4q_launch.h"

namespace {

thread_local char g_err[512];

fp4q_status fail(fp4q_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

fp4q_status ok() {
    g_err[0] = '\0';
    return FP4Q_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_block(int32_t b) { return b == 8 || b == 16 || b == 32 || b == 64 || b == 128 || b == 256; }

// Shape rules shared by all calls.
fp4q_status check_shape(const char* fn, int64_t rows, int64_t cols, int32_t block, int32_t rotate) {
    if (rows < 0 || cols < 0) return fail(FP4Q_ERR_SHAPE, "%s: negative size %lld x %lld", fn, (long long)rows, (long long)cols);
    if (rows > 0 && cols > INT64_MAX / rows) return fail(FP4Q_ERR_SHAPE, "%s: rows * cols overflows", fn);
    // The streaming kernels index 512-element chunks with 32-bit integers.
    if (rows * cols > (int64_t)INT32_MAX * 512)
        return fail(FP4Q_ERR_SHAPE, "%s: %lld elements exceed the limit of (2^31 - 1) * 512", fn,
                    (long long)(rows * cols));
    if (!valid_block(block)) return fail(FP4Q_ERR_SHAPE, "%s: block %d is not one of 8, 16, 32, 64, 128, 256", fn, block);
    if (cols % block != 0) return fail(FP4Q_ERR_SHAPE, "%s: cols %lld is not a multiple of the block %d", fn, (long long)cols, block);
    if (rotate != 0) {
        if (rotate != 16 && rotate != 32) return fail(FP4Q_ERR_SHAPE, "%s: rotate %d is not 0, 16 or 32", fn, rotate);
        if (rotate != block) return fail(FP4Q_ERR_SHAPE, "%s: rotate %d must equal the block %d", fn, rotate, block);
    }
    return FP4Q_OK;
}

fp4q_status check_dtype(const char* fn, int32_t t) {
    if (t != FP4Q_BF16 && t != FP4Q_F32) return fail(FP4Q_ERR_ARG, "%s: dtype %d is not BF16 (0) or F32 (1)", fn, t);
    return FP4Q_OK;
}

fp4q_status check_mse(const char* fn, const float* block_mse, int32_t kind) {
    if (kind != FP4Q_MSE_ABS && kind != FP4Q_MSE_REL) return fail(FP4Q_ERR_ARG, "%s: mse_kind %d is not ABS (0) or REL (1)", fn, kind);
    if (block_mse && !aligned(block_mse, 4)) return fail(FP4Q_ERR_ALIGN, "%s: block_mse is not 4-byte aligned", fn);
    return FP4Q_OK;
}

fp4q_status check_ws(const char* fn, bool needed, void* ws, size_t ws_bytes) {
    if (!needed) return FP4Q_OK;
    if (!ws) return fail(FP4Q_ERR_WORKSPACE, "%s: a workspace is needed (stats or dynamic scale) but ws is NULL", fn);
    if (!aligned(ws, 256)) return fail(FP4Q_ERR_ALIGN, "%s: ws is not 256-byte aligned", fn);
    if (ws_bytes < fp4q::kWsBytes) return fail(FP4Q_ERR_WORKSPACE, "%s: ws has %zu bytes, needs %zu", fn, ws_bytes, fp4q::kWsBytes);
    return FP4Q_OK;
}

fp4q_status launched(int rc, const char* msg) {
    if (rc) return fail(FP4Q_ERR_HIP, "%s", msg);
    return ok();
}

#define TRY(expr)                          \
    do {                                   \
        fp4q_status st_ = (expr);          \
        if (st_ != FP4Q_OK) return st_;    \
    } while (0)

// Validates one quantize call's arguments and fills its job.
fp4q_status quant_job(const char* fn, const void* x, int32_t xt, int64_t rows, int64_t cols,
                      int32_t block, int32_t fmt, int32_t gmode, float* g, int32_t rotate,
                      uint8_t* codes, uint8_t* scales, float* block_mse, int32_t mse_kind,
                      fp4q_stats* stats, void* ws, size_t ws_bytes, void* stream, int32_t radius,
                      bool scratch, fp4q::QuantJob& j) {
    TRY(check_dtype(fn, xt));
    TRY(check_shape(fn, rows, cols, block, rotate));
    TRY(check_mse(fn, block_mse, mse_kind));
    if (gmode != FP4Q_G_NONE && gmode != FP4Q_G_DYNAMIC && gmode != FP4Q_G_GIVEN && gmode != FP4Q_G_ROW)
        return fail(FP4Q_ERR_ARG, "%s: gmode %d is not NONE (0), DYNAMIC (1), GIVEN (2) or ROW (3)", fn, gmode);
    if (fmt == FP4Q_FMT_UE5M3 && gmode != FP4Q_G_NONE)
        return fail(FP4Q_ERR_ARG, "%s: UE5M3 scales take no per-tensor scale (gmode must be NONE)", fn);
    if (gmode == FP4Q_G_ROW && radius >= 0)
        return fail(FP4Q_ERR_ARG, "%s: the scale search does not take per-row scales", fn);
    if (gmode != FP4Q_G_NONE && !g && !(gmode == FP4Q_G_ROW && rows == 0))
        return fail(FP4Q_ERR_ARG, "%s: gmode %d needs a g pointer", fn, gmode);
    if (g && !aligned(g, 4)) return fail(FP4Q_ERR_ALIGN, "%s: g is not 4-byte aligned", fn);
    const int64_t n = rows * cols;
    if (n > 0) {
        if (!x || !codes || !scales) return fail(FP4Q_ERR_ARG, "%s: x, codes and scales must not be NULL", fn);
        if (!aligned(x, 16)) return fail(FP4Q_ERR_ALIGN, "%s: x is not 16-byte aligned", fn);
        if (!aligned(codes, 16)) return fail(FP4Q_ERR_ALIGN, "%s: codes is not 16-byte aligned", fn);
    }
    if (stats && !aligned(stats, 8)) return fail(FP4Q_ERR_ALIGN, "%s: stats is not 8-byte aligned", fn);
    const bool need_ws = stats != nullptr || gmode == FP4Q_G_DYNAMIC;
    if (scratch && need_ws) {  // the library's static scratch instead of a caller's workspace
        char msg[256] = {0};
        if (fp4q::scratch_workspace(&ws, &ws_bytes, msg, sizeof msg))
            return fail(FP4Q_ERR_HIP, "%s: %s", fn, msg);
    }
    TRY(check_ws(fn, need_ws, ws, ws_bytes));
    j = fp4q::QuantJob{};
    j.x = x;
    j.xt = xt;
    j.n = n;
    j.rows = rows;
    j.cols = cols;
    j.block = block;
    j.fmt = fmt;
    j.gmode = gmode;
    j.g = g;
    j.rotate = rotate;
    j.codes = codes;
    j.scales = scales;
    j.block_mse = block_mse;
    j.mse_kind = mse_kind;
    j.stats = stats;
    j.ws = ws;
    j.stream = stream;
    j.radius = radius;
    return FP4Q_OK;
}

fp4q_status quantize_common(const char* fn, const void* x, int32_t xt, int64_t rows, int64_t cols,
                            int32_t block, int32_t fmt, int32_t gmode, float* g, int32_t rotate,
                            uint8_t* codes, uint8_t* scales, float* block_mse, int32_t mse_kind,
                            fp4q_stats* stats, void* ws, size_t ws_bytes, void* stream,
                            int32_t radius = -1, bool scratch = false) {
    fp4q::QuantJob j;
    TRY(quant_job(fn, x, xt, rows, cols, block, fmt, gmode, g, rotate, codes, scales, block_mse,
                  mse_kind, stats, ws, ws_bytes, stream, radius, scratch, j));
    char msg[256] = {0};
    return launched(fp4q::launch_quantize(j, msg, sizeof msg), msg);
}

fp4q_status check_fmt_block(const char* fn, int32_t fmt, int32_t block) {
    if (fmt != FP4Q_FMT_MXFP4 && fmt != FP4Q_FMT_UE4M3 && fmt != FP4Q_FMT_UE5M3)
        return fail(FP4Q_ERR_ARG, "%s: fmt %d is not MXFP4 (0), UE4M3 (1) or UE5M3 (2)", fn, fmt);
    if (fmt == FP4Q_FMT_MXFP4 && block != 32) return fail(FP4Q_ERR_SHAPE, "%s: MXFP4 blocks are 32, not %d", fn, block);
    return FP4Q_OK;
}

}  // namespace

extern "C" {

fp4q_status mxfp4_quantize(const void* x, int32_t xt, int64_t rows, int64_t cols, int32_t rotate,
                           uint8_t* codes, uint8_t* scales, float* block_mse, int32_t mse_kind,
                           fp4q_stats* stats, void* ws, size_t ws_bytes, void* stream) {
    if (rotate != 0 && rotate != 32) return fail(FP4Q_ERR_SHAPE, "mxfp4_quantize: rotate %d is not 0 or 32", rotate);
    return quantize_common("mxfp4_quantize", x, xt, rows, cols, 32, FP4Q_FMT_MXFP4, FP4Q_G_NONE, nullptr,
                           rotate, codes, scales, block_mse, mse_kind, stats, ws, ws_bytes, stream);
}

fp4q_status nvfp4_quantize(const void* x, int32_t xt, int64_t rows, int64_t cols, int32_t block,
                           int32_t scale_fmt, int32_t gmode, float* g, int32_t rotate,
                           uint8_t* codes, uint8_t* scales, float* block_mse, int32_t mse_kind,
                           fp4q_stats* stats, void* ws, size_t ws_bytes, void* stream) {
    if (scale_fmt != FP4Q_FMT_UE4M3 && scale_fmt != FP4Q_FMT_UE5M3)
        return fail(FP4Q_ERR_ARG, "nvfp4_quantize: scale_fmt %d is not UE4M3 (1) or UE5M3 (2)", scale_fmt);
    return quantize_common("nvfp4_quantize", x, xt, rows, cols, block, scale_fmt, gmode, g, rotate,
                           codes, scales, block_mse, mse_kind, stats, ws, ws_bytes, stream);
}

fp4q_status nvfp4_quantize_noalloc(const void* x, int32_t xt, int64_t rows, int64_t cols,
                                   int32_t block, int32_t scale_fmt, int32_t gmode, float* g,
                                   int32_t rotate, uint8_t* codes, uint8_t* scales, float* block_mse,
                                   int32_t mse_kind, fp4q_stats* stats, void* stream) {
    if (scale_fmt != FP4Q_FMT_UE4M3 && scale_fmt != FP4Q_FMT_UE5M3)
        return fail(FP4Q_ERR_ARG, "nvfp4_quantize_noalloc: scale_fmt %d is not UE4M3 (1) or UE5M3 (2)",
                    scale_fmt);
    return quantize_common("nvfp4_quantize_noalloc", x, xt, rows, cols, block, scale_fmt, gmode, g,
                           rotate, codes, scales, block_mse, mse_kind, stats, nullptr, 0, stream, -1,
                           true);
}

fp4q_status fp4_quantize_mx_nv(const void* x, int32_t xt, int64_t rows, int64_t cols,
                               uint8_t* mx_codes, uint8_t* mx_scales, float* mx_block_mse,
                               fp4q_stats* mx_stats, int32_t nv_block, float* g, uint8_t* nv_codes,
                               uint8_t* nv_scales, float* nv_block_mse, fp4q_stats* nv_stats,
                               int32_t mse_kind, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "fp4_quantize_mx_nv";
    fp4q::QuantJob mx, nv;
    TRY(quant_job(fn, x, xt, rows, cols, 32, FP4Q_FMT_MXFP4, FP4Q_G_NONE, nullptr, 0, mx_codes,
                  mx_scales, mx_block_mse, mse_kind, mx_stats, ws, ws_bytes, stream, -1, false, mx));
    TRY(quant_job(fn, x, xt, rows, cols, nv_block, FP4Q_FMT_UE4M3, FP4Q_G_DYNAMIC, g, 0, nv_codes,
                  nv_scales, nv_block_mse, mse_kind, nv_stats, ws, ws_bytes, stream, -1, false, nv));
    char msg[256] = {0};
    return launched(fp4q::launch_quantize_mx_nv(mx, nv, msg, sizeof msg), msg);
}

fp4q_status fp4_quantize_mx_nv_batch(const fp4q_mx_nv_tensor* tensors, int32_t n_tensors,
                                     int32_t xt, int32_t nv_block, int32_t mse_kind, void* ws,
                                     size_t ws_bytes, void* stream) {
    static_assert(FP4Q_MAX_BATCH == fp4q::kMaxBatchTensors, "batch limit");
    const char* fn = "fp4_quantize_mx_nv_batch";
    if (n_tensors < 1 || n_tensors > FP4Q_MAX_BATCH)
        return fail(FP4Q_ERR_ARG, "%s: n_tensors %d is not in 1..%d", fn, n_tensors, FP4Q_MAX_BATCH);
    if (!tensors) return fail(FP4Q_ERR_ARG, "%s: tensors is NULL", fn);
    if (nv_block != 16 && nv_block != 32)
        return fail(FP4Q_ERR_SHAPE, "%s: nv_block %d is not 16 or 32", fn, nv_block);
    fp4q::QuantJob mx[FP4Q_MAX_BATCH], nv[FP4Q_MAX_BATCH];
    char where[96];
    // Outputs wanted: as the first non-empty tensor gives them (an empty
    // tensor's zero-size outputs may be NULL).
    int ref = 0;
    while (ref + 1 < n_tensors && tensors[ref].rows * tensors[ref].cols == 0) ++ref;
    for (int i = 0; i < n_tensors; ++i) {
        const fp4q_mx_nv_tensor& t = tensors[i];
        snprintf(where, sizeof where, "%s tensor %d", fn, i);
        TRY(quant_job(where, t.x, xt, t.rows, t.cols, 32, FP4Q_FMT_MXFP4, FP4Q_G_NONE, nullptr, 0,
                      t.mx_codes, t.mx_scales, t.mx_block_mse, mse_kind, t.mx_stats, ws, ws_bytes,
                      stream, -1, false, mx[i]));
        TRY(quant_job(where, t.x, xt, t.rows, t.cols, nv_block, FP4Q_FMT_UE4M3, FP4Q_G_DYNAMIC, t.g,
                      0, t.nv_codes, t.nv_scales, t.nv_block_mse, mse_kind, t.nv_stats, ws, ws_bytes,
                      stream, -1, false, nv[i]));
        const fp4q_mx_nv_tensor& r = tensors[ref];
        const bool empty = t.rows * t.cols == 0;
        if ((!empty && ((t.mx_block_mse == nullptr) != (r.mx_block_mse == nullptr) ||
                        (t.nv_block_mse == nullptr) != (r.nv_block_mse == nullptr))) ||
            (t.mx_stats == nullptr) != (r.mx_stats == nullptr) ||
            (t.nv_stats == nullptr) != (r.nv_stats == nullptr))
            return fail(FP4Q_ERR_ARG, "%s: block_mse and stats must be given for every tensor or for none",
                        where);
    }
    char msg[256] = {0};
    return launched(fp4q::launch_quantize_mx_nv_batch(mx, nv, n_tensors, msg, sizeof msg), msg);
}

fp4q_status fp4_quantize_search(const void* x, int32_t xt, int64_t rows, int64_t cols, int32_t fmt,
                                int32_t block, int32_t gmode, float* g, int32_t rotate,
                                int32_t radius, uint8_t* codes, uint8_t* scales, float* block_mse,
                                int32_t mse_kind, fp4q_stats* stats, void* ws, size_t ws_bytes,
                                void* stream) {
    const char* fn = "fp4_quantize_search";
    TRY(check_fmt_block(fn, fmt, block));
    if (fmt == FP4Q_FMT_MXFP4 && gmode != FP4Q_G_NONE)
        return fail(FP4Q_ERR_ARG, "%s: MXFP4 takes no per-tensor scale (gmode must be NONE)", fn);
    if (radius < 0 || radius > FP4Q_SEARCH_MAX_RADIUS)
        return fail(FP4Q_ERR_ARG, "%s: radius %d is not in [0, %d]", fn, radius, FP4Q_SEARCH_MAX_RADIUS);
    return quantize_common(fn, x, xt, rows, cols, block, fmt, gmode, g, rotate, codes, scales,
                           block_mse, mse_kind, stats, ws, ws_bytes, stream, radius);
}

fp4q_status fp4_dequantize(const uint8_t* codes, const uint8_t* scales, int32_t fmt, int32_t block,
                           const float* g, int64_t rows, int64_t cols, int32_t rotate, void* out,
                           int32_t ot, void* stream) {
    const char* fn = "fp4_dequantize";
    TRY(check_fmt_block(fn, fmt, block));
    TRY(check_shape(fn, rows, cols, block, rotate));
    TRY(check_dtype(fn, ot));
    if (g && !aligned(g, 4)) return fail(FP4Q_ERR_ALIGN, "%s: g is not 4-byte aligned", fn);
    const int64_t n = rows * cols;
    if (n > 0) {
        if (!codes || !scales || !out) return fail(FP4Q_ERR_ARG, "%s: codes, scales and out must not be NULL", fn);
        if (!aligned(codes, 4)) return fail(FP4Q_ERR_ALIGN, "%s: codes is not 4-byte aligned", fn);
        if (!aligned(out, 16)) return fail(FP4Q_ERR_ALIGN, "%s: out is not 16-byte aligned", fn);
    }
    fp4q::DequantJob j{codes, scales, fmt, block, fmt == FP4Q_FMT_UE4M3 ? g : nullptr, n, rotate, out, ot, stream};
    char msg[256] = {0};
    return launched(fp4q::launch_dequantize(j, msg, sizeof msg), msg);
}

fp4q_status fp4_block_mse(const void* x, int32_t xt, const uint8_t* codes, const uint8_t* scales,
                          int32_t fmt, int32_t block, const float* g, int64_t rows, int64_t cols,
                          int32_t rotate, float* block_mse, int32_t mse_kind, fp4q_stats* stats,
                          void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "fp4_block_mse";
    TRY(check_fmt_block(fn, fmt, block));
    TRY(check_dtype(fn, xt));
    TRY(check_shape(fn, rows, cols, block, rotate));
    TRY(check_mse(fn, block_mse, mse_kind));
    if (g && !aligned(g, 4)) return fail(FP4Q_ERR_ALIGN, "%s: g is not 4-byte aligned", fn);
    const int64_t n = rows * cols;
    if (n > 0) {
        if (!x || !codes || !scales) return fail(FP4Q_ERR_ARG, "%s: x, codes and scales must not be NULL", fn);
        if (!aligned(x, 16)) return fail(FP4Q_ERR_ALIGN, "%s: x is not 16-byte aligned", fn);
        if (!aligned(codes, 4)) return fail(FP4Q_ERR_ALIGN, "%s: codes is not 4-byte aligned", fn);
    }
    if (stats && !aligned(stats, 8)) return fail(FP4Q_ERR_ALIGN, "%s: stats is not 8-byte aligned", fn);
    TRY(check_ws(fn, stats != nullptr, ws, ws_bytes));
    fp4q::MseJob j{x, xt, codes, scales, fmt, block, fmt == FP4Q_FMT_UE4M3 ? g : nullptr, n, rotate,
                   block_mse, mse_kind, stats, ws, stream};
    char msg[256] = {0};
    return launched(fp4q::launch_block_mse(j, msg, sizeof msg), msg);
}

fp4q_status fp4_gemm_mxfp4(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                           const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* c,
                           int32_t ct, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "fp4_gemm_mxfp4";
    TRY(check_dtype(fn, ct));
    if (M < 0 || N < 0 || K < 0) return fail(FP4Q_ERR_SHAPE, "%s: negative size", fn);
    if (K % 32 != 0) return fail(FP4Q_ERR_SHAPE, "%s: K = %lld is not a multiple of 32", fn, (long long)K);
    if (K > (int64_t)1 << 23) return fail(FP4Q_ERR_SHAPE, "%s: K = %lld exceeds 2^23", fn, (long long)K);
    const int64_t eb = ct == FP4Q_F32 ? 4 : 2;
    if (N * eb >= (int64_t)1 << 23)
        return fail(FP4Q_ERR_SHAPE, "%s: N = %lld is too large for this output type", fn, (long long)N);
    if (M >= (int64_t)1 << 31) return fail(FP4Q_ERR_SHAPE, "%s: M = %lld exceeds 2^31", fn, (long long)M);
    if (M > 0 && N > 0) {
        if (!c) return fail(FP4Q_ERR_ARG, "%s: c must not be NULL", fn);
        if (!aligned(c, (size_t)eb)) return fail(FP4Q_ERR_ALIGN, "%s: c is not aligned to its element", fn);
        if (K > 0) {
            if (!a_codes || !a_scales || !b_codes || !b_scales)
                return fail(FP4Q_ERR_ARG, "%s: codes and scales must not be NULL", fn);
            if (!aligned(a_codes, 16) || !aligned(b_codes, 16))
                return fail(FP4Q_ERR_ALIGN, "%s: codes must be 16-byte aligned", fn);
            const size_t need = fp4q::gemm_workspace_bytes(M, N, K);
            if (!ws || ws_bytes < need)
                return fail(FP4Q_ERR_WORKSPACE, "%s: needs a workspace of %zu bytes (got %zu)", fn, need,
                            ws ? ws_bytes : (size_t)0);
            if (!aligned(ws, 16)) return fail(FP4Q_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
        }
    }
    fp4q::GemmJob j{a_codes, a_scales, b_codes, b_scales, M, N, K, c, ct, ws, stream};
    char msg[256] = {0};
    return launched(fp4q::launch_gemm(j, msg, sizeof msg), msg);
}

size_t fp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    return fp4q::gemm_workspace_bytes(M, N, K);
}

fp4q_status fp4_gemm_nvfp4(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_g,
                           const uint8_t* b_codes, const uint8_t* b_scales, const float* b_g, int64_t M,
                           int64_t N, int64_t K, void* c, int32_t ct, void* ws, size_t ws_bytes,
                           void* stream) {
    const char* fn = "fp4_gemm_nvfp4";
    TRY(check_dtype(fn, ct));
    if (M < 0 || N < 0 || K < 0) return fail(FP4Q_ERR_SHAPE, "%s: negative size", fn);
    if (K % 64 != 0) return fail(FP4Q_ERR_SHAPE, "%s: K = %lld is not a multiple of 64", fn, (long long)K);
    if (K > (int64_t)1 << 23) return fail(FP4Q_ERR_SHAPE, "%s: K = %lld exceeds 2^23", fn, (long long)K);
    const int64_t eb = ct == FP4Q_F32 ? 4 : 2;
    if (N * eb >= (int64_t)1 << 23)
        return fail(FP4Q_ERR_SHAPE, "%s: N = %lld is too large for this output type", fn, (long long)N);
    if (M >= (int64_t)1 << 31) return fail(FP4Q_ERR_SHAPE, "%s: M = %lld exceeds 2^31", fn, (long long)M);
    if (M > 0 && N > 0) {
        if (!c) return fail(FP4Q_ERR_ARG, "%s: c must not be NULL", fn);
        if (!aligned(c, (size_t)eb)) return fail(FP4Q_ERR_ALIGN, "%s: c is not aligned to its element", fn);
        if (K > 0) {
            if (!a_codes || !a_scales || !b_codes || !b_scales)
                return fail(FP4Q_ERR_ARG, "%s: codes and scales must not be NULL", fn);
            if (!aligned(a_codes, 16) || !aligned(b_codes, 16))
                return fail(FP4Q_ERR_ALIGN, "%s: codes must be 16-byte aligned", fn);
            if (!aligned(a_scales, 4) || !aligned(b_scales, 4))
                return fail(FP4Q_ERR_ALIGN, "%s: scales must be 4-byte aligned", fn);
            if ((a_g && !aligned(a_g, 4)) || (b_g && !aligned(b_g, 4)))
                return fail(FP4Q_ERR_ALIGN, "%s: per-tensor scales must be 4-byte aligned", fn);
            const size_t need = fp4q::gemm_nvfp4_workspace_bytes(M, N, K);
            if (need > 0 && (!ws || ws_bytes < need))
                return fail(FP4Q_ERR_WORKSPACE, "%s: needs a workspace of %zu bytes (got %zu)", fn, need,
                            ws ? ws_bytes : (size_t)0);
            if (need > 0 && !aligned(ws, 16))
                return fail(FP4Q_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
        }
    }
    fp4q::GemmNvJob j{a_codes, a_scales, b_codes, b_scales, a_g, b_g, M, N, K, c, ct, ws, stream};
    char msg[256] = {0};
    return launched(fp4q::launch_gemm_nvfp4(j, msg, sizeof msg), msg);
}

size_t fp4_gemm_nvfp4_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    return fp4q::gemm_nvfp4_workspace_bytes(M, N, K);
}

fp4q_status hadamard_block_rotate(const void* x, int32_t xt, int64_t rows, int64_t cols, int32_t n_rot,
                                  float* out, void* stream) {
    const char* fn = "hadamard_block_rotate";
    TRY(check_dtype(fn, xt));
    if (n_rot != 16 && n_rot != 32) return fail(FP4Q_ERR_SHAPE, "%s: n %d is not 16 or 32", fn, n_rot);
    TRY(check_shape(fn, rows, cols, n_rot, n_rot));
    const int64_t n = rows * cols;
    if (n > 0) {
        if (!x || !out) return fail(FP4Q_ERR_ARG, "%s: x and out must not be NULL", fn);
        if (!aligned(x, 16) || !aligned(out, 16)) return fail(FP4Q_ERR_ALIGN, "%s: x and out must be 16-byte aligned", fn);
    }
    fp4q::RotateJob j{x, xt, n, n_rot, out, stream};
    char msg[256] = {0};
    return launched(fp4q::launch_rotate(j, msg, sizeof msg), msg);
}

size_t fp4q_workspace_bytes(int64_t rows, int64_t cols, int32_t block) {
    (void)rows;
    (void)cols;
    (void)block;
    return fp4q::kWsBytes;
}

const char* fp4q_last_error(void) { return g_err; }

int32_t fp4q_abi_version(void) { return FP4Q_ABI_VERSION; }

fp4q_status fp4q_profile_events(void* const* events, int32_t n_pairs) {
    if (n_pairs < 0) return fail(FP4Q_ERR_ARG, "fp4q_profile_events: n_pairs %d is negative", n_pairs);
    fp4q::profile_set(events, events ? n_pairs : 0);
    return ok();
}

int32_t fp4q_profile_count(void) { return fp4q::profile_count(); }

}  // extern "C"
