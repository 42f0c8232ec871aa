// C ABI of the FP8 linear layer: argument validation, the weight cache and
// the composition of quantize + GEMM launches for the forward and backward
// passes.  Every check runs before anything is enqueued.
//
// Data flow ("Native FP8 MLP reconstruction", implementation paragraph):
//   forward   X -> E4M3 (row + col layouts), W -> E4M3 (row + col) unless
//             cached, Y = GEMM(Xq_row, Wq_row)
//   backward  dY -> E5M2 (row + col) with its own amax,
//             dX = GEMM(dYq_row, Wq_col), dW = GEMM(dYq_col, Xq_col)
// Weight cache (TransformerEngine issue 2852, opening post): the flag is
// True on the first microbatch of an accumulation cycle, False on the rest
// and None outside training.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "../../include/fp8_linear.h"
#include "internal.hpp"

struct fp8_wcache_s {
    int64_t M, K;
    int recipe;
    fp8_qtensor bufs;
    int valid;
    int64_t fills;
};

namespace {

thread_local std::string g_last_error;

fp8_status fail(fp8_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
fp8_status fail(fp8_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool dim_ok(int64_t d) { return d > 0 && (d % 128) == 0 && d <= (int64_t(1) << 31); }

constexpr size_t kPartialBytes = 4096;   // tensorwise amax partials (2048 x 16 bits)

fp8_status check_dims(const char* what, int64_t a, int64_t b) {
    if (!dim_ok(a) || !dim_ok(b))
        return fail(FP8_ERR_SHAPE, "%s: dimensions %lld x %lld must be positive multiples of 128", what,
                    (long long)a, (long long)b);
    return FP8_OK;
}

fp8_status check_ptr16(const char* what, const void* p) {
    if (!p) return fail(FP8_ERR_NULL, "%s is NULL", what);
    if (!aligned16(p)) return fail(FP8_ERR_ALIGN, "%s is not 16-byte aligned", what);
    return FP8_OK;
}

fp8_status check_ptr4(const char* what, const void* p) {
    if (!p) return fail(FP8_ERR_NULL, "%s is NULL", what);
    if (!aligned4(p)) return fail(FP8_ERR_ALIGN, "%s is not 4-byte aligned", what);
    return FP8_OK;
}

#define FP8_TRY(expr)                    \
    do {                                 \
        fp8_status _s = (expr);          \
        if (_s != FP8_OK) return _s;     \
    } while (0)

// Validate a quantize request (no launch).
fp8_status check_quantize(const void* x, int64_t rows, int64_t cols, int format, int scaling, unsigned layouts,
                          const fp8_qtensor* out) {
    FP8_TRY(check_dims("quantize", rows, cols));
    if (format != FP8_E4M3 && format != FP8_E5M2) return fail(FP8_ERR_ENUM, "unknown format %d", format);
    if (scaling < FP8_SCALE_TENSOR || scaling > FP8_SCALE_BLOCK_128x128)
        return fail(FP8_ERR_ENUM, "unknown scaling %d", scaling);
    if (layouts == 0 || (layouts & ~3u) != 0) return fail(FP8_ERR_ENUM, "bad layout mask %u", layouts);
    FP8_TRY(check_ptr16("x", x));
    if (!out) return fail(FP8_ERR_NULL, "output descriptor is NULL");
    if (layouts & FP8_LAYOUT_ROW) FP8_TRY(check_ptr16("q_row", out->q_row));
    if (layouts & FP8_LAYOUT_COL) FP8_TRY(check_ptr16("q_col", out->q_col));
    const bool row_scales = scaling != FP8_SCALE_BLOCK_1x128 || (layouts & FP8_LAYOUT_ROW);
    // 1x128 scales are written as 8- and 16-byte runs: 16-byte alignment
    auto check_scale = scaling == FP8_SCALE_BLOCK_1x128 ? check_ptr16 : check_ptr4;
    if (row_scales) {
        FP8_TRY(check_scale("scale", out->scale));
        FP8_TRY(check_scale("scale_inv", out->scale_inv));
    }
    if (scaling == FP8_SCALE_BLOCK_1x128 && (layouts & FP8_LAYOUT_COL)) {
        FP8_TRY(check_scale("scale_col", out->scale_col));
        FP8_TRY(check_scale("scale_inv_col", out->scale_inv_col));
    }
    if (out->amax && !aligned4(out->amax)) return fail(FP8_ERR_ALIGN, "amax is not 4-byte aligned");
    return FP8_OK;
}

fp8_status hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(FP8_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return FP8_OK;
}

// given_amax: tensorwise only, the amax partials of x from its producer (the
// amax pass is skipped); otherwise ws holds the pass's partials
// act: 0 quantize x; 1 quantize GELU(x); 2 quantize dGELU(x, x2)
static fp8k::QuantizeLaunch quantize_launch(const void* x, int64_t rows, int64_t cols, int format, int scaling,
                                            unsigned layouts, const fp8_qtensor* out, void* ws,
                                            const void* given_amax, int act, const void* x2,
                                            const void* gelu_keys = nullptr) {
    fp8k::QuantizeLaunch q;
    q.x = x;
    q.rows = rows;
    q.cols = cols;
    q.format = format;
    q.scaling = scaling;
    q.q_row = (layouts & FP8_LAYOUT_ROW) ? out->q_row : nullptr;
    q.q_col = (layouts & FP8_LAYOUT_COL) ? out->q_col : nullptr;
    q.scale = out->scale;
    q.scale_inv = out->scale_inv;
    q.scale_col = out->scale_col;
    q.scale_inv_col = out->scale_inv_col;
    q.amax = scaling == FP8_SCALE_TENSOR ? out->amax : nullptr;
    q.partial = given_amax ? static_cast<uint16_t*>(const_cast<void*>(given_amax)) : static_cast<uint16_t*>(ws);
    q.partial_given = given_amax != nullptr;
    q.hist = nullptr;
    q.hist_len = 0;
    q.act = act;
    q.x2 = x2;
    q.gelu_keys = static_cast<const uint16_t*>(gelu_keys);
    return q;
}

fp8_status do_quantize(const void* x, int64_t rows, int64_t cols, int format, int scaling, unsigned layouts,
                       const fp8_qtensor* out, void* ws, hipStream_t st, const void* given_amax = nullptr,
                       int act = 0, const void* x2 = nullptr, const void* gelu_keys = nullptr) {
    const fp8k::QuantizeLaunch q =
        quantize_launch(x, rows, cols, format, scaling, layouts, out, ws, given_amax, act, x2, gelu_keys);
    return hip_status(fp8k::launch_quantize(q, st), "quantize launch");
}

// Two tensorwise E4M3 quantizes of plain inputs, both layouts, in one amax
// launch and one cast launch (a layer's input and its weight); each tensor's
// amax partials go to its own 4 KiB buffer.
static fp8_status do_quantize_pair(const void* xa, int64_t ra, int64_t ca, const fp8_qtensor* outa, void* wsa,
                                   const void* xb, int64_t rb, int64_t cb, const fp8_qtensor* outb, void* wsb,
                                   hipStream_t st) {
    const unsigned both = FP8_LAYOUT_ROW | FP8_LAYOUT_COL;
    const fp8k::QuantizeLaunch qa = quantize_launch(xa, ra, ca, FP8_E4M3, FP8_SCALE_TENSOR, both, outa, wsa, nullptr, 0,
                                                    nullptr);
    const fp8k::QuantizeLaunch qb = quantize_launch(xb, rb, cb, FP8_E4M3, FP8_SCALE_TENSOR, both, outb, wsb, nullptr, 0,
                                                    nullptr);
    return hip_status(fp8k::launch_quantize_pair(qa, qb, st), "quantize launch");
}

fp8k::GemmScale tensor_scale(const float* sinv) { return fp8k::GemmScale{sinv, 0, 0, 0}; }
fp8k::GemmScale block_scale(const float* sinv, int64_t group, int64_t sr, int64_t sk) {
    return fp8k::GemmScale{sinv, group, sr, sk};
}

// the GEMM kernels address one 256-row operand tile with 32-bit offsets
constexpr int64_t kMaxContraction = int64_t(1) << 23;

fp8_status do_gemm(const void* a, int fa, fp8k::GemmScale sa, const void* b, int fb, fp8k::GemmScale sb, int64_t I,
                   int64_t J, int64_t K, void* c, void* ws, size_t ws_bytes, hipStream_t st,
                   void* c_amax = nullptr, void* c_gelu_keys = nullptr) {
    if (K >= kMaxContraction)
        return fail(FP8_ERR_SHAPE, "contraction length %lld: must be below 2^23", (long long)K);
    fp8k::GemmLaunch g;
    g.a = a;
    g.fa = fa;
    g.sa = sa;
    g.b = b;
    g.fb = fb;
    g.sb = sb;
    g.I = I;
    g.J = J;
    g.K = K;
    g.c = c;
    g.ws = ws;
    g.ws_bytes = ws_bytes;
    g.c_amax = static_cast<uint16_t*>(c_amax);
    g.gelu_keys = static_cast<uint16_t*>(c_gelu_keys);
    return hip_status(fp8k::launch_gemm(g, st), "gemm launch");
}

size_t linear_gemm_ws(int64_t N, int64_t K, int64_t M) {
    size_t a = fp8k::gemm_ws_bytes(N, M, K);   // fprop
    size_t b = fp8k::gemm_ws_bytes(N, K, M);   // dgrad
    size_t c = fp8k::gemm_ws_bytes(M, K, N);   // wgrad
    size_t m = a > b ? a : b;
    return m > c ? m : c;
}

fp8_status check_weight_q(const fp8_qtensor* w, int recipe, bool need_row, bool need_col) {
    if (!w) return fail(FP8_ERR_NULL, "quantized weight descriptor is NULL");
    if (need_row) FP8_TRY(check_ptr16("w_q.q_row", w->q_row));
    if (need_col) FP8_TRY(check_ptr16("w_q.q_col", w->q_col));
    FP8_TRY(check_ptr4("w_q.scale", w->scale));
    FP8_TRY(check_ptr4("w_q.scale_inv", w->scale_inv));
    (void)recipe;
    return FP8_OK;
}

}  // namespace

extern "C" {

const char* fp8_status_string(fp8_status s) {
    switch (s) {
        case FP8_OK: return "FP8_OK";
        case FP8_ERR_NULL: return "FP8_ERR_NULL";
        case FP8_ERR_SHAPE: return "FP8_ERR_SHAPE";
        case FP8_ERR_ALIGN: return "FP8_ERR_ALIGN";
        case FP8_ERR_ENUM: return "FP8_ERR_ENUM";
        case FP8_ERR_WORKSPACE: return "FP8_ERR_WORKSPACE";
        case FP8_ERR_CACHE_EMPTY: return "FP8_ERR_CACHE_EMPTY";
        case FP8_ERR_CACHE_MISMATCH: return "FP8_ERR_CACHE_MISMATCH";
        case FP8_ERR_HIP: return "FP8_ERR_HIP";
        case FP8_ERR_UNIMPLEMENTED: return "FP8_ERR_UNIMPLEMENTED";
    }
    return "FP8_ERR_UNKNOWN";
}

const char* fp8_last_error(void) { return g_last_error.c_str(); }

const char* fp8_version(void) { return "fp8linear-gfx950 0.1"; }

size_t fp8_quantize_workspace_bytes(int64_t rows, int64_t cols, fp8_scaling scaling) {
    (void)rows;
    (void)cols;
    return scaling == FP8_SCALE_TENSOR ? kPartialBytes : 0;
}

fp8_status fp8_quantize(const void* x, int64_t rows, int64_t cols, fp8_format format, fp8_scaling scaling,
                        unsigned layouts, const fp8_qtensor* out, void* ws, size_t ws_bytes, void* stream) {
    FP8_TRY(check_quantize(x, rows, cols, format, scaling, layouts, out));
    const size_t need = fp8_quantize_workspace_bytes(rows, cols, scaling);
    if (need) {
        if (ws_bytes < need) return fail(FP8_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
        FP8_TRY(check_ptr16("ws", ws));
    }
    return do_quantize(x, rows, cols, format, scaling, layouts, out, ws, static_cast<hipStream_t>(stream));
}

fp8_status fp8_quantize_from_amax(const void* x, int64_t rows, int64_t cols, fp8_format format, unsigned layouts,
                                  const fp8_qtensor* out, const void* amax_partials, void* stream) {
    FP8_TRY(check_quantize(x, rows, cols, format, FP8_SCALE_TENSOR, layouts, out));
    FP8_TRY(check_ptr16("amax_partials", amax_partials));
    return do_quantize(x, rows, cols, format, FP8_SCALE_TENSOR, layouts, out, nullptr, static_cast<hipStream_t>(stream),
                       amax_partials);
}

size_t fp8_quantize_delayed_workspace_bytes(int64_t rows, int64_t cols) {
    // one 16-bit amax per 128x128 tile, rounded up to 16 bytes
    if (!dim_ok(rows) || !dim_ok(cols)) return 0;
    const size_t tiles = (size_t)(rows / 128) * (size_t)(cols / 128);
    return (tiles * 2 + 15) & ~(size_t)15;
}

fp8_status fp8_quantize_delayed(const void* x, int64_t rows, int64_t cols, fp8_format format, unsigned layouts,
                                const fp8_qtensor* out, float* amax_history, int64_t history_len, void* ws,
                                size_t ws_bytes, void* stream) {
    FP8_TRY(check_quantize(x, rows, cols, format, FP8_SCALE_TENSOR, layouts, out));
    if (history_len < 1 || history_len > fp8k::kMaxHistory)
        return fail(FP8_ERR_SHAPE, "history_len %lld: must be 1 .. %d", (long long)history_len, fp8k::kMaxHistory);
    FP8_TRY(check_ptr4("amax_history", amax_history));
    const size_t need = fp8_quantize_delayed_workspace_bytes(rows, cols);
    if (ws_bytes < need) return fail(FP8_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    FP8_TRY(check_ptr16("ws", ws));
    fp8k::QuantizeLaunch q;
    q.x = x;
    q.rows = rows;
    q.cols = cols;
    q.format = format;
    q.scaling = 3;
    q.q_row = (layouts & FP8_LAYOUT_ROW) ? out->q_row : nullptr;
    q.q_col = (layouts & FP8_LAYOUT_COL) ? out->q_col : nullptr;
    q.scale = out->scale;
    q.scale_inv = out->scale_inv;
    q.scale_col = nullptr;
    q.scale_inv_col = nullptr;
    q.amax = out->amax;
    q.partial = static_cast<uint16_t*>(ws);
    q.partial_given = false;
    q.hist = amax_history;
    q.hist_len = (int)history_len;
    return hip_status(fp8k::launch_quantize(q, static_cast<hipStream_t>(stream)), "quantize launch");
}

fp8_status fp8_gelu(const void* x, void* y, int64_t n, void* stream) {
    if (n < 0 || n % 8 != 0) return fail(FP8_ERR_SHAPE, "gelu: n = %lld must be a multiple of 8", (long long)n);
    FP8_TRY(check_ptr16("x", x));
    FP8_TRY(check_ptr16("y", y));
    return hip_status(fp8k::launch_gelu(x, y, n, static_cast<hipStream_t>(stream)), "gelu launch");
}

fp8_status fp8_dgelu(const void* dy, const void* x, void* dx, int64_t n, void* stream) {
    if (n < 0 || n % 8 != 0) return fail(FP8_ERR_SHAPE, "dgelu: n = %lld must be a multiple of 8", (long long)n);
    FP8_TRY(check_ptr16("dy", dy));
    FP8_TRY(check_ptr16("x", x));
    FP8_TRY(check_ptr16("dx", dx));
    return hip_status(fp8k::launch_dgelu(dy, x, dx, n, static_cast<hipStream_t>(stream)), "dgelu launch");
}

// Checks shared by the GELU-fused quantizers (tensorwise or 1x128 only).
static fp8_status check_act_quantize(const void* x, int64_t rows, int64_t cols, int format, int scaling,
                                     unsigned layouts, const fp8_qtensor* out, size_t ws_bytes, void* ws) {
    if (scaling != FP8_SCALE_TENSOR && scaling != FP8_SCALE_BLOCK_1x128)
        return fail(FP8_ERR_ENUM, "the GELU-fused quantizers take tensorwise or 1x128 scaling, not %d", scaling);
    FP8_TRY(check_quantize(x, rows, cols, format, scaling, layouts, out));
    const size_t need = fp8_quantize_workspace_bytes(rows, cols, static_cast<fp8_scaling>(scaling));
    if (need) {
        if (ws_bytes < need) return fail(FP8_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
        FP8_TRY(check_ptr16("ws", ws));
    }
    return FP8_OK;
}

fp8_status fp8_quantize_gelu(const void* x, int64_t rows, int64_t cols, fp8_format format, fp8_scaling scaling,
                             unsigned layouts, const fp8_qtensor* out, void* ws, size_t ws_bytes, void* stream) {
    FP8_TRY(check_act_quantize(x, rows, cols, format, scaling, layouts, out, ws_bytes, ws));
    return do_quantize(x, rows, cols, format, scaling, layouts, out, ws, static_cast<hipStream_t>(stream), nullptr, 1);
}

fp8_status fp8_quantize_dgelu(const void* dy, const void* x, int64_t rows, int64_t cols, fp8_format format,
                              fp8_scaling scaling, unsigned layouts, const fp8_qtensor* out, void* ws,
                              size_t ws_bytes, void* stream) {
    FP8_TRY(check_act_quantize(dy, rows, cols, format, scaling, layouts, out, ws_bytes, ws));
    FP8_TRY(check_ptr16("x", x));
    return do_quantize(dy, rows, cols, format, scaling, layouts, out, ws, static_cast<hipStream_t>(stream), nullptr, 2,
                       x);
}

size_t fp8_gemm_workspace_bytes(int64_t I, int64_t J, int64_t K) { return fp8k::gemm_ws_bytes(I, J, K); }

static fp8_status gemm_checked(const void* a, fp8_format fa, fp8_gemm_scale sa, const void* b, fp8_format fb,
                               fp8_gemm_scale sb, int64_t I, int64_t J, int64_t K, void* c, void* ws, size_t ws_bytes,
                               void* stream, void* c_amax, void* c_gelu_keys = nullptr) {
    FP8_TRY(check_dims("gemm I x J", I, J));
    FP8_TRY(check_dims("gemm K", K, 128));
    if (K >= kMaxContraction) return fail(FP8_ERR_SHAPE, "contraction length %lld: must be below 2^23", (long long)K);
    if ((fa != FP8_E4M3 && fa != FP8_E5M2) || (fb != FP8_E4M3 && fb != FP8_E5M2))
        return fail(FP8_ERR_ENUM, "unknown operand format");
    FP8_TRY(check_ptr16("a", a));
    FP8_TRY(check_ptr16("b", b));
    FP8_TRY(check_ptr16("c", c));
    FP8_TRY(check_ptr4("scale_a", sa.scale_inv));
    FP8_TRY(check_ptr4("scale_b", sb.scale_inv));
    if ((sa.group == 0) != (sb.group == 0))
        return fail(FP8_ERR_ENUM, "both operands must be tensorwise or both block-scaled");
    if (sa.group != 0 && sa.group != 1 && sa.group != 128) return fail(FP8_ERR_ENUM, "scale_a.group must be 0, 1 or 128");
    if (sb.group != 0 && sb.group != 1 && sb.group != 128) return fail(FP8_ERR_ENUM, "scale_b.group must be 0, 1 or 128");
    const size_t need = fp8k::gemm_ws_bytes(I, J, K);
    if (need) {
        if (ws_bytes < need) return fail(FP8_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
        FP8_TRY(check_ptr16("ws", ws));
    }
    if (c_amax) {
        if (sa.group != 0) return fail(FP8_ERR_ENUM, "the output amax hand-off is for tensorwise GEMMs");
        FP8_TRY(check_ptr16("c_amax_partials", c_amax));
    }
    if (c_gelu_keys) {
        if (sa.group != 0 || fa != FP8_E4M3 || fb != FP8_E4M3)
            return fail(FP8_ERR_ENUM, "the GELU amax keys are emitted by tensorwise E4M3 x E4M3 GEMMs");
        FP8_TRY(check_ptr16("c_gelu_amax_partials", c_gelu_keys));
    }
    return do_gemm(a, fa, fp8k::GemmScale{sa.scale_inv, sa.group, sa.stride_r, sa.stride_kb}, b, fb,
                   fp8k::GemmScale{sb.scale_inv, sb.group, sb.stride_r, sb.stride_kb}, I, J, K, c, ws, ws_bytes,
                   static_cast<hipStream_t>(stream), c_amax, c_gelu_keys);
}

fp8_status fp8_gemm(const void* a, fp8_format fa, fp8_gemm_scale sa, const void* b, fp8_format fb, fp8_gemm_scale sb,
                    int64_t I, int64_t J, int64_t K, void* c, void* ws, size_t ws_bytes, void* stream) {
    return gemm_checked(a, fa, sa, b, fb, sb, I, J, K, c, ws, ws_bytes, stream, nullptr);
}

fp8_status fp8_gemm_amax(const void* a, fp8_format fa, fp8_gemm_scale sa, const void* b, fp8_format fb,
                         fp8_gemm_scale sb, int64_t I, int64_t J, int64_t K, void* c, void* c_amax_partials, void* ws,
                         size_t ws_bytes, void* stream) {
    if (!c_amax_partials) return fail(FP8_ERR_NULL, "c_amax_partials is NULL");
    return gemm_checked(a, fa, sa, b, fb, sb, I, J, K, c, ws, ws_bytes, stream, c_amax_partials);
}

fp8_status fp8_gemm_gelu_amax(const void* a, fp8_format fa, fp8_gemm_scale sa, const void* b, fp8_format fb,
                              fp8_gemm_scale sb, int64_t I, int64_t J, int64_t K, void* c,
                              void* c_gelu_amax_partials, void* ws, size_t ws_bytes, void* stream) {
    if (!c_gelu_amax_partials) return fail(FP8_ERR_NULL, "c_gelu_amax_partials is NULL");
    return gemm_checked(a, fa, sa, b, fb, sb, I, J, K, c, ws, ws_bytes, stream, nullptr, c_gelu_amax_partials);
}

fp8_status fp8_quantize_gelu_from_amax(const void* x, int64_t rows, int64_t cols, fp8_format format,
                                       unsigned layouts, const fp8_qtensor* out, const void* gelu_amax_partials,
                                       void* stream) {
    FP8_TRY(check_quantize(x, rows, cols, format, FP8_SCALE_TENSOR, layouts, out));
    FP8_TRY(check_ptr16("gelu_amax_partials", gelu_amax_partials));
    return do_quantize(x, rows, cols, format, FP8_SCALE_TENSOR, layouts, out, nullptr,
                       static_cast<hipStream_t>(stream), nullptr, 1, nullptr, gelu_amax_partials);
}

fp8_status fp8_wcache_create(int64_t M, int64_t K, fp8_recipe recipe, const fp8_qtensor* bufs, fp8_wcache* out) {
    if (!out) return fail(FP8_ERR_NULL, "output handle pointer is NULL");
    FP8_TRY(check_dims("weight cache", M, K));
    if (recipe != FP8_RECIPE_TENSOR && recipe != FP8_RECIPE_BLOCK) return fail(FP8_ERR_ENUM, "unknown recipe %d", recipe);
    FP8_TRY(check_weight_q(bufs, recipe, true, true));
    fp8_wcache h = static_cast<fp8_wcache>(std::calloc(1, sizeof(fp8_wcache_s)));
    if (!h) return fail(FP8_ERR_NULL, "out of host memory");
    h->M = M;
    h->K = K;
    h->recipe = recipe;
    h->bufs = *bufs;
    h->valid = 0;
    h->fills = 0;
    *out = h;
    return FP8_OK;
}

fp8_status fp8_wcache_invalidate(fp8_wcache h) {
    if (!h) return fail(FP8_ERR_NULL, "cache handle is NULL");
    h->valid = 0;
    return FP8_OK;
}

int fp8_wcache_valid(fp8_wcache h) { return h ? h->valid : -1; }
int64_t fp8_wcache_fills(fp8_wcache h) { return h ? h->fills : -1; }
void fp8_wcache_destroy(fp8_wcache h) { std::free(h); }

size_t fp8_linear_workspace_bytes(int64_t N, int64_t K, int64_t M, fp8_recipe recipe) {
    (void)recipe;
    // the input's amax partials, then the GEMM workspace; the GEMM part is at
    // least 4 KiB so that the forward can hold the weight's partials there
    // while it quantizes input and weight together
    const size_t g = linear_gemm_ws(N, K, M);
    return kPartialBytes + (g > kPartialBytes ? g : kPartialBytes);
}

static fp8_status check_linear_dims(int64_t N, int64_t K, int64_t M, int recipe) {
    FP8_TRY(check_dims("linear N x K", N, K));
    FP8_TRY(check_dims("linear M", M, 128));
    // N, K and M are each the contraction of one of the three GEMMs
    if (N >= kMaxContraction || K >= kMaxContraction || M >= kMaxContraction)
        return fail(FP8_ERR_SHAPE, "linear dimensions must be below 2^23");
    if (recipe != FP8_RECIPE_TENSOR && recipe != FP8_RECIPE_BLOCK) return fail(FP8_ERR_ENUM, "unknown recipe %d", recipe);
    return FP8_OK;
}

// Workspace of the forward pass alone: the input's amax partials, then the
// forward GEMM's split-K partials (at least 4 KiB, where the tensorwise
// forward keeps the weight's amax partials).
static size_t linear_fwd_ws_bytes(int64_t N, int64_t K, int64_t M) {
    const size_t g = fp8k::gemm_ws_bytes(N, M, K);
    return kPartialBytes + (g > kPartialBytes ? g : kPartialBytes);
}

// need == 0: the whole linear's workspace (fp8_linear_workspace_bytes)
static fp8_status check_linear_common(int64_t N, int64_t K, int64_t M, int recipe, void* ws, size_t ws_bytes,
                                      size_t need = 0) {
    FP8_TRY(check_linear_dims(N, K, M, recipe));
    if (!need) need = fp8_linear_workspace_bytes(N, K, M, static_cast<fp8_recipe>(recipe));
    if (ws_bytes < need) return fail(FP8_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    FP8_TRY(check_ptr16("ws", ws));
    return FP8_OK;
}

static fp8_status check_cache(fp8_wcache cache, int64_t M, int64_t K, int recipe) {
    if (!cache) return fail(FP8_ERR_NULL, "cache handle is NULL");
    if (cache->M != M || cache->K != K || cache->recipe != recipe)
        return fail(FP8_ERR_CACHE_MISMATCH, "cache holds %lld x %lld recipe %d, call has %lld x %lld recipe %d",
                    (long long)cache->M, (long long)cache->K, cache->recipe, (long long)M, (long long)K, recipe);
    return FP8_OK;
}

// The optional amax hand-off buffers of the linear (tensorwise recipe only).
static fp8_status check_amax_handoff(int recipe, const void* in, const void* out, const char* in_name,
                                     const char* out_name) {
    if (!in && !out) return FP8_OK;
    if (recipe != FP8_RECIPE_TENSOR) return fail(FP8_ERR_ENUM, "the amax hand-off is for the tensorwise recipe");
    if (in) FP8_TRY(check_ptr16(in_name, in));
    if (out) FP8_TRY(check_ptr16(out_name, out));
    return FP8_OK;
}

// One forward pass, checked completely before anything is launched.
// act 1: the linear's input is GELU(x) (x the pre-activation), quantized
// without being written out; x_gelu_keys (tensorwise, optional) are then the
// GELU amax keys of x, which replace the amax pass.  y_gelu_keys
// (tensorwise): receives the GELU amax keys of Y.
struct FwdCall {
    const void* x;
    int act;
    const void* w;
    int64_t N, K, M;
    fp8_recipe recipe;
    fp8_wcache cache;
    int flag;
    void* y;
    const fp8_qtensor* saved_x;
    const fp8_qtensor* w_q;
    const void* x_amax_partials;
    void* y_amax_partials;
    void* y_gelu_keys;
    const void* x_gelu_keys;
    void* ws;
    size_t ws_bytes;
    size_t ws_need;            // 0: the whole linear's workspace
    const fp8_qtensor* wq;     // resolved by check_fwd
};

static fp8_status check_fwd(FwdCall& c) {
    FP8_TRY(check_linear_common(c.N, c.K, c.M, c.recipe, c.ws, c.ws_bytes, c.ws_need));
    if (c.flag != -1 && c.flag != 0 && c.flag != 1) return fail(FP8_ERR_ENUM, "is_first_microbatch must be -1, 0 or 1");
    FP8_TRY(check_ptr16("x", c.x));
    FP8_TRY(check_ptr16("y", c.y));
    FP8_TRY(check_amax_handoff(c.recipe, c.x_amax_partials, c.y_amax_partials, "x_amax_partials", "y_amax_partials"));
    FP8_TRY(check_amax_handoff(c.recipe, c.x_gelu_keys, c.y_gelu_keys, "x_gelu_keys", "y_gelu_keys"));
    if (c.x_gelu_keys && (c.act != 1 || c.x_amax_partials))
        return fail(FP8_ERR_ENUM, "GELU amax keys serve the quantize of GELU(x) alone");
    const int xsc = c.recipe == FP8_RECIPE_BLOCK ? FP8_SCALE_BLOCK_1x128 : FP8_SCALE_TENSOR;
    const int wsc = c.recipe == FP8_RECIPE_BLOCK ? FP8_SCALE_BLOCK_128x128 : FP8_SCALE_TENSOR;
    FP8_TRY(check_quantize(c.x, c.N, c.K, FP8_E4M3, xsc, FP8_LAYOUT_ROW | FP8_LAYOUT_COL, c.saved_x));
    if (c.flag == -1) {
        FP8_TRY(check_weight_q(c.w_q, c.recipe, true, true));
        FP8_TRY(check_quantize(c.w, c.M, c.K, FP8_E4M3, wsc, FP8_LAYOUT_ROW | FP8_LAYOUT_COL, c.w_q));
        c.wq = c.w_q;
    } else {
        FP8_TRY(check_cache(c.cache, c.M, c.K, c.recipe));
        if (c.flag == 1) {
            FP8_TRY(check_quantize(c.w, c.M, c.K, FP8_E4M3, wsc, FP8_LAYOUT_ROW | FP8_LAYOUT_COL, &c.cache->bufs));
        } else if (!c.cache->valid) {
            return fail(FP8_ERR_CACHE_EMPTY, "is_first_microbatch=False on an empty weight cache");
        }
        c.wq = &c.cache->bufs;
    }
    return FP8_OK;
}

static fp8_status run_fwd(const FwdCall& c, hipStream_t st) {
    const int xsc = c.recipe == FP8_RECIPE_BLOCK ? FP8_SCALE_BLOCK_1x128 : FP8_SCALE_TENSOR;
    const int wsc = c.recipe == FP8_RECIPE_BLOCK ? FP8_SCALE_BLOCK_128x128 : FP8_SCALE_TENSOR;
    const int64_t N = c.N, K = c.K, M = c.M;
    const fp8_qtensor* wq = c.wq;
    uint8_t* wsb = static_cast<uint8_t*>(c.ws);
    void* gws = wsb + kPartialBytes;
    const size_t gws_bytes = c.ws_bytes - kPartialBytes;
    if (c.flag != 0 && c.recipe == FP8_RECIPE_TENSOR && c.act == 0 && !c.x_amax_partials) {
        // X and W together: one amax launch and one cast launch; W's partials
        // borrow the GEMM workspace (at least 4 KiB, checked above), which the
        // forward GEMM only uses after
        FP8_TRY(do_quantize_pair(c.x, N, K, c.saved_x, c.ws, c.w, M, K, wq, gws, st));
    } else {
        if (c.flag != 0)
            FP8_TRY(do_quantize(c.w, M, K, FP8_E4M3, wsc, FP8_LAYOUT_ROW | FP8_LAYOUT_COL, wq, c.ws, st));
        FP8_TRY(do_quantize(c.x, N, K, FP8_E4M3, xsc, FP8_LAYOUT_ROW | FP8_LAYOUT_COL, c.saved_x, c.ws, st,
                            c.x_amax_partials, c.act, nullptr, c.x_gelu_keys));
    }
    if (c.flag == 1) {
        c.cache->valid = 1;
        c.cache->fills++;
    }
    const fp8_qtensor* sx = c.saved_x;
    if (c.recipe == FP8_RECIPE_TENSOR)
        return do_gemm(sx->q_row, FP8_E4M3, tensor_scale(sx->scale_inv), wq->q_row, FP8_E4M3,
                       tensor_scale(wq->scale_inv), N, M, K, c.y, gws, gws_bytes, st, c.y_amax_partials,
                       c.y_gelu_keys);
    return do_gemm(sx->q_row, FP8_E4M3, block_scale(sx->scale_inv, 1, 1, N), wq->q_row, FP8_E4M3,
                   block_scale(wq->scale_inv, 128, K / 128, 1), N, M, K, c.y, gws, gws_bytes, st);
}

// ws_need: 0 for the whole linear's workspace, else the forward's alone
static fp8_status linear_fwd(const void* x, int act, const void* w, int64_t N, int64_t K, int64_t M,
                             fp8_recipe recipe, fp8_wcache cache, int flag, void* y, const fp8_qtensor* saved_x,
                             const fp8_qtensor* w_q, const void* x_amax_partials, void* y_amax_partials, void* ws,
                             size_t ws_bytes, void* stream, size_t ws_need = 0) {
    FwdCall c{x, act, w, N, K, M, recipe, cache, flag, y, saved_x, w_q, x_amax_partials, y_amax_partials, nullptr,
              nullptr, ws, ws_bytes, ws_need, nullptr};
    FP8_TRY(check_fwd(c));
    return run_fwd(c, static_cast<hipStream_t>(stream));
}

fp8_status fp8_linear_fwd(const void* x, const void* w, int64_t N, int64_t K, int64_t M, fp8_recipe recipe,
                          fp8_wcache cache, int flag, void* y, const fp8_qtensor* saved_x, const fp8_qtensor* w_q,
                          const void* x_amax_partials, void* y_amax_partials, void* ws, size_t ws_bytes,
                          void* stream) {
    return linear_fwd(x, 0, w, N, K, M, recipe, cache, flag, y, saved_x, w_q, x_amax_partials, y_amax_partials, ws,
                      ws_bytes, stream);
}

fp8_status fp8_linear_fwd_noalloc(const void* x, const void* w, int64_t N, int64_t K, int64_t M,
                                  fp8_recipe recipe, fp8_wcache cache, int flag, void* y,
                                  const fp8_qtensor* saved_x, const fp8_qtensor* w_q,
                                  const void* x_amax_partials, void* y_amax_partials, void* stream) {
    FP8_TRY(check_linear_dims(N, K, M, recipe));
    const size_t need = linear_fwd_ws_bytes(N, K, M);
    if (need > fp8k::kNoallocScratchBytes)
        return fail(FP8_ERR_WORKSPACE,
                    "this forward needs %zu bytes of scratch (split-K partials of its GEMM), more than the %zu-byte "
                    "device scratch of fp8_linear_fwd_noalloc; use fp8_linear_fwd with a workspace",
                    need, fp8k::kNoallocScratchBytes);
    void* scratch = nullptr;
    FP8_TRY(hip_status(fp8k::noalloc_scratch(&scratch), "device scratch address"));
    return linear_fwd(x, 0, w, N, K, M, recipe, cache, flag, y, saved_x, w_q, x_amax_partials, y_amax_partials,
                      scratch, fp8k::kNoallocScratchBytes, stream, need);
}

fp8_status fp8_linear_fwd_gelu(const void* x_pre, const void* w, int64_t N, int64_t K, int64_t M, fp8_recipe recipe,
                               fp8_wcache cache, int flag, void* y, const fp8_qtensor* saved_x,
                               const fp8_qtensor* w_q, void* y_amax_partials, void* ws, size_t ws_bytes,
                               void* stream) {
    return linear_fwd(x_pre, 1, w, N, K, M, recipe, cache, flag, y, saved_x, w_q, nullptr, y_amax_partials, ws,
                      ws_bytes, stream);
}

// ------------------------- BF16 comparator -------------------------

size_t fp8_bf16_gemm_workspace_bytes(int64_t I, int64_t J, int64_t K) { return fp8k::gemm_bf16_ws_bytes(I, J, K); }

static fp8_status bf16_gemm_checked(const void* a, int la, const void* b, int lb, int64_t I, int64_t J, int64_t K,
                                    void* c, void* ws, size_t ws_bytes) {
    FP8_TRY(check_dims("bf16 gemm I x J", I, J));
    FP8_TRY(check_dims("bf16 gemm K", K, 128));
    if ((la != 0 && la != 1) || (lb != 0 && lb != 1)) return fail(FP8_ERR_ENUM, "operand layout must be 0 or 1");
    FP8_TRY(check_ptr16("a", a));
    FP8_TRY(check_ptr16("b", b));
    FP8_TRY(check_ptr16("c", c));
    const size_t need = fp8k::gemm_bf16_ws_bytes(I, J, K);
    if (need) {
        if (ws_bytes < need) return fail(FP8_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
        FP8_TRY(check_ptr16("ws", ws));
    }
    return FP8_OK;
}

static fp8_status bf16_gemm_run(const void* a, int la, const void* b, int lb, int64_t I, int64_t J, int64_t K, void* c,
                                void* ws, hipStream_t st) {
    fp8k::Bf16GemmLaunch l{a, la, b, lb, I, J, K, c, ws};
    return hip_status(fp8k::launch_gemm_bf16(l, st), "bf16 gemm launch");
}

fp8_status fp8_bf16_gemm(const void* a, int a_layout, const void* b, int b_layout, int64_t I, int64_t J, int64_t K,
                         void* c, void* ws, size_t ws_bytes, void* stream) {
    FP8_TRY(bf16_gemm_checked(a, a_layout, b, b_layout, I, J, K, c, ws, ws_bytes));
    return bf16_gemm_run(a, a_layout, b, b_layout, I, J, K, c, ws, static_cast<hipStream_t>(stream));
}

size_t fp8_bf16_linear_workspace_bytes(int64_t N, int64_t K, int64_t M) {
    if (!dim_ok(N) || !dim_ok(K) || !dim_ok(M)) return 0;
    const size_t a = fp8k::gemm_bf16_ws_bytes(N, M, K), b = fp8k::gemm_bf16_ws_bytes(N, K, M),
                 c = fp8k::gemm_bf16_ws_bytes(M, K, N);
    const size_t m = a > b ? a : b;
    return m > c ? m : c;
}

fp8_status fp8_bf16_linear_fwd(const void* x, const void* w, int64_t N, int64_t K, int64_t M, void* y, void* ws,
                               size_t ws_bytes, void* stream) {
    FP8_TRY(bf16_gemm_checked(x, 0, w, 0, N, M, K, y, ws, ws_bytes));
    return bf16_gemm_run(x, 0, w, 0, N, M, K, y, ws, static_cast<hipStream_t>(stream));
}

fp8_status fp8_bf16_linear_bwd(const void* dy, const void* x, const void* w, int64_t N, int64_t K, int64_t M,
                               void* dx, void* dw, void* ws, size_t ws_bytes, void* stream) {
    if (!dx && !dw) return fail(FP8_ERR_NULL, "dx and dw are both NULL");
    // dX [N, K] = dY W: contraction over M, W read output-major
    if (dx) FP8_TRY(bf16_gemm_checked(dy, 0, w, 1, N, K, M, dx, ws, ws_bytes));
    // dW [M, K] = dY^T X: contraction over N, both read output-major
    if (dw) FP8_TRY(bf16_gemm_checked(dy, 1, x, 1, M, K, N, dw, ws, ws_bytes));
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dx) FP8_TRY(bf16_gemm_run(dy, 0, w, 1, N, K, M, dx, ws, st));
    if (dw) FP8_TRY(bf16_gemm_run(dy, 1, x, 1, M, K, N, dw, ws, st));
    return FP8_OK;
}

// The MLP block's forward: the up projection writes the pre-activation A and,
// tensorwise, the GELU amax keys of A; the down projection's input GELU(A)
// is then quantized in one pass (its amax from the keys).
constexpr size_t kGeluKeyBytes = 4 * kPartialBytes;

size_t fp8_mlp_workspace_bytes(int64_t N, int64_t D, int64_t H, fp8_recipe recipe) {
    (void)recipe;
    if (!dim_ok(N) || !dim_ok(D) || !dim_ok(H)) return 0;
    const size_t a = linear_fwd_ws_bytes(N, D, H), b = linear_fwd_ws_bytes(N, H, D);
    return kGeluKeyBytes + (a > b ? a : b);
}

fp8_status fp8_mlp_fwd(const void* x, const void* w1, const void* w2, int64_t N, int64_t D, int64_t H,
                       fp8_recipe recipe, fp8_wcache cache1, fp8_wcache cache2, int flag, void* a, void* y,
                       const fp8_qtensor* saved_x1, const fp8_qtensor* w1_q, const fp8_qtensor* saved_x2,
                       const fp8_qtensor* w2_q, const void* x_amax_partials, void* y_amax_partials, void* ws,
                       size_t ws_bytes, void* stream) {
    FP8_TRY(check_linear_dims(N, D, H, recipe));
    FP8_TRY(check_linear_dims(N, H, D, recipe));
    const size_t need = fp8_mlp_workspace_bytes(N, D, H, recipe);
    if (ws_bytes < need) return fail(FP8_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    FP8_TRY(check_ptr16("ws", ws));
    if (a == y) return fail(FP8_ERR_SHAPE, "a and y must be different buffers");
    const bool keys = recipe == FP8_RECIPE_TENSOR;
    uint8_t* wsb = static_cast<uint8_t*>(ws);
    void* kbuf = wsb;                       // GELU amax keys of A
    void* lws = wsb + kGeluKeyBytes;        // the linears' workspace
    const size_t lws_bytes = ws_bytes - kGeluKeyBytes;
    FwdCall up{x, 0, w1, N, D, H, recipe, cache1, flag, a, saved_x1, w1_q, x_amax_partials, nullptr,
               keys ? kbuf : nullptr, nullptr, lws, lws_bytes, linear_fwd_ws_bytes(N, D, H), nullptr};
    FwdCall down{a, 1, w2, N, H, D, recipe, cache2, flag, y, saved_x2, w2_q, nullptr, y_amax_partials, nullptr,
                 keys ? kbuf : nullptr, lws, lws_bytes, linear_fwd_ws_bytes(N, H, D), nullptr};
    FP8_TRY(check_fwd(up));
    FP8_TRY(check_fwd(down));
    if (cache1 && cache1 == cache2) return fail(FP8_ERR_CACHE_MISMATCH, "the two linears need their own caches");
    hipStream_t st = static_cast<hipStream_t>(stream);
    FP8_TRY(run_fwd(up, st));
    return run_fwd(down, st);
}

// act 2: the incoming gradient is dGELU(dy, y_pre): dy the gradient of
// GELU's output and y_pre its input (this linear's output in the forward
// pass), quantized without being written out
static fp8_status linear_bwd(const void* dy, int act, const void* y_pre, int64_t N, int64_t K, int64_t M,
                             fp8_recipe recipe, const fp8_qtensor* saved_x, fp8_wcache cache, const fp8_qtensor* w_q,
                             const fp8_qtensor* dy_q, void* dx, void* dw, const void* dy_amax_partials,
                             void* dx_amax_partials, void* ws, size_t ws_bytes, void* stream) {
    FP8_TRY(check_linear_common(N, K, M, recipe, ws, ws_bytes));
    FP8_TRY(check_ptr16("dy", dy));
    if (!dx && !dw) return fail(FP8_ERR_NULL, "both dx and dw are NULL: nothing to compute");
    FP8_TRY(check_amax_handoff(recipe, dy_amax_partials, dx_amax_partials, "dy_amax_partials", "dx_amax_partials"));
    if (dx_amax_partials && !dx) return fail(FP8_ERR_NULL, "dx_amax_partials given without dx");
    if (dx) FP8_TRY(check_ptr16("dx", dx));
    if (dw) FP8_TRY(check_ptr16("dw", dw));
    const int gsc = recipe == FP8_RECIPE_BLOCK ? FP8_SCALE_BLOCK_1x128 : FP8_SCALE_TENSOR;
    const unsigned lay = (dx ? FP8_LAYOUT_ROW : 0u) | (dw ? FP8_LAYOUT_COL : 0u);
    FP8_TRY(check_quantize(dy, N, M, FP8_E5M2, gsc, lay, dy_q));
    if (act == 2) FP8_TRY(check_ptr16("y_pre", y_pre));
    const fp8_qtensor* wq = nullptr;
    if (dx) {
        if (cache) {
            FP8_TRY(check_cache(cache, M, K, recipe));
            if (!cache->valid) return fail(FP8_ERR_CACHE_EMPTY, "backward with an empty weight cache");
            wq = &cache->bufs;
        } else {
            FP8_TRY(check_weight_q(w_q, recipe, false, true));
            wq = w_q;
        }
    }
    if (dw) {
        if (!saved_x) return fail(FP8_ERR_NULL, "saved_x is NULL");
        FP8_TRY(check_ptr16("saved_x.q_col", saved_x->q_col));
        if (recipe == FP8_RECIPE_BLOCK) FP8_TRY(check_ptr4("saved_x.scale_inv_col", saved_x->scale_inv_col));
        else FP8_TRY(check_ptr4("saved_x.scale_inv", saved_x->scale_inv));
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t* wsb = static_cast<uint8_t*>(ws);
    void* gws = wsb + kPartialBytes;
    const size_t gws_bytes = ws_bytes - kPartialBytes;
    FP8_TRY(do_quantize(dy, N, M, FP8_E5M2, gsc, lay, dy_q, ws, st, dy_amax_partials, act, y_pre));
    if (dx) {
        if (recipe == FP8_RECIPE_TENSOR)
            FP8_TRY(do_gemm(dy_q->q_row, FP8_E5M2, tensor_scale(dy_q->scale_inv), wq->q_col, FP8_E4M3,
                            tensor_scale(wq->scale_inv), N, K, M, dx, gws, gws_bytes, st, dx_amax_partials));
        else
            FP8_TRY(do_gemm(dy_q->q_row, FP8_E5M2, block_scale(dy_q->scale_inv, 1, 1, N), wq->q_col, FP8_E4M3,
                            block_scale(wq->scale_inv, 128, 1, K / 128), N, K, M, dx, gws, gws_bytes, st));
    }
    if (dw) {
        if (recipe == FP8_RECIPE_TENSOR)
            FP8_TRY(do_gemm(dy_q->q_col, FP8_E5M2, tensor_scale(dy_q->scale_inv), saved_x->q_col, FP8_E4M3,
                            tensor_scale(saved_x->scale_inv), M, K, N, dw, gws, gws_bytes, st));
        else
            FP8_TRY(do_gemm(dy_q->q_col, FP8_E5M2, block_scale(dy_q->scale_inv_col, 1, 1, M), saved_x->q_col,
                            FP8_E4M3, block_scale(saved_x->scale_inv_col, 1, 1, K), M, K, N, dw, gws, gws_bytes,
                            st));
    }
    return FP8_OK;
}

fp8_status fp8_linear_bwd(const void* dy, int64_t N, int64_t K, int64_t M, fp8_recipe recipe,
                          const fp8_qtensor* saved_x, fp8_wcache cache, const fp8_qtensor* w_q,
                          const fp8_qtensor* dy_q, void* dx, void* dw, const void* dy_amax_partials,
                          void* dx_amax_partials, void* ws, size_t ws_bytes, void* stream) {
    return linear_bwd(dy, 0, nullptr, N, K, M, recipe, saved_x, cache, w_q, dy_q, dx, dw, dy_amax_partials,
                      dx_amax_partials, ws, ws_bytes, stream);
}

fp8_status fp8_linear_bwd_dgelu(const void* dh, const void* y_pre, int64_t N, int64_t K, int64_t M,
                                fp8_recipe recipe, const fp8_qtensor* saved_x, fp8_wcache cache,
                                const fp8_qtensor* w_q, const fp8_qtensor* dy_q, void* dx, void* dw,
                                void* dx_amax_partials, void* ws, size_t ws_bytes, void* stream) {
    return linear_bwd(dh, 2, y_pre, N, K, M, recipe, saved_x, cache, w_q, dy_q, dx, dw, nullptr, dx_amax_partials,
                      ws, ws_bytes, stream);
}

}  // extern "C"
