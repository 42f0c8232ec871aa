// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8k {

constexpr int kMaxAmaxPartials = 2048;   // 16-bit slots, a multiple of 512
constexpr int kMaxHistory = 1024;        // longest amax history of delayed scaling

struct QuantizeLaunch {
    const void* x;      // [rows, cols] bf16
    int64_t rows, cols;
    int format;         // 0 E4M3, 1 E5M2
    int scaling;        // 0 tensor, 1 1x128, 2 128x128, 3 tensor with delayed scaling
    void* q_row;        // may be null
    void* q_col;        // may be null
    float* scale;
    float* scale_inv;
    float* scale_col;
    float* scale_inv_col;
    float* amax;        // optional
    uint16_t* partial;  // tensor: kMaxAmaxPartials 16-bit slots of scratch (16-byte aligned)
    bool partial_given; // tensor: partial already holds the amax partials of x (written by
                        // the producer of x); the amax pass is skipped
    float* hist;        // delayed: amax history [hist_len], most recent first (read, then rolled);
    int hist_len;       // partial then holds one 16-bit amax per 128x128 tile
    int act = 0;        // 0: quantize x; 1: quantize GELU(x); 2: quantize dGELU(x, x2), x the
                        // gradient of GELU's output and x2 its input (scaling 0 or 1 only)
    const void* x2 = nullptr;
    const uint16_t* gelu_keys = nullptr;   // act 1, tensorwise: the GELU amax keys x's producer
                                           // wrote (gelu_keys.hpp); the amax pass is skipped
};

int amax_partial_count(int64_t numel);
hipError_t launch_quantize(const QuantizeLaunch& q, hipStream_t stream);
// two tensorwise quantizes, same format, no transform, amax pass included
// (partial_given false), each with its own partials buffer
hipError_t launch_quantize_pair(const QuantizeLaunch& qa, const QuantizeLaunch& qb, hipStream_t stream);

// GELU tables of the current device (gelu.hip): built on first use, which
// waits for them and cannot be captured into a graph.
struct ActTables {
    const uint16_t* gelu;   // bf16 GELU of the table's inputs
    const float* dgelu;     // fp32 GELU' of the table's inputs
};
hipError_t act_tables(hipStream_t stream, ActTables& out);
// elementwise GELU / dGELU over n bf16 values (n a multiple of 8)
hipError_t launch_gelu(const void* x, void* y, int64_t n, hipStream_t stream);
hipError_t launch_dgelu(const void* dy, const void* x, void* dx, int64_t n, hipStream_t stream);

struct GemmScale {
    const float* sinv;
    int64_t group;      // 0 tensorwise, else rows per scale group (1 or 128)
    int64_t stride_r;
    int64_t stride_kb;
};

struct GemmLaunch {
    const void* a;      // [I, K] FP8
    int fa;
    GemmScale sa;
    const void* b;      // [J, K] FP8
    int fb;
    GemmScale sb;
    int64_t I, J, K;
    void* c;            // [I, J] bf16
    void* ws;           // split-K partials
    size_t ws_bytes;
    uint16_t* c_amax;   // tensorwise, optional: kMaxAmaxPartials partial maxima of |C|
                        // (bf16 magnitude bits, 0 in unused slots)
    uint16_t* gelu_keys = nullptr;   // tensorwise E4M3 x E4M3, optional: the GELU amax keys
                                     // of C (4 arrays of kMaxAmaxPartials slots, gelu_keys.hpp)
};

// Split-K factor the GEMM launcher will use for this shape (1 = none) and
// the workspace bytes that needs.
// tensorwise kernel (gemm_tensor.hip)
int gemm_tensor_splits(int64_t I, int64_t J, int64_t K);
hipError_t launch_gemm_tensor(const GemmLaunch& l, int splits, hipStream_t stream);
// block-scaled kernel (gemm_block.hip)
int gemm_block_splits(int64_t I, int64_t J, int64_t K);
hipError_t launch_gemm_block(const GemmLaunch& l, int splits, hipStream_t stream);
// block-scaled kernel for B factors shared by 128-row groups (gemm_block_wide.hip)
int gemm_block_wide_splits(int64_t I, int64_t J, int64_t K);
hipError_t launch_gemm_block_wide(const GemmLaunch& l, int splits, hipStream_t stream);
size_t gemm_ws_bytes(int64_t I, int64_t J, int64_t K);
hipError_t launch_gemm(const GemmLaunch& g, hipStream_t stream);

// Deterministic sum of split-K fp32 partials [splits][I][J] in slice order,
// times fl32(sa[0] * sb[0]) when sa is given (tensorwise), rounded to bf16
// into c (gemm.hip).
hipError_t launch_splitk_reduce(const float* part, int splits, int64_t I, int64_t J, const float* sa,
                                const float* sb, uint16_t* c, hipStream_t stream);

// BF16 GEMM (gemm_bf16.hip): C [I, J] = bf16(sum_k A[i][k] B[j][k]) with
// fp32 accumulation; layout 0: contraction-major (A[i][k] at i*K + k),
// 1: output-major (A[i][k] at k*I + i; B likewise with J).  ws: split-K
// partials, gemm_bf16_ws_bytes.
struct Bf16GemmLaunch {
    const void* a;
    int ta;
    const void* b;
    int tb;
    int64_t I, J, K;
    void* c;
    void* ws;
};
int gemm_bf16_splits(int64_t I, int64_t J, int64_t K);
size_t gemm_bf16_ws_bytes(int64_t I, int64_t J, int64_t K);
hipError_t launch_gemm_bf16(const Bf16GemmLaunch& l, hipStream_t stream);

// Scratch of the entry point that allocates nothing (noalloc.hip): a device
// array of kNoallocScratchBytes per GPU; *out receives the current device's
// address of it (taken once per device).
constexpr size_t kNoallocScratchBytes = size_t(8) << 20;
hipError_t noalloc_scratch(void** out);

}  // namespace fp8k
