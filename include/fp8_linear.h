/*
 * fp8_linear.h -- C ABI of the MI355X (gfx950) FP8 linear layer.
 *
 * The library computes the forward and backward pass of a linear layer in
 * FP8 with current scaling, as described in "Native FP8 MLP reconstruction"
 * (rstation.ai, implementation paragraph): every tensor's scale is set from
 * its amax on the call that uses it, X and W are coded as E4M3 and the
 * gradient dY as E5M2, a single cast pass yields the row-major codes and
 * their transpose, the three GEMMs (Y = X W^T, dX = dY W, dW = dY^T X) sum
 * in fp32 (no fast accumulation) and write BF16, and the backward pass
 * treats the scales as constants, takes the X and W codes of the forward
 * pass and quantizes dY by itself.  A block-scaled recipe (the Float8BlockScaling recipe
 * of TransformerEngine issue 2852, opening post) quantizes activations and
 * gradients in 1x128 blocks and weights in 128x128 blocks.  A weight cache
 * implements the is_first_microbatch protocol of the same issue (opening
 * post and the user's description of their flag injection): True quantizes
 * the weight and keeps it, False reuses the kept copy, None (-1) neither
 * reads nor writes it; for these non-delayed recipes the cached and
 * recomputed results are bitwise identical (maintainer reply in the issue).
 *
 * Conventions
 *  - Shapes follow nn.Linear: X [N, K], W [M, K] (out x in), Y [N, M],
 *    dY [N, M], dX [N, K], dW [M, K].  Every dimension must be a positive
 *    multiple of 128 (FP8_ERR_SHAPE otherwise).
 *  - Every tensor argument is a DEVICE pointer owned by the caller, row-major
 *    and 16-byte aligned (FP8_ERR_ALIGN otherwise).  bf16 tensors are raw
 *    16-bit patterns; FP8 tensors are one OCP code per byte (E4M3 "FN":
 *    max 448, NaN 0x7F; E5M2: max 57344).
 *  - The library allocates no device memory.  Functions that need scratch
 *    take (ws, ws_bytes); the needed size comes from the *_workspace_bytes
 *    queries.  Workspace contents need no initialisation and are not
 *    preserved between calls.
 *  - stream is a hipStream_t passed as void* (NULL = the default stream).
 *    All device work is enqueued on it asynchronously; no call synchronises
 *    the host.  Calls that share a workspace or a cache must be ordered on
 *    one stream (or by the caller).
 *  - Errors: every argument, shape, alignment and enum check happens before
 *    anything is enqueued, and a failed check leaves every output untouched.
 *    A failed kernel launch returns FP8_ERR_HIP.  fp8_last_error() gives a
 *    message for the calling thread's last failure.  Non-finite inputs are
 *    not errors: NaN encodes to 0x7F, +-Inf saturates to +-max, and a
 *    non-finite or zero amax gives scale 1.
 *
 * Scale semantics (per tensor, or per block)
 *    amax      = max |x| over the tensor / block (NaN if any NaN)
 *    scale     = FMAX / amax (fp32 division; 1 if amax is 0, Inf or NaN;
 *                FLT_MAX if the division overflows)
 *    scale_inv = 1 / scale (fp32 division), the dequantisation factor
 *    q         = encode_rne_saturating(fl32(x * scale))
 */
#ifndef FP8_LINEAR_H
#define FP8_LINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FP8_E4M3 = 0, FP8_E5M2 = 1 } fp8_format;

/* Per-tensor scaling of one quantized tensor. */
typedef enum {
    FP8_SCALE_TENSOR = 0,        /* one current amax for the whole tensor */
    FP8_SCALE_BLOCK_1x128 = 1,   /* row layout: blocks of 1 row x 128 columns;
                                    col layout: blocks of 128 rows x 1 column */
    FP8_SCALE_BLOCK_128x128 = 2  /* 128x128 tiles, shared by both layouts */
} fp8_scaling;

/* Recipe of a whole linear layer. */
typedef enum {
    FP8_RECIPE_TENSOR = 0,       /* X, W, dY tensorwise */
    FP8_RECIPE_BLOCK = 1         /* X, dY 1x128; W 128x128 */
} fp8_recipe;

enum { FP8_LAYOUT_ROW = 1, FP8_LAYOUT_COL = 2 };   /* bitmask */

typedef enum {
    FP8_OK = 0,
    FP8_ERR_NULL = 1,            /* a required pointer is NULL */
    FP8_ERR_SHAPE = 2,           /* a dimension is not a positive multiple of 128, or a
                                    contraction length is 2^23 or more */
    FP8_ERR_ALIGN = 3,           /* a pointer is not 16-byte aligned */
    FP8_ERR_ENUM = 4,            /* unknown format / scaling / recipe / layout / flag */
    FP8_ERR_WORKSPACE = 5,       /* ws_bytes smaller than the query returned */
    FP8_ERR_CACHE_EMPTY = 6,     /* is_first_microbatch = 0 on a cache never filled */
    FP8_ERR_CACHE_MISMATCH = 7,  /* cache shape or recipe differs from the call */
    FP8_ERR_HIP = 8,             /* a kernel launch failed */
    FP8_ERR_UNIMPLEMENTED = 9
} fp8_status;

/*
 * A quantized tensor: caller-owned device buffers.  For a source of shape
 * [R, C]:
 *   q_row      [R, C] codes (row layout), or NULL when not requested
 *   q_col      [C, R] codes (transposed layout), or NULL when not requested
 *   scale, scale_inv
 *              TENSOR:  1 float each
 *              1x128:   scales of the row layout, stored block-major as
 *                       [C/128, R]: block (r, cb) covering
 *                       x[r][cb*128 .. cb*128+127] at index cb*R + r
 *                       (16-byte aligned)
 *              128x128: [R/128, C/128] (shared by both layouts)
 *   scale_col, scale_inv_col
 *              1x128 only: scales of the col layout, stored block-major as
 *              [R/128, C]: block (c, rb) covering x[rb*128 .. rb*128+127][c]
 *              at index rb*C + c (16-byte aligned); ignored otherwise
 *   amax       optional (may be NULL): TENSOR: 1 float, the tensor's amax;
 *              ignored for block scaling
 */
typedef struct {
    void* q_row;
    void* q_col;
    float* scale;
    float* scale_inv;
    float* scale_col;
    float* scale_inv_col;
    float* amax;
} fp8_qtensor;

/* Opaque host-side weight-cache handle (holds shape, recipe, a valid bit and
 * a fill counter; the quantized bytes live in caller buffers). */
typedef struct fp8_wcache_s* fp8_wcache;

/* ------------------------------------------------------------------ */

/* Workspace bytes needed by fp8_quantize for a [rows, cols] source. */
size_t fp8_quantize_workspace_bytes(int64_t rows, int64_t cols, fp8_scaling scaling);

/*
 * Quantize a bf16 tensor x [rows, cols] to FP8 with current scaling
 * (amax computed now, from these values).  layouts is a bitmask of
 * FP8_LAYOUT_ROW / FP8_LAYOUT_COL; both layouts come from one pass over x
 * (the fused dual-layout cast of "Native FP8 MLP reconstruction",
 * implementation paragraph).  Requesting a single layout gives bytes
 * identical to those of the fused call.
 * Writes out->q_row / out->q_col (as requested), out->scale, out->scale_inv,
 * and for 1x128 with the col layout out->scale_col / out->scale_inv_col;
 * out->amax if non-NULL and TENSOR.
 */
fp8_status fp8_quantize(const void* x_bf16, int64_t rows, int64_t cols,
                        fp8_format format, fp8_scaling scaling, unsigned layouts,
                        const fp8_qtensor* out, void* ws, size_t ws_bytes, void* stream);

/*
 * Amax hand-off (producer-side amax).  The tensorwise quantize of x needs
 * amax(x) before it can encode, so by itself it reads x twice (the amax pass,
 * then the cast); the quantization reductions are the non-GEMM work of an FP8
 * linear ("Native FP8 MLP reconstruction", discussion: the model's FLOP
 * estimate leaves them out with the casts and layout writes).  When x is the
 * bf16 output of a GEMM of this library, that GEMM can emit the amax as it
 * writes x, and the quantize then reads x once:
 *   amax partials  FP8_AMAX_PARTIALS_BYTES of device memory (16-byte aligned):
 *                  2048 16-bit slots, each the maximum bf16 magnitude bits
 *                  (|x| as a bf16 bit pattern, NaN above +Inf) over a part of
 *                  x, unused slots 0.  amax(x) = the maximum over the slots.
 * Written by fp8_gemm_amax (and the linear entry points' *_amax_partials
 * outputs), read by fp8_quantize_from_amax (and their *_amax_partials
 * inputs).  The quantized bytes and scales are identical to fp8_quantize's
 * on the same x.
 */
#define FP8_AMAX_PARTIALS_BYTES 4096

/*
 * Tensorwise quantize of x whose amax partials were written by the producer
 * of x (see above): the cast pass alone, no workspace.  Arguments and outputs
 * as fp8_quantize with scaling = FP8_SCALE_TENSOR; amax_partials must be
 * non-NULL and 16-byte aligned.  Results are undefined if the partials do not
 * describe x.
 */
fp8_status fp8_quantize_from_amax(const void* x_bf16, int64_t rows, int64_t cols, fp8_format format,
                                  unsigned layouts, const fp8_qtensor* out, const void* amax_partials,
                                  void* stream);

/*
 * Delayed tensorwise scaling with an amax history: the DelayedScaling case
 * the weight-caching issue contrasts with block scaling ("FP8 weight caching
 * shows no speedup ... under Float8BlockScaling", TransformerEngine issue
 * 2852: the opening post and its third question).  amax_history
 * [history_len] (device fp32, 1 .. 1024 entries) holds the amaxes of this
 * tensor's previous quantize calls, most recent first.  The call encodes x
 * with scale = FMAX / max(history) (the current-scaling rules: 1 for a
 * history max of 0, +Inf or NaN, FLT_MAX on overflow), writes out->scale,
 * out->scale_inv (and out->amax, if non-NULL, with amax(x)), then rolls the
 * history by one entry and stores amax(x) in front.  One pass over x (the
 * encode needs no amax of x).  Workspace: one 16-bit amax per 128x128 tile,
 * fp8_quantize_delayed_workspace_bytes.  Calls that share a history must be
 * ordered (same stream); every call rolls it, so skipping a call (a cached
 * weight) changes the scales of later calls.
 */
size_t fp8_quantize_delayed_workspace_bytes(int64_t rows, int64_t cols);
fp8_status fp8_quantize_delayed(const void* x_bf16, int64_t rows, int64_t cols, fp8_format format,
                                unsigned layouts, const fp8_qtensor* out, float* amax_history,
                                int64_t history_len, void* ws, size_t ws_bytes, void* stream);

/*
 * Scale of an FP8 GEMM operand (dequantisation factors):
 *   group == 0:  tensorwise, the factor is scale_inv[0]
 *   group >= 1:  the factor of operand row r in contraction block kb
 *                (128 contraction elements) is
 *                scale_inv[(r / group) * stride_r + kb * stride_kb];
 *                group is 1 (1x128 blocks) or 128 (128x128 blocks).
 *                The 1x128 scales fp8_quantize writes give, for the row
 *                layout of an [R, C] source, stride_r = 1 and stride_kb = R,
 *                for its col layout stride_r = 1 and stride_kb = C.
 * Both operands of one GEMM must be tensorwise or both block-scaled.
 */
typedef struct {
    const float* scale_inv;
    int64_t group;
    int64_t stride_r;
    int64_t stride_kb;
} fp8_gemm_scale;

size_t fp8_gemm_workspace_bytes(int64_t I, int64_t J, int64_t K);

/*
 * C[i][j] = bf16( sum_k A[i][k] * B[j][k] * scales ), A [I, K] and B [J, K]
 * FP8 codes (both contraction-contiguous), C [I, J] bf16 row-major.
 * fp32 accumulation on the FP8 matrix cores.  Tensorwise: the fp32 sum is
 * multiplied by fl32(sA * sB) and rounded to bf16 (round to nearest even).
 * Block-scaled: every 128-long contraction block's fp32 partial sum is
 * multiplied by its two block factors and added to an fp32 accumulator.
 * format_a may be E4M3 or E5M2; format_b likewise.  The contraction length
 * K must be below 2^23 (FP8_ERR_SHAPE), which bounds the linear's N, K and M,
 * each the contraction of one of its GEMMs.
 */
fp8_status fp8_gemm(const void* a, fp8_format format_a, fp8_gemm_scale scale_a,
                    const void* b, fp8_format format_b, fp8_gemm_scale scale_b,
                    int64_t I, int64_t J, int64_t K, void* c_bf16,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * fp8_gemm (tensorwise operands only: FP8_ERR_ENUM otherwise) that also
 * writes the amax partials of its bf16 output C into c_amax_partials (see
 * "Amax hand-off"; NULL is FP8_ERR_NULL).  C is bitwise the same as
 * fp8_gemm's.
 */
fp8_status fp8_gemm_amax(const void* a, fp8_format format_a, fp8_gemm_scale scale_a,
                         const void* b, fp8_format format_b, fp8_gemm_scale scale_b,
                         int64_t I, int64_t J, int64_t K, void* c_bf16, void* c_amax_partials,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * GELU amax hand-off.  In the MLP block the down projection's input is
 * GELU(A), A the up projection's bf16 output, and amax(GELU(A)) is not a
 * function of amax(A): GELU falls to its minimum near -0.7518 and rises on
 * either side.  The GEMM that writes A therefore emits four 16-bit keys per
 * workgroup instead of one magnitude:
 *   gelu amax partials  FP8_GELU_AMAX_PARTIALS_BYTES of device memory
 *                  (16-byte aligned): four arrays of 2048 16-bit slots,
 *                  each reduced by unsigned maximum, 0 meaning "nothing":
 *     [0]  (v ^ 0x8000) for the largest non-negative value (bf16 pattern v,
 *          compared as signed 16-bit; NaN above +Inf)
 *     [1]  the largest bf16 pattern as unsigned (>= 0xFF80: a -Inf or a
 *          negative NaN is present, whose GELU is NaN)
 *     [2]  (v - 0xBF41) mod 2^16 maximised: at or above 0xC0BF it names the
 *          smallest value in [-0.75, 0)
 *     [3]  the complement of (v - 0xBF41) mod 2^16 minimised: at or above
 *          0xBF41 (complemented: a minimum at or below 0x40BE) it names the
 *          largest value below -0.75
 * -0.75 is the smallest bf16 value above GELU's minimiser; bf16(GELU) is
 * monotone on each side of it, so max |GELU| over the tensor is the largest
 * of |GELU| at the (at most three) values the keys name, or NaN.
 * Written by fp8_gemm_gelu_amax (and inside fp8_mlp_fwd), read by
 * fp8_quantize_gelu_from_amax (and inside fp8_mlp_fwd).
 */
#define FP8_GELU_AMAX_PARTIALS_BYTES 16384

/*
 * fp8_gemm for tensorwise E4M3 x E4M3 operands (FP8_ERR_ENUM otherwise) that
 * also writes the GELU amax partials of its bf16 output C into
 * c_gelu_amax_partials (NULL is FP8_ERR_NULL).  C is bitwise fp8_gemm's.
 */
fp8_status fp8_gemm_gelu_amax(const void* a, fp8_format format_a, fp8_gemm_scale scale_a,
                              const void* b, fp8_format format_b, fp8_gemm_scale scale_b,
                              int64_t I, int64_t J, int64_t K, void* c_bf16, void* c_gelu_amax_partials,
                              void* ws, size_t ws_bytes, void* stream);

/*
 * Tensorwise quantize of GELU(x) (as fp8_quantize_gelu) whose amax comes from
 * the GELU amax partials the producer of x wrote: the cast pass alone (each
 * of its workgroups reduces the 16 KiB of keys and evaluates GELU at the
 * values they name), no workspace.  The bytes and scales equal
 * fp8_quantize_gelu's on the same x; results are undefined if the partials
 * do not describe x.
 */
fp8_status fp8_quantize_gelu_from_amax(const void* x_bf16, int64_t rows, int64_t cols, fp8_format format,
                                       unsigned layouts, const fp8_qtensor* out,
                                       const void* gelu_amax_partials, void* stream);

/* ---------------------------- weight cache --------------------------- */

/*
 * Create a cache for a weight [M, K] under `recipe`.  bufs names caller
 * buffers for the quantized weight: q_row [M, K], q_col [K, M], scale and
 * scale_inv (1 float for TENSOR; [M/128, K/128] for BLOCK).  The handle
 * keeps these pointers; they must outlive it.  The cache starts empty.
 */
fp8_status fp8_wcache_create(int64_t M, int64_t K, fp8_recipe recipe,
                             const fp8_qtensor* bufs, fp8_wcache* out);
/* Mark the cache empty (e.g. after an optimizer step or loading weights). */
fp8_status fp8_wcache_invalidate(fp8_wcache cache);
/* 1 if the cache holds a quantized weight, 0 if empty, -1 on a NULL handle. */
int fp8_wcache_valid(fp8_wcache cache);
/* Number of times the cache has been filled since creation. */
int64_t fp8_wcache_fills(fp8_wcache cache);
void fp8_wcache_destroy(fp8_wcache cache);

/* ---------------------------- linear layer --------------------------- */

size_t fp8_linear_workspace_bytes(int64_t N, int64_t K, int64_t M, fp8_recipe recipe);

/*
 * Forward: Y [N, M] = X [N, K] W [M, K]^T in FP8 (E4M3 x E4M3), BF16 out.
 *   saved_x  receives X quantized in both layouts (q_row [N, K], q_col [K, N])
 *            with its scales; the backward pass reads its col layout.
 *   Weight source, by is_first_microbatch:
 *     -1 (None): W is quantized into w_q (both layouts); cache may be NULL
 *                and is neither read nor written.
 *      1 (True): W is quantized into the cache's buffers and the cache is
 *                marked valid; w_q is ignored.
 *      0 (False): the cache's quantized weight is used and w_bf16 is not
 *                read (it may be NULL); FP8_ERR_CACHE_EMPTY if the cache was
 *                never filled.
 *   A cache whose M, K or recipe differ gives FP8_ERR_CACHE_MISMATCH.
 *   Amax hand-off (tensorwise recipe only, FP8_ERR_ENUM otherwise; each may
 *   be NULL): x_amax_partials, written by the producer of X (the previous
 *   layer's forward), replaces X's amax pass; y_amax_partials receives Y's
 *   partials for the next layer.
 */
fp8_status fp8_linear_fwd(const void* x_bf16, const void* w_bf16,
                          int64_t N, int64_t K, int64_t M, fp8_recipe recipe,
                          fp8_wcache cache, int is_first_microbatch,
                          void* y_bf16, const fp8_qtensor* saved_x, const fp8_qtensor* w_q,
                          const void* x_amax_partials, void* y_amax_partials,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * Backward: dY [N, M] is quantized to E5M2 (both layouts, its own current
 * amax) into dy_q; then dX [N, K] = dY W (E5M2 x E4M3, W's col layout) and
 * dW [M, K] = dY^T X (E5M2 x E4M3, both col layouts).  The weight comes from
 * the cache when cache != NULL (it must be valid), else from w_q as written
 * by fp8_linear_fwd.  dx_bf16 or dw_bf16 may be NULL to skip that GEMM.
 * Amax hand-off (tensorwise recipe only; each may be NULL): dy_amax_partials,
 * written by the producer of dY (the next layer's backward), replaces dY's
 * amax pass; dx_amax_partials receives dX's partials (dx_bf16 must be given).
 */
fp8_status fp8_linear_bwd(const void* dy_bf16, int64_t N, int64_t K, int64_t M, fp8_recipe recipe,
                          const fp8_qtensor* saved_x, fp8_wcache cache, const fp8_qtensor* w_q,
                          const fp8_qtensor* dy_q, void* dx_bf16, void* dw_bf16,
                          const void* dy_amax_partials, void* dx_amax_partials,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * The MLP block's forward in one call: the up projection A [N, H] = X W1^T
 * (X [N, D], W1 [H, D]) and the down projection Y [N, D] = GELU(A) W2^T
 * (W2 [D, H]), each exactly as fp8_linear_fwd / fp8_linear_fwd_gelu would
 * compute it (bitwise the same A, Y, saved inputs and quantized weights).
 * Under the tensorwise recipe the up projection's GEMM writes the GELU amax
 * partials of A into the workspace, so the quantize of GELU(A) is the cast
 * pass alone instead of an amax pass plus the cast ("Native FP8 MLP
 * reconstruction", discussion: quantization reductions are the work the
 * model's FLOP estimate leaves out); under the block recipe that quantize is
 * one pass already.  A is written out because the backward pass
 * (fp8_linear_bwd on the down projection, fp8_linear_bwd_dgelu on the up
 * projection) needs it.  cache1 / cache2 follow the weight-cache protocol of
 * fp8_linear_fwd with one is_first_microbatch flag for both; saved_x1,
 * w1_q, saved_x2, w2_q are those of the two linears.  x_amax_partials
 * (tensorwise, may be NULL) replaces X's amax pass; y_amax_partials (may be
 * NULL) receives Y's.  Every check of both linears happens before anything
 * is enqueued.  ws: fp8_mlp_workspace_bytes bytes (0 for invalid sizes).
 */
size_t fp8_mlp_workspace_bytes(int64_t N, int64_t D, int64_t H, fp8_recipe recipe);
fp8_status fp8_mlp_fwd(const void* x_bf16, const void* w1_bf16, const void* w2_bf16,
                       int64_t N, int64_t D, int64_t H, fp8_recipe recipe,
                       fp8_wcache cache1, fp8_wcache cache2, int is_first_microbatch,
                       void* a_bf16, void* y_bf16,
                       const fp8_qtensor* saved_x1, const fp8_qtensor* w1_q,
                       const fp8_qtensor* saved_x2, const fp8_qtensor* w2_q,
                       const void* x_amax_partials, void* y_amax_partials,
                       void* ws, size_t ws_bytes, void* stream);

/* --------------------------- BF16 comparator --------------------------- */

/*
 * The pages' baseline: the same linears in BF16 without any quantization
 * ("Native FP8 MLP reconstruction", isolated-linear table, the compiled
 * BF16 column), here as hand-written BF16 matrix-core GEMMs so that the
 * FP8/BF16 speed ratio on this GPU comes from this library's own kernels.
 *
 * C [I, J] = bf16(sum_k A[i][k] B[j][k]), bf16 operands, fp32 accumulation,
 * round to nearest even.  Operand layouts (no transposed copies needed):
 *   layout 0  contraction-major: A[i][k] at a[i * K + k]  (B: b[j * K + k])
 *   layout 1  output-major:      A[i][k] at a[k * I + i]  (B: b[k * J + j])
 * I, J, K positive multiples of 128; pointers 16-byte aligned; ws holds the
 * split-K partial sums (fp8_bf16_gemm_workspace_bytes; 0 when none).
 */
size_t fp8_bf16_gemm_workspace_bytes(int64_t I, int64_t J, int64_t K);
fp8_status fp8_bf16_gemm(const void* a_bf16, int a_layout, const void* b_bf16, int b_layout,
                         int64_t I, int64_t J, int64_t K, void* c_bf16, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * BF16 linear: forward Y [N, M] = X [N, K] W [M, K]^T; backward dX [N, K] =
 * dY W (W read output-major) and dW [M, K] = dY^T X (both read output-major);
 * dx or dw may be NULL to skip that product.  Workspace from
 * fp8_bf16_linear_workspace_bytes (covers all three products).
 */
size_t fp8_bf16_linear_workspace_bytes(int64_t N, int64_t K, int64_t M);
fp8_status fp8_bf16_linear_fwd(const void* x_bf16, const void* w_bf16, int64_t N, int64_t K, int64_t M,
                               void* y_bf16, void* ws, size_t ws_bytes, void* stream);
fp8_status fp8_bf16_linear_bwd(const void* dy_bf16, const void* x_bf16, const void* w_bf16,
                               int64_t N, int64_t K, int64_t M, void* dx_bf16, void* dw_bf16,
                               void* ws, size_t ws_bytes, void* stream);

/* ------------------- forward without any allocation ------------------ */

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * forward pass exactly as fp8_linear_fwd (same kernels, bitwise the same
 * Y, saved_x and quantized weight), with no workspace argument.  Its scratch
 * (the amax partials of X and W, and the forward GEMM's split-K partials) is
 * a device array of FP8_NOALLOC_SCRATCH_BYTES that the library holds on each
 * GPU it runs on until the process ends; nothing is allocated, and nothing
 * in it needs clearing (every call writes what it reads).
 *  - A shape whose forward needs more scratch than that (a short output
 *    whose GEMM would split a long contraction into large partial sums)
 *    gives FP8_ERR_WORKSPACE before anything is enqueued; fp8_linear_fwd
 *    with a workspace serves it.
 *  - All calls on one GPU share that GPU's array: calls that may overlap on
 *    one GPU (different streams, different threads) race and give undefined
 *    results; order them (one stream, or events).
 *  - The first call on a device looks up that device's copy of the array
 *    (hipGetSymbolAddress); a failure there gives FP8_ERR_HIP.
 * Arguments as fp8_linear_fwd without (ws, ws_bytes).
 */
#define FP8_NOALLOC_SCRATCH_BYTES (8u << 20)
fp8_status fp8_linear_fwd_noalloc(const void* x_bf16, const void* w_bf16,
                                  int64_t N, int64_t K, int64_t M, fp8_recipe recipe,
                                  fp8_wcache cache, int is_first_microbatch,
                                  void* y_bf16, const fp8_qtensor* saved_x, const fp8_qtensor* w_q,
                                  const void* x_amax_partials, void* y_amax_partials, void* stream);

/* ----------------------- GELU in an MLP block ------------------------ */

/*
 * The MLP block of the pages' workload (512 -> 2048 -> 512 linears with GELU
 * between them, as in "Native FP8 MLP reconstruction", where the MLP linears
 * are the ones run in FP8) needs GELU on the up projection's output and
 * GELU's derivative on the way back.  The exact (erf) form is used:
 *   GELU(x) = x Phi(x),  GELU'(x) = Phi(x) + x phi(x)
 * (Phi, phi the standard normal CDF and density), each rounded once to fp32
 * from an fp64 evaluation.  The activation is bf16(fl32(GELU(x))), the
 * gradient through GELU bf16(fl32(dy * fl32(GELU'(x)))) (one fp32 multiply),
 * both rounded to nearest even; every NaN result is the quiet NaN 0x7FC0
 * (GELU(-Inf) = -Inf * 0 is one, so is GELU' of either infinity).
 *
 * The values come from tables of both functions over the bf16 inputs, built
 * on each device the first time one of these functions runs there: that
 * call waits for the tables (on a stream of its own) and fails with
 * FP8_ERR_HIP if its stream is being captured into a graph.  Later calls
 * enqueue only.
 */

/* y [n] = GELU(x [n]), bf16 in and out; n a multiple of 8 (FP8_ERR_SHAPE),
 * pointers 16-byte aligned.  The unfused form, for comparison and for a
 * caller that needs the activation in bf16. */
fp8_status fp8_gelu(const void* x_bf16, void* y_bf16, int64_t n, void* stream);

/* dx [n] = dGELU(dy [n], x [n]): dy the gradient of GELU's output, x GELU's
 * input; bf16 in and out, n a multiple of 8. */
fp8_status fp8_dgelu(const void* dy_bf16, const void* x_bf16, void* dx_bf16, int64_t n, void* stream);

/*
 * Quantize GELU(x) [rows, cols] exactly as fp8_quantize would quantize the
 * bf16 activation, without writing the activation out: the bytes and scales
 * are identical to fp8_gelu followed by fp8_quantize.  scaling is
 * FP8_SCALE_TENSOR (two passes over x: amax, then the cast) or
 * FP8_SCALE_BLOCK_1x128 (one pass); FP8_ERR_ENUM otherwise.  Workspace and
 * the other arguments as fp8_quantize.
 */
fp8_status fp8_quantize_gelu(const void* x_bf16, int64_t rows, int64_t cols, fp8_format format,
                             fp8_scaling scaling, unsigned layouts, const fp8_qtensor* out,
                             void* ws, size_t ws_bytes, void* stream);

/* Quantize dGELU(dy, x) [rows, cols] likewise (identical to fp8_dgelu
 * followed by fp8_quantize); x is 16-byte aligned and has dy's shape. */
fp8_status fp8_quantize_dgelu(const void* dy_bf16, const void* x_bf16, int64_t rows, int64_t cols,
                              fp8_format format, fp8_scaling scaling, unsigned layouts,
                              const fp8_qtensor* out, void* ws, size_t ws_bytes, void* stream);

/*
 * The second linear of an MLP block: fp8_linear_fwd with X = GELU(x_pre),
 * x_pre [N, K] the first linear's output.  X's quantize applies GELU as it
 * reads x_pre; saved_x holds X's codes (and scales), exactly what
 * fp8_linear_fwd gives for X = fp8_gelu(x_pre).  No X amax hand-off; the
 * other arguments as fp8_linear_fwd.
 */
fp8_status fp8_linear_fwd_gelu(const void* x_pre_bf16, const void* w_bf16,
                               int64_t N, int64_t K, int64_t M, fp8_recipe recipe,
                               fp8_wcache cache, int is_first_microbatch,
                               void* y_bf16, const fp8_qtensor* saved_x, const fp8_qtensor* w_q,
                               void* y_amax_partials, void* ws, size_t ws_bytes, void* stream);

/*
 * The first linear of an MLP block, backward: fp8_linear_bwd with the
 * incoming gradient dY = dGELU(dh, y_pre), dh [N, M] the gradient of GELU's
 * output and y_pre [N, M] GELU's input (this linear's forward output).  dY's
 * quantize applies dGELU as it reads both; the results equal fp8_linear_bwd
 * on dY = fp8_dgelu(dh, y_pre).  No dY amax hand-off; the other arguments as
 * fp8_linear_bwd.
 */
fp8_status fp8_linear_bwd_dgelu(const void* dh_bf16, const void* y_pre_bf16, int64_t N, int64_t K,
                                int64_t M, fp8_recipe recipe, const fp8_qtensor* saved_x,
                                fp8_wcache cache, const fp8_qtensor* w_q, const fp8_qtensor* dy_q,
                                void* dx_bf16, void* dw_bf16, void* dx_amax_partials,
                                void* ws, size_t ws_bytes, void* stream);

/* ------------------------------- misc -------------------------------- */

const char* fp8_status_string(fp8_status status);
/* Message of the calling thread's most recent failure ("" if none). */
const char* fp8_last_error(void);
/* Library version string. */
const char* fp8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8_LINEAR_H */
