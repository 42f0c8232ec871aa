/*
 * CPU oracle for the FP8 linear layer (forward and backward) with current
 * amax scaling.  TEST INFRASTRUCTURE ONLY: nothing on the product path may
 * link, load or call this file.  It shares no code, header, table or
 * constant generator with the HIP library; it is written from the method's
 * description and from the OCP 8-bit floating point format definition.
 *
 * Sources followed (page titles as published):
 *  - "Native FP8 MLP reconstruction" (rstation.ai, general_pretraining post 23),
 *    implementation paragraph: every tensor's scale is set from its amax on
 *    the call that uses it; X and W are coded as E4M3 and dY as E5M2; the
 *    GEMMs sum in fp32 (no fast accumulation) and write BF16; one cast pass
 *    yields both the row-major codes and their transpose; the backward pass
 *    treats the scales as constants, takes the X and W codes of the forward
 *    pass and quantizes dY by itself.
 *  - "FP8 weight caching shows no speedup (sometimes slowdown) and causes
 *    training curve differences under Float8BlockScaling" (TransformerEngine
 *    issue 2852), opening post and maintainer reply: block-scaled (non-delayed)
 *    quantization, and weight caching that must give the same result as
 *    re-quantizing the weight every microbatch.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - OCP E4M3 ("E4M3FN": no infinities, NaN = S.1111.111, max 448) and OCP
 *    E5M2 (IEEE-like, max 57344).
 *  - scale = FMAX / amax as one IEEE fp32 division, scale_inv = 1 / scale;
 *    amax that is 0, +Inf or NaN gives scale 1; an overflowing scale is
 *    clamped to FLT_MAX.
 *  - element code = encode(fl32(x * scale)): an fp32 multiply, then a
 *    saturating round-to-nearest-even encode (NaN -> 0x7F, |v| >= FMAX ->
 *    +-FMAX code, signed zero kept).
 *  - blocks: 1x128 along the contraction dimension of the GEMM that consumes
 *    each layout; 128x128 tiles for weights.
 *  - GEMMs accumulate in fp32 with k ascending; tensorwise epilogue is
 *    bf16(fl32(acc * fl32(sinvA * sinvB))); block mode promotes every
 *    128-long contraction block: acc = fl32(acc + fl32(p * fl32(sa * sb))).
 *  - the GELU between an MLP block's two linears is the exact (erf) form,
 *    GELU and GELU' each rounded once to fp32 from an fp64 evaluation; the
 *    activation is bf16(fl32(GELU(x))), the gradient through it
 *    bf16(fl32(dy * fl32(GELU'(x)))); NaN results are the quiet NaN 0x7FC0.
 *  - the BF16 comparator linear (the pages' baseline) multiplies bf16
 *    operands exactly, sums in fp32 with k ascending and rounds to bf16.
 *
 * Compile with -O2 -ffp-contract=off (no fused multiply-add, no fast-math).
 * Parity status: every function below is pinned by the CPU test-suite
 * (exhaustive code tables, brute-force encoders, exact integer GEMMs,
 * closed-form invariants, 45-digit evaluations of GELU and GELU' at every
 * bf16 input); none is "parity unpinned".
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* OCP FP8 formats                                                     */
/* ------------------------------------------------------------------ */

enum { ORC_E4M3 = 0, ORC_E5M2 = 1 };

typedef struct {
    int ebits;         /* exponent field width */
    int mbits;         /* mantissa field width */
    int bias;          /* exponent bias */
    double fmax;       /* largest finite magnitude */
    uint8_t fmax_code; /* code of +fmax */
} orc_fmt;

static orc_fmt fmt_of(int f) {
    orc_fmt r;
    if (f == ORC_E4M3) {
        r.ebits = 4; r.mbits = 3; r.bias = 7; r.fmax = 448.0; r.fmax_code = 0x7E;
    } else {
        r.ebits = 5; r.mbits = 2; r.bias = 15; r.fmax = 57344.0; r.fmax_code = 0x7B;
    }
    return r;
}

float orc_fmax(int f) { return (float)fmt_of(f).fmax; }

/* Value of an FP8 code, from the field definition of the format. */
float orc_dec(uint8_t code, int f) {
    orc_fmt F = fmt_of(f);
    int sign = (code >> 7) & 1;
    int e = (code >> F.mbits) & ((1 << F.ebits) - 1);
    int m = code & ((1 << F.mbits) - 1);
    int emax_field = (1 << F.ebits) - 1;
    double v;
    if (f == ORC_E4M3 && e == emax_field && m == (1 << F.mbits) - 1)
        return NAN;                                  /* S.1111.111 */
    if (f == ORC_E5M2 && e == emax_field)
        return m == 0 ? (sign ? -INFINITY : INFINITY) : NAN;
    if (e == 0)
        v = (double)m * ldexp(1.0, 1 - F.bias - F.mbits);          /* subnormal */
    else
        v = (1.0 + (double)m / (double)(1 << F.mbits)) * ldexp(1.0, e - F.bias);
    return (float)(sign ? -v : v);
}

/* Round a non-negative real (held exactly in a double) to an integer,
 * ties to even. */
static double round_half_even(double m) {
    double fl = floor(m);
    double frac = m - fl;
    if (frac > 0.5) return fl + 1.0;
    if (frac < 0.5) return fl;
    return fmod(fl, 2.0) == 0.0 ? fl : fl + 1.0;
}

/* Saturating round-to-nearest-even encode of an fp32 value. */
uint8_t orc_enc(float v, int f) {
    orc_fmt F = fmt_of(f);
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= F.fmax) return sign | F.fmax_code;      /* saturation, Inf included */
    if (a == 0.0) return sign;
    int emin = 1 - F.bias;                           /* exponent of the smallest normal */
    int e;
    frexp(a, &e);
    e -= 1;                                          /* a in [2^e, 2^(e+1)) */
    if (e < emin) e = emin;                          /* gradual underflow: fixed quantum */
    double quantum = ldexp(1.0, e - F.mbits);        /* spacing of codes in this binade */
    double r = round_half_even(a / quantum);         /* a / quantum is exact in double */
    double val = r * quantum;                        /* never above fmax (a < fmax) */
    if (val == 0.0) return sign;
    int ev;
    frexp(val, &ev);
    ev -= 1;
    if (ev < emin)                                   /* subnormal code */
        return sign | (uint8_t)(val / ldexp(1.0, emin - F.mbits));
    int efield = ev + F.bias;
    int mfield = (int)((val / ldexp(1.0, ev) - 1.0) * (double)(1 << F.mbits));
    return sign | (uint8_t)(efield << F.mbits) | (uint8_t)mfield;
}

void orc_enc_array(const float* v, int64_t n, int f, uint8_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = orc_enc(v[i], f);
}

void orc_dec_array(const uint8_t* c, int64_t n, int f, float* out) {
    for (int64_t i = 0; i < n; i++) out[i] = orc_dec(c[i], f);
}

/* ------------------------------------------------------------------ */
/* BF16                                                                */
/* ------------------------------------------------------------------ */

static float f32_from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

/* bf16 is the upper half of an fp32 bit pattern. */
float orc_dec_bf16(uint16_t b) { return f32_from_bits((uint32_t)b << 16); }

/* fp32 -> bf16, round to nearest even on the 16 dropped bits; NaN stays a
 * quiet NaN of the same sign. */
uint16_t orc_bf16_rne(float v) {
    uint32_t b = bits_from_f32(v);
    if (isnan(v)) return (uint16_t)((b >> 16) | 0x0040);
    uint32_t keep_lsb = (b >> 16) & 1u;
    b += 0x7FFFu + keep_lsb;
    return (uint16_t)(b >> 16);
}

void orc_bf16_rne_array(const float* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; i++) out[i] = orc_bf16_rne(v[i]);
}

/* ------------------------------------------------------------------ */
/* amax and scale (current scaling)                                    */
/* ------------------------------------------------------------------ */

/* max |x| over a bf16 tensor; NaN if any element is NaN. */
float orc_amax_bf16(const uint16_t* x, int64_t n) {
    float m = 0.0f;
    for (int64_t i = 0; i < n; i++) {
        float a = fabsf(orc_dec_bf16(x[i]));
        if (isnan(a)) return NAN;
        if (a > m) m = a;
    }
    return m;
}

/* Strided amax: n elements at x[0], x[stride], ... */
static float amax_strided(const uint16_t* x, int64_t n, int64_t stride) {
    float m = 0.0f;
    for (int64_t i = 0; i < n; i++) {
        float a = fabsf(orc_dec_bf16(x[i * stride]));
        if (isnan(a)) return NAN;
        if (a > m) m = a;
    }
    return m;
}

void orc_scale_from_amax(float amax, int f, float* scale, float* scale_inv) {
    float fmax = orc_fmax(f);
    float s;
    if (isnan(amax) || isinf(amax) || amax == 0.0f) {
        s = 1.0f;
    } else {
        s = fmax / amax;
        if (isinf(s)) s = FLT_MAX;
    }
    *scale = s;
    *scale_inv = 1.0f / s;
}

static uint8_t quant_elem(uint16_t x, float s, int f) {
    float p = orc_dec_bf16(x) * s;                  /* one fp32 rounding */
    return orc_enc(p, f);                           /* then the encode */
}

/* ------------------------------------------------------------------ */
/* Quantizers.  x is row-major [R, C] bf16.  q_row is [R, C], q_col is  */
/* [C, R] (the transposed layout).  Either output pointer may be NULL.  */
/* ------------------------------------------------------------------ */

void orc_quant_tensor(const uint16_t* x, int64_t R, int64_t C, int f,
                      uint8_t* q_row, uint8_t* q_col,
                      float* amax_out, float* scale_out, float* sinv_out) {
    float amax = orc_amax_bf16(x, R * C);
    float s, si;
    orc_scale_from_amax(amax, f, &s, &si);
    if (amax_out) *amax_out = amax;
    *scale_out = s;
    *sinv_out = si;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; r++)
        for (int64_t c = 0; c < C; c++) {
            uint8_t q = quant_elem(x[r * C + c], s, f);
            if (q_row) q_row[r * C + c] = q;
            if (q_col) q_col[c * R + r] = q;
        }
}

/* Delayed tensorwise scaling with an amax history (the DelayedScaling case
 * the weight-caching issue contrasts with block scaling: TransformerEngine
 * issue 2852, opening post and question 3).  Readings (not on the pages):
 * hist[0..H-1] holds the amaxes of the tensor's previous quantize calls, most
 * recent first; the scale comes from the largest of them (NaN if any is NaN),
 * by the same rules as current scaling; then this call's amax is pushed in
 * front and the oldest entry dropped.  A history of zeros gives scale 1. */
void orc_quant_delayed(const uint16_t* x, int64_t R, int64_t C, int f, float* hist, int64_t H,
                       uint8_t* q_row, uint8_t* q_col,
                       float* amax_out, float* scale_out, float* sinv_out) {
    float hmax = 0.0f;
    for (int64_t i = 0; i < H; i++) {
        if (isnan(hist[i])) { hmax = NAN; break; }
        if (hist[i] > hmax) hmax = hist[i];
    }
    float s, si;
    orc_scale_from_amax(hmax, f, &s, &si);
    *scale_out = s;
    *sinv_out = si;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; r++)
        for (int64_t c = 0; c < C; c++) {
            uint8_t q = quant_elem(x[r * C + c], s, f);
            if (q_row) q_row[r * C + c] = q;
            if (q_col) q_col[c * R + r] = q;
        }
    float amax = orc_amax_bf16(x, R * C);
    if (amax_out) *amax_out = amax;
    for (int64_t i = H - 1; i > 0; i--) hist[i] = hist[i - 1];
    hist[0] = amax;
}

/* 1x128 blocks.  Row layout: one block per (row r, 128 columns), scales
 * s_row[R][C/128].  Col layout: one block per (column c, 128 rows), scales
 * s_col[C][R/128]; q_col[c][r] uses the scale of block (c, r/128). */
void orc_quant_block_1x128(const uint16_t* x, int64_t R, int64_t C, int f,
                           uint8_t* q_row, float* s_row, float* sinv_row,
                           uint8_t* q_col, float* s_col, float* sinv_col) {
    int64_t CB = C / 128, RB = R / 128;
    if (q_row) {
        #pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < R; r++)
            for (int64_t cb = 0; cb < CB; cb++) {
                const uint16_t* blk = x + r * C + cb * 128;
                float s, si;
                orc_scale_from_amax(amax_strided(blk, 128, 1), f, &s, &si);
                s_row[r * CB + cb] = s;
                sinv_row[r * CB + cb] = si;
                for (int64_t j = 0; j < 128; j++)
                    q_row[r * C + cb * 128 + j] = quant_elem(blk[j], s, f);
            }
    }
    if (q_col) {
        #pragma omp parallel for schedule(static)
        for (int64_t c = 0; c < C; c++)
            for (int64_t rb = 0; rb < RB; rb++) {
                const uint16_t* blk = x + rb * 128 * C + c;   /* column c, rows rb*128.. */
                float s, si;
                orc_scale_from_amax(amax_strided(blk, 128, C), f, &s, &si);
                s_col[c * RB + rb] = s;
                sinv_col[c * RB + rb] = si;
                for (int64_t j = 0; j < 128; j++)
                    q_col[c * R + rb * 128 + j] = quant_elem(blk[j * C], s, f);
            }
    }
}

/* 128x128 blocks, scales s[R/128][C/128]; the col layout is the transpose
 * of the row layout and uses the same scales. */
void orc_quant_block_128x128(const uint16_t* x, int64_t R, int64_t C, int f,
                             uint8_t* q_row, uint8_t* q_col, float* s_blk, float* sinv_blk) {
    int64_t CB = C / 128, RB = R / 128;
    #pragma omp parallel for schedule(static)
    for (int64_t rb = 0; rb < RB; rb++)
        for (int64_t cb = 0; cb < CB; cb++) {
            float m = 0.0f;
            int nan = 0;
            for (int64_t i = 0; i < 128; i++) {
                float a = amax_strided(x + (rb * 128 + i) * C + cb * 128, 128, 1);
                if (isnan(a)) nan = 1;
                else if (a > m) m = a;
            }
            float s, si;
            orc_scale_from_amax(nan ? NAN : m, f, &s, &si);
            s_blk[rb * CB + cb] = s;
            sinv_blk[rb * CB + cb] = si;
            for (int64_t i = 0; i < 128; i++)
                for (int64_t j = 0; j < 128; j++) {
                    int64_t r = rb * 128 + i, c = cb * 128 + j;
                    uint8_t q = quant_elem(x[r * C + c], s, f);
                    if (q_row) q_row[r * C + c] = q;
                    if (q_col) q_col[c * R + r] = q;
                }
        }
}

/* ------------------------------------------------------------------ */
/* GELU between the two linears of an MLP block.  The pages name no     */
/* formula; the exact (erf) GELU is read:                               */
/*   GELU(x)  = x Phi(x),  Phi(x) = erfc(-x / sqrt 2) / 2               */
/*   GELU'(x) = Phi(x) + x phi(x),  phi(x) = exp(-x^2 / 2) / sqrt(2 pi) */
/* each evaluated in fp64 and rounded once to fp32.  The activation     */
/* passed on is bf16(fl32(GELU(x))); the gradient passed back is        */
/* bf16(fl32(dy * fl32(GELU'(x)))), one fp32 multiply.  Every NaN result */
/* is the canonical quiet NaN 0x7FC0 (GELU(-Inf) = -Inf * 0 is one).    */
/* ------------------------------------------------------------------ */

static const double ORC_SQRT1_2 = 0.70710678118654752440;       /* 1 / sqrt(2) */
static const double ORC_INV_SQRT_2PI = 0.39894228040143267794;  /* 1 / sqrt(2 pi) */

float orc_gelu_f32(uint16_t x) {
    double a = (double)orc_dec_bf16(x);
    double phi_cdf = 0.5 * erfc(-a * ORC_SQRT1_2);
    return (float)(a * phi_cdf);
}

float orc_gelu_grad_f32(uint16_t x) {
    double a = (double)orc_dec_bf16(x);
    double phi_cdf = 0.5 * erfc(-a * ORC_SQRT1_2);
    double phi_pdf = exp(-0.5 * a * a) * ORC_INV_SQRT_2PI;
    double g = phi_cdf + a * phi_pdf;
    /* below x = -38 both terms underflow in fp64 and their sum is +0; the
     * exact value is negative there (x phi(x) dominates), so it rounds to -0 */
    if (g == 0.0 && a < 0.0) g = -0.0;
    return (float)g;
}

static uint16_t bf16_canon(float v) { return isnan(v) ? (uint16_t)0x7FC0 : orc_bf16_rne(v); }

void orc_gelu_array(const uint16_t* x, int64_t n, uint16_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = bf16_canon(orc_gelu_f32(x[i]));
}

void orc_gelu_f32_array(const uint16_t* x, int64_t n, float* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = orc_gelu_f32(x[i]);
}

void orc_gelu_grad_f32_array(const uint16_t* x, int64_t n, float* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = orc_gelu_grad_f32(x[i]);
}

void orc_dgelu_array(const uint16_t* dy, const uint16_t* x, int64_t n, uint16_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        float p = orc_dec_bf16(dy[i]) * orc_gelu_grad_f32(x[i]);   /* one fp32 rounding */
        out[i] = bf16_canon(p);
    }
}

/* ------------------------------------------------------------------ */
/* GEMMs.  C[i][j] = sum_k A[i][k] * B[j][k]; A is [I, K], B is [J, K],  */
/* both K-contiguous FP8 codes; C is [I, J] bf16 (and optionally fp32).  */
/* ------------------------------------------------------------------ */

static void decode_matrix(const uint8_t* q, int64_t n, int f, float* out) {
    float table[256];
    for (int c = 0; c < 256; c++) table[c] = orc_dec((uint8_t)c, f);
    for (int64_t i = 0; i < n; i++) out[i] = table[q[i]];
}

/* Tensorwise scaling.  Each output sums its K products in ascending k with
 * one fp32 add per product (the products of two FP8 values are exact in
 * fp32).  The loop order is i, k, j so that the inner loop runs over j;
 * every C[i][j] still receives its products in ascending k.
 * work: caller-provided fp32 scratch of (I + J) * K floats. */
void orc_gemm_tensor(const uint8_t* A, int fa, const uint8_t* B, int fb,
                     int64_t I, int64_t J, int64_t K, float sinvA, float sinvB,
                     uint16_t* C, float* C32, float* work) {
    float* Ad = work;                   /* [I, K] */
    float* Bt = work + I * K;           /* [K, J]: B transposed */
    decode_matrix(A, I * K, fa, Ad);
    {
        float table[256];
        for (int c = 0; c < 256; c++) table[c] = orc_dec((uint8_t)c, fb);
        for (int64_t j = 0; j < J; j++)
            for (int64_t k = 0; k < K; k++) Bt[k * J + j] = table[B[j * K + k]];
    }
    float t = sinvA * sinvB;
    #pragma omp parallel
    {
        float* acc = (float*)malloc(sizeof(float) * (size_t)J);
        #pragma omp for schedule(static)
        for (int64_t i = 0; i < I; i++) {
            for (int64_t j = 0; j < J; j++) acc[j] = 0.0f;
            for (int64_t k = 0; k < K; k++) {
                float a = Ad[i * K + k];
                const float* brow = Bt + k * J;
                for (int64_t j = 0; j < J; j++) acc[j] += a * brow[j];
            }
            for (int64_t j = 0; j < J; j++) {
                float y = acc[j] * t;
                if (C32) C32[i * J + j] = y;
                C[i * J + j] = orc_bf16_rne(y);
            }
        }
        free(acc);
    }
}

/* Block-scale lookup: the scale of operand row r in contraction block kb is
 * s[(r / group) * stride_r + kb * stride_kb]; group is 1 (1x128 blocks) or
 * 128 (128x128 blocks). */
static float bscale_at(const float* s, int64_t group, int64_t stride_r, int64_t stride_kb,
                       int64_t r, int64_t kb) {
    return s[(r / group) * stride_r + kb * stride_kb];
}

/* Block scaling: for each 128-long contraction block kb, p = sum over the
 * block (fp32, ascending k, starting from zero), then
 * acc = fl32(acc + fl32(p * fl32(sa * sb))); C = bf16(acc). */
void orc_gemm_block(const uint8_t* A, int fa, const float* sA, int64_t gA, int64_t srA, int64_t skA,
                    const uint8_t* B, int fb, const float* sB, int64_t gB, int64_t srB, int64_t skB,
                    int64_t I, int64_t J, int64_t K, uint16_t* C, float* C32, float* work) {
    float* Ad = work;
    float* Bt = work + I * K;
    decode_matrix(A, I * K, fa, Ad);
    {
        float table[256];
        for (int c = 0; c < 256; c++) table[c] = orc_dec((uint8_t)c, fb);
        for (int64_t j = 0; j < J; j++)
            for (int64_t k = 0; k < K; k++) Bt[k * J + j] = table[B[j * K + k]];
    }
    int64_t KB = K / 128;
    #pragma omp parallel
    {
        float* acc = (float*)malloc(sizeof(float) * (size_t)J);
        float* p = (float*)malloc(sizeof(float) * (size_t)J);
        #pragma omp for schedule(static)
        for (int64_t i = 0; i < I; i++) {
            for (int64_t j = 0; j < J; j++) acc[j] = 0.0f;
            for (int64_t kb = 0; kb < KB; kb++) {
                for (int64_t j = 0; j < J; j++) p[j] = 0.0f;
                for (int64_t k = kb * 128; k < kb * 128 + 128; k++) {
                    float a = Ad[i * K + k];
                    const float* brow = Bt + k * J;
                    for (int64_t j = 0; j < J; j++) p[j] += a * brow[j];
                }
                float sa = bscale_at(sA, gA, srA, skA, i, kb);
                for (int64_t j = 0; j < J; j++) {
                    float t = sa * bscale_at(sB, gB, srB, skB, j, kb);
                    float pt = p[j] * t;
                    acc[j] = acc[j] + pt;
                }
            }
            for (int64_t j = 0; j < J; j++) {
                if (C32) C32[i * J + j] = acc[j];
                C[i * J + j] = orc_bf16_rne(acc[j]);
            }
        }
        free(acc);
        free(p);
    }
}

/* Sampled outputs for large shapes: out[n] = C[ii[n]][jj[n]], computed as a
 * plain dot product in ascending k (same arithmetic as the full GEMMs). */
void orc_gemm_tensor_sampled(const uint8_t* A, int fa, const uint8_t* B, int fb, int64_t K,
                             float sinvA, float sinvB, const int64_t* ii, const int64_t* jj,
                             int64_t n, uint16_t* out, float* out32) {
    float ta[256], tb[256];
    for (int c = 0; c < 256; c++) { ta[c] = orc_dec((uint8_t)c, fa); tb[c] = orc_dec((uint8_t)c, fb); }
    float t = sinvA * sinvB;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n_ = 0; n_ < n; n_++) {
        const uint8_t* a = A + ii[n_] * K;
        const uint8_t* b = B + jj[n_] * K;
        float acc = 0.0f;
        for (int64_t k = 0; k < K; k++) acc += ta[a[k]] * tb[b[k]];
        float y = acc * t;
        if (out32) out32[n_] = y;
        out[n_] = orc_bf16_rne(y);
    }
}

void orc_gemm_block_sampled(const uint8_t* A, int fa, const float* sA, int64_t gA, int64_t srA, int64_t skA,
                            const uint8_t* B, int fb, const float* sB, int64_t gB, int64_t srB, int64_t skB,
                            int64_t K, const int64_t* ii, const int64_t* jj, int64_t n,
                            uint16_t* out, float* out32) {
    float ta[256], tb[256];
    for (int c = 0; c < 256; c++) { ta[c] = orc_dec((uint8_t)c, fa); tb[c] = orc_dec((uint8_t)c, fb); }
    int64_t KB = K / 128;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n_ = 0; n_ < n; n_++) {
        int64_t i = ii[n_], j = jj[n_];
        const uint8_t* a = A + i * K;
        const uint8_t* b = B + j * K;
        float acc = 0.0f;
        for (int64_t kb = 0; kb < KB; kb++) {
            float p = 0.0f;
            for (int64_t k = kb * 128; k < kb * 128 + 128; k++) p += ta[a[k]] * tb[b[k]];
            float t = bscale_at(sA, gA, srA, skA, i, kb) * bscale_at(sB, gB, srB, skB, j, kb);
            float pt = p * t;
            acc = acc + pt;
        }
        if (out32) out32[n_] = acc;
        out[n_] = orc_bf16_rne(acc);
    }
}

/* ------------------------------------------------------------------ */
/* BF16 comparator GEMM (the pages' baseline, "Native FP8 MLP           */
/* reconstruction", isolated-linear table: the same linears in BF16).   */
/* C[i][j] = bf16_rne(sum_k A[i][k] * B[j][k]), A [I, K] and B [J, K]    */
/* bf16 bit patterns, both K-contiguous; every product of two bf16       */
/* values is exact in fp32 (8-bit significands), and the sum runs in    */
/* fp32 with k ascending, one add per product.                          */
/* work: caller-provided fp32 scratch of (I + J) * K floats.            */
/* ------------------------------------------------------------------ */

void orc_gemm_bf16(const uint16_t* A, const uint16_t* B, int64_t I, int64_t J, int64_t K,
                   uint16_t* C, float* C32, float* work) {
    float* Ad = work;                   /* [I, K] */
    float* Bt = work + I * K;           /* [K, J]: B transposed */
    for (int64_t i = 0; i < I * K; i++) Ad[i] = orc_dec_bf16(A[i]);
    for (int64_t j = 0; j < J; j++)
        for (int64_t k = 0; k < K; k++) Bt[k * J + j] = orc_dec_bf16(B[j * K + k]);
    #pragma omp parallel
    {
        float* acc = (float*)malloc(sizeof(float) * (size_t)J);
        #pragma omp for schedule(static)
        for (int64_t i = 0; i < I; i++) {
            for (int64_t j = 0; j < J; j++) acc[j] = 0.0f;
            for (int64_t k = 0; k < K; k++) {
                float a = Ad[i * K + k];
                const float* brow = Bt + k * J;
                for (int64_t j = 0; j < J; j++) acc[j] += a * brow[j];
            }
            for (int64_t j = 0; j < J; j++) {
                if (C32) C32[i * J + j] = acc[j];
                C[i * J + j] = orc_bf16_rne(acc[j]);
            }
        }
        free(acc);
    }
}

/* Sampled outputs of the same GEMM: out[n] = C[ii[n]][jj[n]]. */
void orc_gemm_bf16_sampled(const uint16_t* A, const uint16_t* B, int64_t K, const int64_t* ii,
                           const int64_t* jj, int64_t n, uint16_t* out, float* out32) {
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n_ = 0; n_ < n; n_++) {
        const uint16_t* a = A + ii[n_] * K;
        const uint16_t* b = B + jj[n_] * K;
        float acc = 0.0f;
        for (int64_t k = 0; k < K; k++) acc += orc_dec_bf16(a[k]) * orc_dec_bf16(b[k]);
        if (out32) out32[n_] = acc;
        out[n_] = orc_bf16_rne(acc);
    }
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
    omp_set_num_threads(n);
#else
    (void)n;
#endif
}
