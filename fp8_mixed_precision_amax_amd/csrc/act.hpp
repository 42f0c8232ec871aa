// GELU and its derivative on bf16 inputs, for the activation between the two
// linears of an MLP block (the exact erf form: GELU(x) = x Phi(x), GELU'(x) =
// Phi(x) + x phi(x); Phi, phi the standard normal CDF and density).
//
// A bf16 input has 65536 possible values, so both functions are tables,
// computed once per device in fp64 and rounded once to fp32 (gelu.hip), and
// every element costs one LDS lookup.  The tables cover the inputs with
// 2^-40 <= |x| < 16 (exponent fields 87 .. 130: 44 binades of 128 mantissas,
// the positive half first).  Outside that range both functions have closed
// forms in fp32:
//   |x| < 2^-40    GELU(x) rounds to x / 2, GELU'(x) to 1/2
//   |x| >= 16      GELU(x) = x above 0 and rounds to -0 below; GELU'(x) is
//                  1 above 0 and rounds to -0 below
//   +-Inf, NaN     GELU(+Inf) = +Inf; GELU(-Inf), GELU(NaN) and GELU' of
//                  either infinity or NaN are NaN
// Results: the activation is bf16(fl32(GELU(x))) and the gradient through it
// bf16(fl32(dy * fl32(GELU'(x)))) (one fp32 multiply), both rounded to
// nearest even; every NaN result is the quiet NaN 0x7FC0.
//
// The fast path handles a pair of bf16 values with packed 16-bit index
// arithmetic and one hardware bf16 conversion; a wave whose elements are all
// inside the table (and, for dGELU, whose gradients are all finite) never
// runs the closed forms.
#pragma once

#include "device.hpp"

namespace fp8k {

constexpr uint32_t kActLo = 87u << 7;           // magnitude bits of 2^-40
constexpr uint32_t kActHalf = 44u * 128u;       // entries per sign
constexpr uint32_t kActEntries = 2u * kActHalf;


// Table indices of the two bf16 halves of w, clamped into the table; far
// receives the offsets from the table's start, >= kActHalf where a value lies
// outside it.
__device__ __forceinline__ us2_t act_index2(uint32_t w, us2_t& far) {
    const us2_t m = __builtin_bit_cast(us2_t, w & 0x7FFF7FFFu);
    const us2_t off = m - (us2_t){(unsigned short)kActLo, (unsigned short)kActLo};
    far = off;
    const us2_t sg = __builtin_bit_cast(us2_t, (w >> 15) & 0x00010001u);
    const us2_t top = {(unsigned short)(kActHalf - 1), (unsigned short)(kActHalf - 1)};
    return __builtin_elementwise_min(off, top) + sg * (us2_t){(unsigned short)kActHalf, (unsigned short)kActHalf};
}

__device__ __forceinline__ bool act_outside(uint32_t b) { return (b & 0x7FFFu) - kActLo >= kActHalf; }

// An opaque copy of v: the compiler cannot see how a table result was put
// together (otherwise it keeps the shifted high half alive as well, since
// the cast later needs exactly that fp32 pattern, doubling the registers the
// transformed data occupies).
__device__ __forceinline__ uint32_t act_opaque(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}

// Materialise v here: both arms of a select below are then computed
// unconditionally and the select stays a v_cndmask, instead of being turned
// into divergent branches with the table read sunk into one of them.
__device__ __forceinline__ uint32_t act_pin(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// GELU of one bf16 value b outside the table, as bf16 bits (selects, no
// branches).
__device__ __forceinline__ uint32_t gelu_closed(uint32_t b) {
    const uint32_t m = b & 0x7FFFu, s = b & 0x8000u;
    // x / 2: one exponent lower; from the smallest normal binade down the
    // halving shifts the subnormal significand, rounded to nearest even
    const uint32_t half = m >= 0x100u ? m - 0x80u : (m >> 1) + (m & (m >> 1) & 1u);
    uint32_t r = s | half;                                  // |x| < 2^-40
    r = m >= kActLo ? (s ? 0x8000u : b) : r;                // |x| >= 16: x, or -0
    r = m >= 0x7F80u ? (b == 0x7F80u ? 0x7F80u : 0x7FC0u) : r;   // +Inf; -Inf and NaN
    return r;
}

// GELU' of one bf16 value b outside the table.
__device__ __forceinline__ float dgelu_closed(uint32_t b) {
    const uint32_t m = b & 0x7FFFu;
    uint32_t r = 0x3F000000u;                                       // 1/2
    r = m >= kActLo ? ((b & 0x8000u) ? 0x80000000u : 0x3F800000u) : r;   // 1, or -0
    r = m >= 0x7F80u ? 0x7FC00000u : r;                              // NaN
    return __uint_as_float(r);
}

// bf16 GELU of one bf16 pattern b: the table (LDS or global), or the closed
// forms outside it.
__device__ __forceinline__ uint32_t gelu_one(uint32_t b, const uint16_t* tab) {
    if (((b & 0x7FFFu) - kActLo) >= kActHalf) return gelu_closed(b);
    return tab[((b & 0x7FFFu) - kActLo) + ((b & 0x8000u) ? kActHalf : 0u)];
}

// fp32 -> bf16 bits, round to nearest even; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t bf16_rne_canon(float v) {
    const uint32_t u = __float_as_uint(v);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// GELU of the 8 bf16 values of x from the table alone (values outside it
// get a wrong result); far accumulates the table offsets (>= kActHalf marks
// a value outside the table).
__device__ __forceinline__ uint4 gelu8_fast(uint4 x, const uint16_t* tab, us2_t& far) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t r[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        us2_t f;
        const us2_t idx = act_index2(w[k], f);
        far = __builtin_elementwise_max(far, f);
        r[k] = act_opaque((uint32_t)tab[idx.x] | ((uint32_t)tab[idx.y] << 16));
    }
    return make_uint4(r[0], r[1], r[2], r[3]);
}

// GELU of the 8 bf16 values of x, every value exact.
__device__ __forceinline__ uint4 gelu8_full(uint4 x, const uint16_t* tab) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t r[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint32_t lo = w[k] & 0xFFFFu, hi = w[k] >> 16;
        us2_t f;
        const us2_t idx = act_index2(w[k], f);
        // the table is read in bounds for every value (the index is clamped)
        const uint32_t tl = act_pin(tab[idx.x]), th = act_pin(tab[idx.y]);
        const uint32_t cl = act_pin(gelu_closed(lo)), ch = act_pin(gelu_closed(hi));
        const uint32_t rl = act_outside(lo) ? cl : tl;
        const uint32_t rh = act_outside(hi) ? ch : th;
        r[k] = act_opaque(rl | (rh << 16));
    }
    return make_uint4(r[0], r[1], r[2], r[3]);
}

// GELU of 8 values: the table, and the closed forms only in waves that need
// them.
__device__ __forceinline__ uint4 gelu8(uint4 x, const uint16_t* tab) {
    us2_t far = {0, 0};
    const uint4 r = gelu8_fast(x, tab, far);
    if (__ballot(hmax_u16(__builtin_bit_cast(uint32_t, far)) >= kActHalf)) return gelu8_full(x, tab);
    return r;
}

// dGELU of 8 elements, bf16(fl32(dy * GELU'(x))), from the table alone
// (exact when every x lies in the table and every dy is finite); far and
// dm accumulate the table offsets and the gradient magnitudes.
__device__ __forceinline__ uint4 dgelu8_fast(uint4 dy, uint4 x, const float* tab, us2_t& far, uint32_t& dm) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    const uint32_t d[4] = {dy.x, dy.y, dy.z, dy.w};
    uint32_t r[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        us2_t f;
        const us2_t idx = act_index2(w[k], f);
        far = __builtin_elementwise_max(far, f);
        dm = pkmax_u16(dm, mag2(d[k]));
        r[k] = act_opaque(pack_bf16x2(bf16_lo(d[k]) * tab[idx.x], bf16_hi(d[k]) * tab[idx.y]));
    }
    return make_uint4(r[0], r[1], r[2], r[3]);
}

// dGELU of 8 elements, every element exact (NaN results canonical).
__device__ __forceinline__ uint4 dgelu8_full(uint4 dy, uint4 x, const float* tab) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    const uint32_t d[4] = {dy.x, dy.y, dy.z, dy.w};
    uint32_t r[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint32_t lo = w[k] & 0xFFFFu, hi = w[k] >> 16;
        us2_t f;
        const us2_t idx = act_index2(w[k], f);
        // the table is read in bounds for every value (the index is clamped)
        const uint32_t tl = act_pin(__float_as_uint(tab[idx.x])), th = act_pin(__float_as_uint(tab[idx.y]));
        const uint32_t cl = act_pin(__float_as_uint(dgelu_closed(lo))), ch = act_pin(__float_as_uint(dgelu_closed(hi)));
        const float gl = __uint_as_float(act_outside(lo) ? cl : tl);
        const float gh = __uint_as_float(act_outside(hi) ? ch : th);
        const uint32_t pl = act_pin(bf16_rne_canon(bf16_lo(d[k]) * gl));
        const uint32_t ph = act_pin(bf16_rne_canon(bf16_hi(d[k]) * gh));
        r[k] = act_opaque(pl | (ph << 16));
    }
    return make_uint4(r[0], r[1], r[2], r[3]);
}

// True (wave-uniform) if any lane saw a value outside the table or, with
// dm, a non-finite gradient (the only way to a NaN product): such waves
// take the exact path.
__device__ __forceinline__ bool act_need_full(us2_t far, uint32_t dm = 0) {
    return __ballot(hmax_u16(__builtin_bit_cast(uint32_t, far)) >= kActHalf || hmax_u16(dm) >= 0x7F80u) != 0;
}

__device__ __forceinline__ uint4 dgelu8(uint4 dy, uint4 x, const float* tab) {
    us2_t far = {0, 0};
    uint32_t dm = 0;
    const uint4 r = dgelu8_fast(dy, x, tab, far, dm);
    if (act_need_full(far, dm)) return dgelu8_full(dy, x, tab);
    return r;
}

// Cooperative copy of a table (bytes a multiple of 16) from global memory to
// LDS by the whole workgroup; the caller synchronises.
__device__ __forceinline__ void act_table_to_lds(void* lds, const void* g, uint32_t bytes) {
    const uint4* src = static_cast<const uint4*>(g);
    uint4* dst = static_cast<uint4*>(lds);
    for (uint32_t i = threadIdx.x; i < bytes / 16; i += blockDim.x) dst[i] = src[i];
}

}  // namespace fp8k
