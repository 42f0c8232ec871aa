// Device helpers for gfx950 (CDNA4): bf16 unpacking, saturating FP8 packing
// on the hardware converters, wave reductions and DPP row reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8k {

// OCP FP8 limits.  E4M3 ("FN") saturates at 448, E5M2 at 57344.
template <int FMT> struct FmtTraits;
template <> struct FmtTraits<0> { static constexpr float fmax = 448.0f; };
template <> struct FmtTraits<1> { static constexpr float fmax = 57344.0f; };

// Streaming (non-temporal) 16/8-byte loads and stores through native vectors.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st_nt16(void* p, uint4 w) {
    u32x4_t v = {w.x, w.y, w.z, w.w};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void st_nt8(void* p, uint2 w) {
    u32x2_t v = {w.x, w.y};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t*>(p));
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats to bf16 (round to nearest even, NaN stays NaN) packed low/high
// in one dword: a single v_cvt_pk_bf16_f32.  Converting each float on its own
// and packing with shifts costs four more VALU operations per pair.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// |x| of both bf16 halves of a dword, as two unsigned 16-bit magnitudes.
// NaN magnitudes (> 0x7F80) compare above +Inf (0x7F80), above every finite
// value; so the unsigned max of magnitudes is a NaN-propagating amax.
__device__ __forceinline__ uint32_t mag2(uint32_t w) { return w & 0x7FFF7FFFu; }

typedef unsigned short us2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pkmax_u16(uint32_t a, uint32_t b) {
    us2_t x = __builtin_bit_cast(us2_t, a);
    us2_t y = __builtin_bit_cast(us2_t, b);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}
__device__ __forceinline__ uint32_t hmax_u16(uint32_t a) {
    uint32_t lo = a & 0xFFFFu, hi = a >> 16;
    return lo > hi ? lo : hi;
}

// Scale from an amax given as bf16 magnitude bits (0 .. 0x7FFF):
// scale = FMAX / amax (IEEE fp32 division), 1 for amax 0 / Inf / NaN,
// FLT_MAX if the division overflows; scale_inv = 1 / scale.
template <int FMT>
__device__ __forceinline__ void scale_from_amax_bits(uint32_t m, float& s, float& si) {
    if (m == 0u || m >= 0x7F80u) {
        s = 1.0f;
    } else {
        float amax = __uint_as_float(m << 16);
        s = FmtTraits<FMT>::fmax / amax;
        if (__builtin_isinf(s)) s = 3.40282346638528859812e+38f;
    }
    si = 1.0f / s;
}

// Scale from an fp32 amax >= 0 or NaN (the largest entry of an amax
// history): scale = FMAX / amax (IEEE fp32 division), 1 for amax 0 / +Inf /
// NaN, FLT_MAX if the division overflows; scale_inv = 1 / scale.
template <int FMT>
__device__ __forceinline__ void scale_from_amax_f32(float amax, float& s, float& si) {
    if (!(amax > 0.0f) || __builtin_isinf(amax)) {
        s = 1.0f;
    } else {
        s = FmtTraits<FMT>::fmax / amax;
        if (__builtin_isinf(s)) s = 3.40282346638528859812e+38f;
    }
    si = 1.0f / s;
}

// Four fp32 values -> four FP8 codes (byte 0 = a), round to nearest even,
// saturating: values are clamped to [-FMAX, FMAX] before the hardware
// conversion.  NaN inputs are patched separately (patch_nan8).
template <int FMT>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
    constexpr float F = FmtTraits<FMT>::fmax;
    a = __builtin_amdgcn_fmed3f(a, -F, F);
    b = __builtin_amdgcn_fmed3f(b, -F, F);
    c = __builtin_amdgcn_fmed3f(c, -F, F);
    d = __builtin_amdgcn_fmed3f(d, -F, F);
    int r;
    if constexpr (FMT == 0) {
        r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
        r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    } else {
        r = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
        r = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, r, true);
    }
    return (uint32_t)r;
}

// Eight bf16 (one 16-byte load) times one scale -> eight codes.
template <int FMT>
__device__ __forceinline__ uint2 enc8(const uint4 w, float s) {
    uint2 r;
    r.x = cvt4<FMT>(bf16_lo(w.x) * s, bf16_hi(w.x) * s, bf16_lo(w.y) * s, bf16_hi(w.y) * s);
    r.y = cvt4<FMT>(bf16_lo(w.z) * s, bf16_hi(w.z) * s, bf16_lo(w.w) * s, bf16_hi(w.w) * s);
    return r;
}

// Eight bf16 of one row, each column with its own scale s[0..7].
template <int FMT>
__device__ __forceinline__ uint2 enc8_cols(const uint4 w, const float* s) {
    uint2 r;
    r.x = cvt4<FMT>(bf16_lo(w.x) * s[0], bf16_hi(w.x) * s[1], bf16_lo(w.y) * s[2], bf16_hi(w.y) * s[3]);
    r.y = cvt4<FMT>(bf16_lo(w.z) * s[4], bf16_hi(w.z) * s[5], bf16_lo(w.w) * s[6], bf16_hi(w.w) * s[7]);
    return r;
}

// Replace the code of every NaN input by 0x7F (slow path, taken only when
// the governing amax says a NaN is present).
__device__ __forceinline__ uint32_t patch_nan2(uint32_t w, uint32_t code, int byte0) {
    if ((w & 0x7FFFu) > 0x7F80u) code = (code & ~(0xFFu << (8 * byte0))) | (0x7Fu << (8 * byte0));
    if (((w >> 16) & 0x7FFFu) > 0x7F80u)
        code = (code & ~(0xFFu << (8 * (byte0 + 1)))) | (0x7Fu << (8 * (byte0 + 1)));
    return code;
}
__device__ __forceinline__ uint2 patch_nan8(const uint4 w, uint2 c) {
    c.x = patch_nan2(w.x, c.x, 0);
    c.x = patch_nan2(w.y, c.x, 2);
    c.y = patch_nan2(w.z, c.y, 0);
    c.y = patch_nan2(w.w, c.y, 2);
    return c;
}

// 4x4 byte transpose: rows d0..d3 (byte c of d_r = element (r, c)) ->
// columns e0..e3 (byte r of e_c = element (r, c)).
__device__ __forceinline__ void transpose4x4(uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3,
                                             uint32_t& e0, uint32_t& e1, uint32_t& e2, uint32_t& e3) {
    // interleave bytes of row pairs: (d0.b0, d1.b0, d0.b1, d1.b1) etc.
    uint32_t lo01 = __builtin_amdgcn_perm(d1, d0, 0x05010400u);
    uint32_t hi01 = __builtin_amdgcn_perm(d1, d0, 0x07030602u);
    uint32_t lo23 = __builtin_amdgcn_perm(d3, d2, 0x05010400u);
    uint32_t hi23 = __builtin_amdgcn_perm(d3, d2, 0x07030602u);
    e0 = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
    e1 = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
    e2 = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
    e3 = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
}

// Max over the 16 lanes of a DPP row (lanes 16r .. 16r+15), result in all 16.
// Packed unsigned 16-bit max: two independent reductions per dword.
__device__ __forceinline__ uint32_t row16_pkmax(uint32_t v) {
    v = pkmax_u16(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));   // quad xor 1
    v = pkmax_u16(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));   // quad xor 2
    v = pkmax_u16(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true));  // half-row mirror
    v = pkmax_u16(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true));  // row mirror
    return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        uint32_t w = (uint32_t)__shfl_xor((int)v, o, 64);
        v = v > w ? v : w;
    }
    return v;
}

}  // namespace fp8k
