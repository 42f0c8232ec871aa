// GELU amax keys: what a GEMM epilogue emits about its bf16 output y so that
// the tensorwise quantize of GELU(y) (the next linear's input in an MLP
// block) needs no amax pass of its own.
//
// amax(GELU(y)) is not a function of max |y|: GELU is increasing above its
// minimiser x* = -0.75179... and decreasing below it, so |GELU| grows with y
// for y >= 0, shrinks as y rises from x* to 0, and shrinks as y falls below
// x*.  With s = -0.75 (bf16 0xBF40), the smallest bf16 value above x*, the
// activation act(y) = bf16(fl32(GELU(y))) is non-decreasing on y >= s and
// non-increasing on y < s (rounding keeps monotonicity), so over any set of
// bf16 values
//   max |act| = max( act(P),  |act(K2)|,  |act(K3)| )
// with P the largest y >= 0, K2 the smallest y in [s, 0), K3 the largest
// y < s (each where it exists); every NaN or -Inf input (GELU(-Inf) is NaN)
// makes the amax NaN, and a NaN among the y >= 0 shows up as P.
//
// On the bf16 bit patterns v these are four maxima/minima of packed 16-bit
// integers, five packed operations per pair of outputs:
//   P   = max over v as signed 16-bit (the non-negative values are the
//         positive int16s, ordered as the floats; a negative P means none)
//   V   = max over v as unsigned (>= 0xFF80: a -Inf or negative NaN exists)
//   d   = v - 0xBF41 (mod 2^16): the negative values in [s, 0), v in
//         [0x8000, 0xBF40], map to [0xC0BF, 0xFFFF] and the ones below s,
//         v in [0xBF41, 0xFFFF], to [0, 0x40BE]; the non-negative ones land
//         in between, [0x40BF, 0xC0BE], so
//   K2  = max over d (in [0xC0BF, 0xFFFF] when some y lies in [s, 0); its
//         pattern is d + 0xBF41, the largest magnitude there)
//   K3  = min over d (in [0, 0x40BE] when some y lies below s; pattern
//         d + 0xBF41, the smallest magnitude there)
// The partials buffer (FP8_GELU_AMAX_PARTIALS_BYTES) holds four arrays of
// kMaxAmaxPartials 16-bit slots, all reduced by unsigned max with 0 as
// "nothing": [P ^ 0x8000, V, K2, ~K3].
#pragma once

#include "device.hpp"

namespace fp8k {

constexpr uint32_t kGeluSplit = 0xBF40u;     // bf16 -0.75
constexpr uint32_t kGeluKeyAdd = 0x40BFu;    // d = v + 0x40BF = v - (kGeluSplit + 1)  (mod 2^16)
constexpr int kGeluKeyArrays = 4;

typedef short s2_t __attribute__((ext_vector_type(2)));

struct GeluKeys {
    uint32_t p = 0x80008000u;   // packed int16 max (starts at INT16_MIN)
    uint32_t v = 0u;            // packed uint16 max
    uint32_t lo = 0u;           // packed uint16 max of d
    uint32_t hi = 0xFFFFFFFFu;  // packed uint16 min of d

    __device__ __forceinline__ void add(uint32_t w) {
        const us2_t u = __builtin_bit_cast(us2_t, w);
        const us2_t d = u + (us2_t){(unsigned short)kGeluKeyAdd, (unsigned short)kGeluKeyAdd};
        p = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s2_t, p),
                                                                    __builtin_bit_cast(s2_t, w)));
        v = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2_t, v), u));
        lo = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2_t, lo), d));
        hi = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(us2_t, hi), d));
    }

    // the lane's four keys in max-reducible form ([P ^ 0x8000, V, K2, ~K3])
    __device__ __forceinline__ void fold(uint32_t out[4]) const {
        const uint32_t po = p ^ 0x80008000u;             // int16 order -> uint16 order
        out[0] = hmax_u16(po);
        out[1] = hmax_u16(v);
        out[2] = hmax_u16(lo);
        out[3] = hmax_u16(~hi);
    }
};

// amax(GELU) as bf16 magnitude bits (NaN above +Inf) from the four reduced
// keys k[0..3] in their stored form; gelu(b) returns the bf16 GELU of the
// bf16 pattern b.
template <class Gelu>
__device__ __forceinline__ uint32_t gelu_amax_from_keys(const uint32_t k[kGeluKeyArrays], Gelu gelu) {
    const uint32_t p = k[0] ^ 0x8000u;             // back to int16 order: below 0x8000 is non-negative
    const uint32_t k2 = k[2];
    const uint32_t k3 = (~k[3]) & 0xFFFFu;
    uint32_t amax = 0;
    if (p < 0x8000u) {
        const uint32_t a = gelu(p) & 0x7FFFu;
        amax = a > amax ? a : amax;
    }
    if (k2 >= 0xC0BFu) {                           // the smallest value in [-0.75, 0)
        const uint32_t a = gelu((k2 + 0xBF41u) & 0xFFFFu) & 0x7FFFu;
        amax = a > amax ? a : amax;
    }
    if (k3 <= 0x40BEu) {                           // the largest value below -0.75
        const uint32_t a = gelu((k3 + 0xBF41u) & 0xFFFFu) & 0x7FFFu;
        amax = a > amax ? a : amax;
    }
    if (k[1] >= 0xFF80u) amax = 0x7FC0u;           // -Inf or a negative NaN: GELU is NaN there
    return amax;
}

}  // namespace fp8k
