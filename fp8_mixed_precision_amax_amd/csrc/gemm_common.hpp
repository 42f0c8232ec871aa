// Building blocks shared by the FP8 GEMM kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8k {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16 bytes of the bf16 output.  NT: a non-temporal (streaming) store.  The
// bf16 output of a short contraction is large next to its operands and
// leaves the GPU anyway; streamed, its stores retire faster, and the next
// tile's operand loads, issued after them and waited for in order with them
// (one vmcnt for loads and stores), stall less: 131072 x 2048 x 512
// 203 -> 144 us, 131072 x 512 x 2048 127 -> 115 us; on 8192^3, where the
// output is small next to the contraction, 375 -> 399 us, so only
// contractions up to 2048 use them.
template <bool NT>
__device__ __forceinline__ void st_out16(void* p, u32x4 v) {
    if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
    else *reinterpret_cast<u32x4*>(p) = v;
}
constexpr int64_t kNtMaxContraction = 2048;

// One v_mfma_f32_32x32x64_f8f6f4 (scale operands 0: the unscaled form).
// Matrix-core operand 0 = B fragment (rows j), operand 1 = A fragment (rows i),
// so each lane's accumulators hold one output row i and runs of 4 columns j.
// FA / FB: 0 = E4M3, 1 = E5M2.
template <int FA, int FB>
__device__ __forceinline__ v16f mfma(const v8i& bfrag, const v8i& afrag, const v16f& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfrag, afrag, c, FB, FA, 0, 0, 0, 0);
}

// XOR swizzle of the 16-byte chunk index of an LDS row of BK bytes: the
// fragment reads of 16 consecutive rows then touch 16 distinct bank groups.
template <int BK>
__device__ __forceinline__ int swz(int row) {
    return BK == 64 ? ((row >> 2) & 3) : ((row >> 1) & 7);
}

__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(n) for n in 0..63 (gfx9 encoding: low 4 bits + bits 15:14;
// expcnt and lgkmcnt fields left at "no wait")
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N <= 63, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Byte offset of a __shared__ object in the workgroup's LDS.
__device__ __forceinline__ uint32_t lds_off(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16-byte LDS read issued as inline assembly.  The compiler cannot tell these
// reads from the asynchronous LDS-DMA writes into other stage buffers and
// would otherwise precede every read with s_waitcnt vmcnt(0), draining the
// whole prefetch queue; the stage hand-off is synchronised explicitly
// (s_waitcnt vmcnt(n) on the DMA of the stage + s_barrier) instead.  The
// result is valid only after an s_waitcnt lgkmcnt(0) that takes the value
// as an operand.
template <int OFF>
__device__ __forceinline__ u32x4 ds_read16(uint32_t addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}

// 32-byte matrix-core fragment: chunks at a0 + OFF and a1 + OFF.
template <int OFF>
__device__ __forceinline__ v8i ds_frag(uint32_t a0, uint32_t a1) {
    const u32x4 lo = ds_read16<OFF>(a0), hi = ds_read16<OFF>(a1);
    return __builtin_bit_cast(v8i, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Buffer resource over `bytes` bytes at `base` (raw, stride 0): reads at
// offsets >= bytes return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

int cu_count();

}  // namespace fp8k
