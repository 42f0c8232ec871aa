// Measured ceilings of the GPU the path runs on, for reading its rooflines:
// the HBM bandwidth that plain streaming kernels reach (read, write, copy)
// and the rate and shader clock of back-to-back FP8 matrix-core
// instructions.  Built as its own library (libfp8ceilings.so), loaded by the
// benchmark only; nothing of the FP8 linear depends on it.
//
// Every kernel is a grid-stride loop over 16-byte elements whose indices
// stay below n16 (the caller passes buffers of at least 16 * n16 bytes).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Read: U loads in flight per thread, non-temporal or ordinary.  The xor of
// the data decides a store that never happens in practice, so the loads
// cannot be dropped.
template <int U, bool NT>
__global__ __launch_bounds__(256) void read_kernel(const u4* __restrict__ x, int64_t n16, uint32_t* out) {
    uint32_t m = 0;
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u4 v[U];
#pragma unroll
        for (int k = 0; k < U; k++) v[k] = NT ? __builtin_nontemporal_load(x + i + k * stride) : x[i + k * stride];
#pragma unroll
        for (int k = 0; k < U; k++) m ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    for (; i < n16; i += stride) m ^= x[i].x;
    if (m == 0x9E3779B9u) out[0] = m;
}

template <bool NT>
__global__ __launch_bounds__(256) void write_kernel(u4* __restrict__ y, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    const u4 v = {(uint32_t)threadIdx.x, 1u, 2u, 3u};
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
        if (NT) __builtin_nontemporal_store(v, y + i);
        else y[i] = v;
    }
}

__global__ __launch_bounds__(256) void copy_kernel(const u4* __restrict__ x, u4* __restrict__ y, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(x + i), y + i);
}

// Four independent chains of v_mfma_f32_32x32x64_f8f6f4 per wave, register
// operands only.  Lane 0 of each workgroup records the shader-clock and
// 100 MHz real-time counters around the loop.
__global__ __launch_bounds__(512) void mfma_kernel(int iters, float* out, unsigned long long* clk) {
    const int lane = threadIdx.x & 63;
    v8i a, b;
    for (int i = 0; i < 8; i++) {
        a[i] = 0x38383838 ^ (lane * 7 + i);
        b[i] = 0x30303030 ^ (lane * 3 + i);
    }
    v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; it++) {
        c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, 0, 0, 0, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, 0, 0, 0, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, 0, 0, 0, 0, 0, 0);
    }
    float s = 0.f;
    for (int i = 0; i < 16; i++) s += c0[i] + c1[i] + c2[i] + c3[i];
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = t1 - t0;
        clk[2 * blockIdx.x + 1] = r1 - r0;
    }
}

}  // namespace

// variant 0: one ordinary load per thread per step; 1: four non-temporal
// loads in flight; 2: one non-temporal load.  out: 4 bytes of device memory.
extern "C" int fp8c_hbm_read(int variant, int grid, const void* x, int64_t n16, void* out, hipStream_t st) {
    const u4* p = static_cast<const u4*>(x);
    uint32_t* o = static_cast<uint32_t*>(out);
    if (variant == 0) hipLaunchKernelGGL((read_kernel<1, false>), dim3(grid), dim3(256), 0, st, p, n16, o);
    else if (variant == 1) hipLaunchKernelGGL((read_kernel<4, true>), dim3(grid), dim3(256), 0, st, p, n16, o);
    else hipLaunchKernelGGL((read_kernel<1, true>), dim3(grid), dim3(256), 0, st, p, n16, o);
    return (int)hipGetLastError();
}

// variant 0: ordinary stores; 1: non-temporal stores
extern "C" int fp8c_hbm_write(int variant, int grid, void* y, int64_t n16, hipStream_t st) {
    u4* q = static_cast<u4*>(y);
    if (variant == 0) hipLaunchKernelGGL((write_kernel<false>), dim3(grid), dim3(256), 0, st, q, n16);
    else hipLaunchKernelGGL((write_kernel<true>), dim3(grid), dim3(256), 0, st, q, n16);
    return (int)hipGetLastError();
}

extern "C" int fp8c_hbm_copy(int grid, const void* x, void* y, int64_t n16, hipStream_t st) {
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, st, static_cast<const u4*>(x), static_cast<u4*>(y),
                       n16);
    return (int)hipGetLastError();
}

// grid workgroups of `block` threads (a multiple of 64, at most 512);
// out: grid * block floats; clk: 2 * grid counters (shader clocks, then
// 100 MHz ticks, per workgroup).
extern "C" int fp8c_mfma(int grid, int block, int iters, float* out, unsigned long long* clk, hipStream_t st) {
    if (block <= 0 || block > 512 || block % 64) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_kernel, dim3(grid), dim3(block), 0, st, iters, out, clk);
    return (int)hipGetLastError();
}
