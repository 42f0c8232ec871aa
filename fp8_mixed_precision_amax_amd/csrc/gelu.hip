// GELU tables and the elementwise GELU / dGELU kernels (gfx950).
//
// The MLP block of the workload puts GELU between its two linears; its exact
// (erf) form is used: GELU(x) = x Phi(x), GELU'(x) = Phi(x) + x phi(x).  The
// lookup scheme and the closed forms outside the tables are described in
// act.hpp.
//
// Tables: one copy per device, in module-scope device arrays (no allocation),
// filled on the first call that needs them on a device by act_table_kernel:
// one thread per entry evaluates both functions in fp64 (the device math
// library's erfc and exp) and rounds once to fp32; every exact value lies at
// least 2^-38 (relative) from an fp32 rounding boundary, so an fp64
// evaluation good to a few units in its last place rounds correctly.
//
// Kernels
//   act_table_kernel  fills both tables
//   gelu_kernel       y = GELU(x), 16-byte loads and stores, table in LDS
//   dgelu_kernel      dx = dy * GELU'(x), likewise
#include <mutex>

#include "act.hpp"
#include "internal.hpp"

namespace fp8k {

__device__ __align__(16) uint16_t g_gelu_tab[kActEntries];
__device__ __align__(16) float g_dgelu_tab[kActEntries];

__global__ __launch_bounds__(256) void act_table_kernel(uint16_t* __restrict__ gt, float* __restrict__ dt) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= kActEntries) return;
    const uint32_t b = (i >= kActHalf ? 0x8000u : 0u) | (kActLo + i % kActHalf);
    const double x = (double)__uint_as_float(b << 16);
    const double cdf = 0.5 * erfc(-x * 0.70710678118654752440);          // Phi(x)
    const double pdf = exp(-0.5 * x * x) * 0.39894228040143267794;        // phi(x)
    gt[i] = (uint16_t)bf16_rne_canon((float)(x * cdf));
    dt[i] = (float)(cdf + x * pdf);
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_act_mu;
ActTables g_act[kMaxDevices];
bool g_act_ready[kMaxDevices];
}  // namespace

hipError_t act_tables(hipStream_t stream, ActTables& out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_act_mu);
    if (!g_act_ready[dev]) {
        // the first use on a device builds the tables and waits for them, so
        // it cannot be captured into a graph
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(stream, &cs);
        if (e != hipSuccess) return e;
        if (cs != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
        void* pg = nullptr;
        void* pd = nullptr;
        if ((e = hipGetSymbolAddress(&pg, HIP_SYMBOL(g_gelu_tab))) != hipSuccess) return e;
        if ((e = hipGetSymbolAddress(&pd, HIP_SYMBOL(g_dgelu_tab))) != hipSuccess) return e;
        // a stream of its own, so the wait covers nothing the caller queued
        hipStream_t s = nullptr;
        if ((e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking)) != hipSuccess) return e;
        hipLaunchKernelGGL(act_table_kernel, dim3((kActEntries + 255) / 256), dim3(256), 0, s,
                           static_cast<uint16_t*>(pg), static_cast<float*>(pd));
        e = hipGetLastError();
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        hipError_t e2 = hipStreamDestroy(s);
        if (e != hipSuccess) return e;
        if (e2 != hipSuccess) return e2;
        g_act[dev].gelu = static_cast<const uint16_t*>(pg);
        g_act[dev].dgelu = static_cast<const float*>(pd);
        g_act_ready[dev] = true;
    }
    out = g_act[dev];
    return hipSuccess;
}

constexpr int kActThreads = 256;

__global__ __launch_bounds__(kActThreads) void gelu_kernel(const uint4* __restrict__ x, uint4* __restrict__ y,
                                                           int64_t n16, const uint16_t* __restrict__ gtab) {
    __shared__ __align__(16) uint16_t tab[kActEntries];
    act_table_to_lds(tab, gtab, sizeof(tab));
    __syncthreads();
    const int64_t stride = (int64_t)gridDim.x * kActThreads;
    int64_t i = (int64_t)blockIdx.x * kActThreads + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; u++) v[u] = ld_nt16(x + i + u * stride);
#pragma unroll
        for (int u = 0; u < 4; u++) st_nt16(y + i + u * stride, gelu8(v[u], tab));
    }
    for (; i < n16; i += stride) st_nt16(y + i, gelu8(ld_nt16(x + i), tab));
}

__global__ __launch_bounds__(kActThreads) void dgelu_kernel(const uint4* __restrict__ dy, const uint4* __restrict__ x,
                                                            uint4* __restrict__ dx, int64_t n16,
                                                            const float* __restrict__ dtab) {
    __shared__ __align__(16) float tab[kActEntries];
    act_table_to_lds(tab, dtab, sizeof(tab));
    __syncthreads();
    const int64_t stride = (int64_t)gridDim.x * kActThreads;
    int64_t i = (int64_t)blockIdx.x * kActThreads + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        uint4 d[4], v[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            d[u] = ld_nt16(dy + i + u * stride);
            v[u] = ld_nt16(x + i + u * stride);
        }
#pragma unroll
        for (int u = 0; u < 4; u++) st_nt16(dx + i + u * stride, dgelu8(d[u], v[u], tab));
    }
    for (; i < n16; i += stride) st_nt16(dx + i, dgelu8(ld_nt16(dy + i), ld_nt16(x + i), tab));
}

// workgroups of the elementwise kernels: about four per CU, each reading its
// table once
int act_grid(int64_t n16) {
    int64_t g = (n16 + kActThreads - 1) / kActThreads;
    if (g > 1024) g = 1024;
    return g < 1 ? 1 : (int)g;
}

hipError_t launch_gelu(const void* x, void* y, int64_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    ActTables t;
    hipError_t e = act_tables(stream, t);
    if (e != hipSuccess) return e;
    const int64_t n16 = n / 8;
    hipLaunchKernelGGL(gelu_kernel, dim3(act_grid(n16)), dim3(kActThreads), 0, stream, static_cast<const uint4*>(x),
                       static_cast<uint4*>(y), n16, t.gelu);
    return hipGetLastError();
}

hipError_t launch_dgelu(const void* dy, const void* x, void* dx, int64_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    ActTables t;
    hipError_t e = act_tables(stream, t);
    if (e != hipSuccess) return e;
    const int64_t n16 = n / 8;
    hipLaunchKernelGGL(dgelu_kernel, dim3(act_grid(n16)), dim3(kActThreads), 0, stream, static_cast<const uint4*>(dy),
                       static_cast<const uint4*>(x), static_cast<uint4*>(dx), n16, t.dgelu);
    return hipGetLastError();
}

}  // namespace fp8k
