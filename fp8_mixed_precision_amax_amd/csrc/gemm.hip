// GEMM dispatcher: the tensorwise kernel (gemm_tensor.hip) or the
// block-scaled kernel (gemm_block.hip), then, for split-K launches, the
// deterministic reduction of the fp32 slice partials.
//
// Method ("Native FP8 MLP reconstruction", implementation paragraph): the
// three GEMMs of the FP8 linear accumulate in fp32 and write BF16.  Split-K
// (small outputs with long contractions, e.g. the weight gradient): each
// slice writes fp32 partials; the reduce kernel sums the slices in fixed
// order, applies the tensorwise factor (block-scaled partials already carry
// theirs) and rounds to bf16.
#include "device.hpp"
#include "gelu_keys.hpp"
#include "gemm_common.hpp"
#include "internal.hpp"

namespace fp8k {

// Sum split-K partials in split order, apply the tensorwise factor, bf16.
// With amax_part, also one partial max |bf16 C| per block (block 0 zeroes the
// slots no block owns); with gelu_keys, the four GELU amax keys of C per
// block likewise (gelu_keys.hpp).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits, int64_t n4,
                                                            int64_t IJ, const float* sa, const float* sb,
                                                            int tensorwise, uint16_t* __restrict__ c,
                                                            uint16_t* __restrict__ amax_part,
                                                            uint16_t* __restrict__ gelu_keys) {
    const float t = tensorwise ? sa[0] * sb[0] : 1.0f;
    uint32_t amx = 0;
    GeluKeys gk;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
        float4 s = reinterpret_cast<const float4*>(part)[i];
        for (int z = 1; z < splits; z++) {
            const float4 p = reinterpret_cast<const float4*>(part + (int64_t)z * IJ)[i];
            s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
        }
        if (tensorwise) { s.x *= t; s.y *= t; s.z *= t; s.w *= t; }
        uint2 w;
        w.x = pack_bf16x2(s.x, s.y);
        w.y = pack_bf16x2(s.z, s.w);
        reinterpret_cast<uint2*>(c)[i] = w;
        amx = pkmax_u16(amx, pkmax_u16(mag2(w.x), mag2(w.y)));
        if (gelu_keys) {
            gk.add(w.x);
            gk.add(w.y);
        }
    }
    if (gelu_keys) {
        __shared__ uint32_t kred[kGeluKeyArrays][4];
        uint32_t k[kGeluKeyArrays];
        gk.fold(k);
#pragma unroll
        for (int q = 0; q < kGeluKeyArrays; q++) k[q] = wave_max_u32(k[q]);
        if ((threadIdx.x & 63) == 0)
#pragma unroll
            for (int q = 0; q < kGeluKeyArrays; q++) kred[q][threadIdx.x >> 6] = k[q];
        __syncthreads();
        if (threadIdx.x < kGeluKeyArrays) {
            const int q = (int)threadIdx.x;
            uint32_t r = kred[q][0];
            for (int w = 1; w < 4; w++) r = r > kred[q][w] ? r : kred[q][w];
            gelu_keys[q * kMaxAmaxPartials + blockIdx.x] = (uint16_t)r;
        }
        if (blockIdx.x == 0)
            for (int p = (int)gridDim.x + (int)threadIdx.x; p < kMaxAmaxPartials; p += 256)
#pragma unroll
                for (int q = 0; q < kGeluKeyArrays; q++) gelu_keys[q * kMaxAmaxPartials + p] = 0;
    }
    if (amax_part) {
        __shared__ uint32_t red[4];
        const uint32_t m = wave_max_u32(hmax_u16(amx));
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t r = red[0];
            for (int w = 1; w < 4; w++) r = r > red[w] ? r : red[w];
            amax_part[blockIdx.x] = (uint16_t)r;
        }
        if (blockIdx.x == 0)
            for (int p = (int)gridDim.x + (int)threadIdx.x; p < kMaxAmaxPartials; p += 256) amax_part[p] = 0;
    }
}

hipError_t launch_splitk_reduce(const float* part, int splits, int64_t I, int64_t J, const float* sa,
                                const float* sb, uint16_t* c, hipStream_t stream) {
    const int64_t n4 = I * J / 4;
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > kMaxAmaxPartials) blocks = kMaxAmaxPartials;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, part, splits, n4, I * J, sa,
                       sb, sa ? 1 : 0, c, nullptr, nullptr);
    return hipGetLastError();
}

int cu_count() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

size_t gemm_ws_bytes(int64_t I, int64_t J, int64_t K) {
    // the largest split count any of the kernels would use for this shape
    int s = gemm_tensor_splits(I, J, K);
    const int b = gemm_block_splits(I, J, K), w = gemm_block_wide_splits(I, J, K);
    s = s > b ? s : b;
    s = s > w ? s : w;
    return s > 1 ? (size_t)s * (size_t)I * (size_t)J * sizeof(float) : 0;
}

hipError_t launch_gemm(const GemmLaunch& l, hipStream_t stream) {
    const bool block = l.sa.group != 0;
    int splits;
    hipError_t e;
    if (!block) {
        splits = gemm_tensor_splits(l.I, l.J, l.K);
        e = launch_gemm_tensor(l, splits, stream);
    } else if (l.sb.group == 128) {
        // B factors shared by 128-row groups (a 128x128-block weight)
        splits = gemm_block_wide_splits(l.I, l.J, l.K);
        e = launch_gemm_block_wide(l, splits, stream);
    } else {
        splits = gemm_block_splits(l.I, l.J, l.K);
        e = launch_gemm_block(l, splits, stream);
    }
    if (e != hipSuccess || splits == 1) return e;
    const int64_t n4 = l.I * l.J / 4;
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > kMaxAmaxPartials) blocks = kMaxAmaxPartials;   // one amax partial per block
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const float*>(l.ws), splits, n4, l.I * l.J, l.sa.sinv, l.sb.sinv, block ? 0 : 1,
                       static_cast<uint16_t*>(l.c), block ? nullptr : l.c_amax, block ? nullptr : l.gelu_keys);
    return hipGetLastError();
}

}  // namespace fp8k
