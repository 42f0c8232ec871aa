// BF16 GEMM on the gfx950 matrix cores: C[i][j] = bf16(sum_k A[i][k] B[j][k]),
// fp32 accumulation, the comparator the pages time the FP8 linear against
// ("Native FP8 MLP reconstruction", isolated-linear table: the same linears
// in BF16).  Each operand is either contraction-major (A[i][k] at i*K + k) or
// output-major (A[i][k] at k*I + i), so the linear's three products need no
// transposed copies: the forward X W^T has both contraction-major, the data
// gradient dY W has W output-major, the weight gradient dY^T X has both
// output-major.
//
// Design
//  - persistent: one workgroup of 8 waves per CU walks 256 x 256 output tiles
//    (with split-K slices for short outputs over long contractions), dealt
//    XCD by XCD and rastered in groups of tile rows like the FP8 kernels.
//  - each wave owns a 128 x 64 block of the tile: 4 x 2 instructions
//    v_mfma_f32_32x32x16_bf16 per 16-long contraction step, 128 fp32
//    accumulators.  The operands go in swapped (B's fragment first), so each
//    lane ends up holding one output row and runs of 4 consecutive columns.
//  - a stage is 64 contraction elements of both operands, 32 KiB each,
//    double-buffered in LDS: the next stage's global loads are issued at the
//    top of a stage into registers and written to the other buffer after its
//    MFMAs; one barrier per stage.
//  - contraction-major tiles are stored as 256 rows of 128 bytes, 16-byte
//    chunk c of row r at c ^ (r mod 8); a fragment (8 contraction elements of
//    one row per lane) is one 16-byte LDS read.
//  - output-major tiles are stored as 64 contraction rows of 512 bytes,
//    64-byte segment s of row k at s ^ (k mod 8); a fragment is two
//    ds_read_b64_tr_b16: within a group of 16 lanes, lane t loads 4
//    consecutive output elements of contraction row k0 + t/4, and the
//    transposing read hands lane L the 4 consecutive contraction elements of
//    output element L (pinned on the GPU: lane L's element e comes from lane
//    4e + L/4's element L mod 4).
//  - epilogue: bf16 through LDS (the stage buffers, 512-byte rows, 16-byte
//    chunk c of row r at c ^ (r mod 32)), stored as whole 16-byte chunks;
//    split-K slices write fp32 partial sums that the split-K reduce adds in
//    slice order.
#include "device.hpp"
#include "gemm_common.hpp"
#include "internal.hpp"

namespace fp8k {
namespace bf16g {

constexpr int BM = 256, BN = 256, BK = 64, NW = 8;
constexpr int OP_BYTES = BM * BK * 2;            // one operand's stage: 32 KiB
constexpr int STAGE = 2 * OP_BYTES;
constexpr int LDS_BYTES = 2 * STAGE;             // two stages: 128 KiB (also the epilogue's staging)
static_assert(BM == BN, "square tiles");
static_assert(BM * BN * 2 <= LDS_BYTES, "epilogue staging");

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct Args {
    const uint16_t* a;
    const uint16_t* b;
    int64_t I, J, K;
    uint16_t* c;
    float* part;          // split-K partials [splits][I][J]
    int splits, tiles_i, tiles_j, items, gi;
};

struct Item {
    int ti, tj, z;
    int64_t k0, k1;
};

__device__ __forceinline__ bool item_at(const Args& g, int r, Item& it) {
    const int G = gridDim.x, b = blockIdx.x;
    const int Lg = r * G + ((G & 7) == 0 ? (b & 7) * (G >> 3) + (b >> 3) : b);
    if (Lg >= g.items) return false;
    const int tiles = g.tiles_i * g.tiles_j;
    const int z = Lg / tiles, t = Lg - z * tiles;
    const int per_group = g.gi * g.tiles_j, grp = t / per_group, local = t - grp * per_group;
    int rows = g.tiles_i - grp * g.gi;
    rows = rows < g.gi ? rows : g.gi;
    it.ti = grp * g.gi + local % rows;
    it.tj = local / rows;
    it.z = z;
    const int64_t stages = g.K / BK;
    it.k0 = stages * z / g.splits * BK;
    it.k1 = stages * (z + 1) / g.splits * BK;
    return true;
}

// Global -> register loads of one operand's stage (4 x 16 bytes per thread),
// zero outside the operand.  T = 0: contraction-major [rows][K]; T = 1:
// output-major [K][rows].
template <int T>
__device__ __forceinline__ void load_stage(const uint16_t* __restrict__ base, int64_t rows, int64_t K, int64_t r0,
                                           int64_t k0, uint4 (&v)[4]) {
#pragma unroll
    for (int u = 0; u < 4; u++) {
        const int q = (int)threadIdx.x + u * NW * 64;
        int64_t row, col;
        bool ok;
        if (T == 0) {
            row = r0 + (q >> 3);
            col = k0 + (q & 7) * 8;
            ok = row < rows;
            v[u] = ok ? *reinterpret_cast<const uint4*>(base + row * K + col) : make_uint4(0, 0, 0, 0);
        } else {
            row = k0 + (q >> 5);
            col = r0 + (q & 31) * 8;
            ok = col < rows;
            v[u] = ok ? *reinterpret_cast<const uint4*>(base + row * rows + col) : make_uint4(0, 0, 0, 0);
        }
    }
}

// LDS byte offset of 16-byte chunk q (the load's numbering) of a stage tile.
template <int T>
__device__ __forceinline__ uint32_t chunk_off(int q) {
    if (T == 0) {
        const int r = q >> 3, c = q & 7;
        return (uint32_t)(r * 128 + ((c ^ (r & 7)) << 4));
    }
    const int kr = q >> 5, c = q & 31;
    return (uint32_t)(kr * 512 + ((((c >> 2) ^ (kr & 7)) << 2) + (c & 3)) * 16);
}

template <int T>
__device__ __forceinline__ void store_stage(uint8_t* tile, const uint4 (&v)[4]) {
#pragma unroll
    for (int u = 0; u < 4; u++) {
        const int q = (int)threadIdx.x + u * NW * 64;
        *reinterpret_cast<uint4*>(tile + chunk_off<T>(q)) = v[u];
    }
}

// Fragment of rows rb .. rb+31 of a stage tile for contraction step kk
// (elements kk*16 .. kk*16+15): lane l gets row rb + l % 32, contraction
// elements kk*16 + 8 (l / 32) .. +7.
template <int T>
__device__ __forceinline__ bf16x8_t frag(const uint8_t* tile, int rb, int kk, int lane) {
    if (T == 0) {
        const int r = rb + (lane & 31), c = kk * 2 + (lane >> 5);
        return *reinterpret_cast<const bf16x8_t*>(tile + r * 128 + ((c ^ (r & 7)) << 4));
    }
    const int kbase = kk * 16 + 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int seg = rb >> 5;
    const int wb = 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
    const int k0 = kbase, k1 = kbase + 4;
    typedef __attribute__((address_space(3))) s4_t lds_s4;
    const uint32_t o0 = (uint32_t)(k0 * 512 + ((seg ^ (k0 & 7)) << 6) + wb);
    const uint32_t o1 = (uint32_t)(k1 * 512 + ((seg ^ (k1 & 7)) << 6) + wb);
    const s4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(tile + o0));
    const s4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(tile + o1));
    const s4_t w[2] = {lo, hi};
    return __builtin_bit_cast(bf16x8_t, w);
}

template <int TA, int TB>
__global__ __launch_bounds__(NW * 64, 1) void gemm_bf16_kernel(Args g) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];
    const int lane = (int)(threadIdx.x & 63);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wr = wave >> 2, wc = wave & 3;      // 2 x 4 waves: rows wr*128, columns wc*64
    Item it;
    for (int r = 0; item_at(g, r, it); r++) {
        const int64_t i0 = (int64_t)it.ti * BM, j0 = (int64_t)it.tj * BN;
        f32x16_t acc[4][2];
#pragma unroll
        for (int mi = 0; mi < 4; mi++)
#pragma unroll
            for (int nj = 0; nj < 2; nj++) acc[mi][nj] = f32x16_t{};
        uint4 va[4], vb[4];
        __syncthreads();     // the previous item's epilogue has read the staging
        load_stage<TA>(g.a, g.I, g.K, i0, it.k0, va);
        load_stage<TB>(g.b, g.J, g.K, j0, it.k0, vb);
        store_stage<TA>(smem, va);
        store_stage<TB>(smem + OP_BYTES, vb);
        int buf = 0;
        for (int64_t k = it.k0; k < it.k1; k += BK) {
            __syncthreads();
            const bool more = k + BK < it.k1;
            if (more) {
                load_stage<TA>(g.a, g.I, g.K, i0, k + BK, va);
                load_stage<TB>(g.b, g.J, g.K, j0, k + BK, vb);
            }
            const uint8_t* ta = smem + buf * STAGE;
            const uint8_t* tb = ta + OP_BYTES;
#pragma unroll
            for (int kk = 0; kk < BK / 16; kk++) {
                bf16x8_t fa[4], fb[2];
#pragma unroll
                for (int mi = 0; mi < 4; mi++) fa[mi] = frag<TA>(ta, wr * 128 + mi * 32, kk, lane);
#pragma unroll
                for (int nj = 0; nj < 2; nj++) fb[nj] = frag<TB>(tb, wc * 64 + nj * 32, kk, lane);
#pragma unroll
                for (int mi = 0; mi < 4; mi++)
#pragma unroll
                    for (int nj = 0; nj < 2; nj++)
                        acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[nj], fa[mi], acc[mi][nj], 0, 0, 0);
            }
            if (more) {
                uint8_t* nt = smem + (buf ^ 1) * STAGE;
                store_stage<TA>(nt, va);
                store_stage<TB>(nt + OP_BYTES, vb);
            }
            buf ^= 1;
        }
        // lane l holds output row (block row) l % 32 and, per group of 4
        // registers q, columns 8q + 4 (l / 32) .. +3 of the block
        if (g.splits > 1) {
            float* out = g.part + (int64_t)it.z * g.I * g.J;
#pragma unroll
            for (int mi = 0; mi < 4; mi++)
#pragma unroll
                for (int nj = 0; nj < 2; nj++) {
                    const int64_t row = i0 + wr * 128 + mi * 32 + (lane & 31);
                    const int64_t colb = j0 + wc * 64 + nj * 32 + 4 * (lane >> 5);
                    if (row < g.I && colb < g.J)
#pragma unroll
                        for (int q = 0; q < 4; q++)
                            *reinterpret_cast<float4*>(out + row * g.J + colb + 8 * q) =
                                make_float4(acc[mi][nj][4 * q], acc[mi][nj][4 * q + 1], acc[mi][nj][4 * q + 2],
                                            acc[mi][nj][4 * q + 3]);
                }
            continue;
        }
        __syncthreads();     // every wave is done with the stage buffers
#pragma unroll
        for (int mi = 0; mi < 4; mi++)
#pragma unroll
            for (int nj = 0; nj < 2; nj++) {
                const int rr = wr * 128 + mi * 32 + (lane & 31);
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const int c = (wc * 64 + nj * 32) / 8 + q;
                    uint2 w;
                    w.x = pack_bf16x2(acc[mi][nj][4 * q], acc[mi][nj][4 * q + 1]);
                    w.y = pack_bf16x2(acc[mi][nj][4 * q + 2], acc[mi][nj][4 * q + 3]);
                    *reinterpret_cast<uint2*>(smem + rr * 512 + ((c ^ (rr & 31)) << 4) + 8 * (lane >> 5)) = w;
                }
            }
        __syncthreads();
#pragma unroll 4
        for (int u = 0; u < (BM * BN / 8) / (NW * 64); u++) {
            const int q = (int)threadIdx.x + u * NW * 64;
            const int rr = q >> 5, c = q & 31;
            const int64_t row = i0 + rr, col = j0 + c * 8;
            const uint4 v = *reinterpret_cast<const uint4*>(smem + rr * 512 + ((c ^ (rr & 31)) << 4));
            if (row < g.I && col < g.J) *reinterpret_cast<uint4*>(g.c + row * g.J + col) = v;
        }
    }
}

}  // namespace bf16g

using namespace bf16g;

int gemm_bf16_splits(int64_t I, int64_t J, int64_t K) {
    const int64_t tiles = ((I + BM - 1) / BM) * ((J + BN - 1) / BN);
    // one work item per CU where the output is short, slices of >= 1024
    int64_t s = 1;
    while (tiles * s < 256 && K / (s * 2) >= 1024 && s < 64) s *= 2;
    return (int)s;
}

size_t gemm_bf16_ws_bytes(int64_t I, int64_t J, int64_t K) {
    const int s = gemm_bf16_splits(I, J, K);
    return s > 1 ? (size_t)s * (size_t)I * (size_t)J * sizeof(float) : 0;
}

hipError_t launch_gemm_bf16(const Bf16GemmLaunch& l, hipStream_t stream) {
    Args g;
    g.a = static_cast<const uint16_t*>(l.a);
    g.b = static_cast<const uint16_t*>(l.b);
    g.I = l.I;
    g.J = l.J;
    g.K = l.K;
    g.c = static_cast<uint16_t*>(l.c);
    g.part = static_cast<float*>(l.ws);
    g.splits = gemm_bf16_splits(l.I, l.J, l.K);
    g.tiles_i = (int)((l.I + BM - 1) / BM);
    g.tiles_j = (int)((l.J + BN - 1) / BN);
    g.items = g.tiles_i * g.tiles_j * g.splits;
    g.gi = g.tiles_j >= 16 ? 8 : 2;
    int grid = cu_count();
    if (grid > g.items) grid = g.items;
#define FP8K_BF16(TA, TB) hipLaunchKernelGGL((gemm_bf16_kernel<TA, TB>), dim3(grid), dim3(NW * 64), 0, stream, g)
    if (l.ta == 0 && l.tb == 0) FP8K_BF16(0, 0);
    else if (l.ta == 0 && l.tb == 1) FP8K_BF16(0, 1);
    else if (l.ta == 1 && l.tb == 0) FP8K_BF16(1, 0);
    else FP8K_BF16(1, 1);
#undef FP8K_BF16
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || g.splits == 1) return e;
    return launch_splitk_reduce(static_cast<const float*>(l.ws), g.splits, l.I, l.J, nullptr, nullptr,
                                static_cast<uint16_t*>(l.c), stream);
}

}  // namespace fp8k
