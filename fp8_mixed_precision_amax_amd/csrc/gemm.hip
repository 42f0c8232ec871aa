// FP8 GEMM C[i][j] = sum_k A[i][k] B[j][k] on the gfx950 FP8 matrix cores.
//
// Method ("Native FP8 MLP reconstruction", implementation paragraph): the
// three GEMMs of the FP8 linear take FP8 operands (E4M3 x E4M3 forward,
// E5M2 x E4M3 for both gradients), accumulate at full fp32 precision (no
// fast accumulation) and write BF16.  Tensorwise scales are applied once in
// the epilogue; block scales (Float8BlockScaling, TransformerEngine issue
// 2852) are applied to every 128-long contraction block's partial sum, which
// is then added to an fp32 accumulator.
//
// Design (one kernel for all three GEMMs: every operand is contraction-
// contiguous, "NT"):
//  - workgroup 256 threads = 4 waves in 2x2; tile BM=256 (i) x BN (j) x BK=128;
//    tensorwise BN=256 (wave 128x128 = 4x4 MFMA 32x32x64 blocks),
//    block-scaled BN=128 (wave 128x64) so the per-block fp32 accumulators fit.
//  - v_mfma_f32_32x32x64_f8f6f4 with the B tile as the matrix-core "A"
//    operand, so each lane's accumulators hold one output row i and runs of
//    4 consecutive columns j (8-byte bf16 runs in the epilogue).
//  - global -> registers (16-byte loads) -> LDS, double-buffered, one barrier
//    per K step; LDS rows are 128 bytes with the 16-byte chunk index XORed
//    by (row/2)%8, so both the 16-byte stores and the fragment reads of 16
//    consecutive rows hit 16 distinct bank groups.
//  - workgroup ids are remapped so consecutive tiles land on one XCD (the
//    dispatcher deals workgroups round-robin over the 8 XCDs) and rastered in
//    groups of 8 tile-rows for L2 reuse of A.
//  - epilogue: scale, bf16 (v_cvt_pk_bf16_f32, round to nearest even), stage
//    the tile in LDS (XOR-swizzled), write 16-byte coalesced rows.
//  - split-K (for small outputs with long contractions, e.g. the weight
//    gradient): each split writes fp32 partials; a reduce kernel sums the
//    splits in fixed order (deterministic), applies the tensorwise factor
//    and rounds to bf16.
#include "internal.hpp"

namespace fp8k {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 256;
constexpr int kBK = 128;
constexpr int kThreads = 256;

struct GemmArgs {
    const uint8_t* a;
    const uint8_t* b;
    GemmScale sa, sb;
    int64_t I, J, K;
    uint16_t* c;
    float* part;      // split-K partials [splits][I][J]
    int splits;
    int tiles_i, tiles_j;
    int ktiles;       // K / 128
};

template <int FA, int FB>
__device__ __forceinline__ v16f mfma(const v8i& bfrag, const v8i& afrag, const v16f& c) {
    // matrix-core operand 0 = B fragment (rows j), operand 1 = A fragment (rows i)
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfrag, afrag, c, FB, FA, 0, 0, 0, 0);
}

__device__ __forceinline__ v8i lds_frag(const uint8_t* tile, int row, int kk, int lane) {
    // 32 bytes of row `row`, logical 16-byte chunks kk*4 + (lane/32)*2 + {0,1}
    const int swz = (row >> 1) & 7;
    const int c0 = kk * 4 + (lane >> 5) * 2;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(tile + row * kBK + ((c0 ^ swz) << 4));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(tile + row * kBK + (((c0 + 1) ^ swz) << 4));
    return __builtin_bit_cast(v8i, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Map the linear workgroup id to a (tile_i, tile_j) pair.
__device__ __forceinline__ void tile_of(int bid, int tiles_i, int tiles_j, int& ti, int& tj) {
    const int nwg = tiles_i * tiles_j;
    if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);   // XCD-contiguous
    constexpr int G = 8;
    const int per_group = G * tiles_j;
    const int g = bid / per_group;
    const int local = bid - g * per_group;
    int rows = tiles_i - g * G;
    rows = rows < G ? rows : G;
    ti = g * G + local % rows;
    tj = local / rows;
}

template <int FA, int FB, bool BLOCK>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs g) {
    constexpr int WNJ = BLOCK ? 2 : 4;          // 32-col blocks per wave in j
    constexpr int BN = 2 * WNJ * 32;
    constexpr int A_BYTES = kBM * kBK;
    constexpr int B_BYTES = BN * kBK;
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int APASS = kBM / 32;             // 16-byte loads per thread for A
    constexpr int BPASS = BN / 32;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wi = wave >> 1, wj = wave & 1;

    int ti, tj;
    tile_of(blockIdx.x, g.tiles_i, g.tiles_j, ti, tj);
    const int64_t i0 = (int64_t)ti * kBM;
    const int64_t j0 = (int64_t)tj * BN;
    const int z = blockIdx.y;
    const int kt_begin = (int)(((int64_t)g.ktiles * z) / g.splits);
    const int kt_end = (int)(((int64_t)g.ktiles * (z + 1)) / g.splits);

    // ---- global load mapping: thread -> row tid/8 (+32p), 16-byte chunk tid%8
    const int lrow = tid >> 3, lchunk = tid & 7;
    const int sw_st = (lchunk ^ ((lrow >> 1) & 7)) << 4;
    const bool a_hi_ok = (i0 + 128) < g.I;     // I is a multiple of 128
    const bool b_hi_ok = (BN <= 128) || (j0 + 128) < g.J;
    const uint8_t* gA = g.a + (i0 + lrow) * g.K + lchunk * 16;
    const uint8_t* gB = g.b + (j0 + lrow) * g.K + lchunk * 16;

    u32x4 ra[APASS], rb[BPASS];
#define FP8K_LOAD_TILE(kt)                                                                  \
    do {                                                                                    \
        const int64_t koff_ = (int64_t)(kt) * kBK;                                          \
        _Pragma("unroll") for (int p = 0; p < APASS; p++) {                                 \
            const int pr = (p >= 4 && !a_hi_ok) ? p - 4 : p;                                \
            ra[p] = *reinterpret_cast<const u32x4*>(gA + (int64_t)pr * 32 * g.K + koff_);   \
        }                                                                                   \
        _Pragma("unroll") for (int p = 0; p < BPASS; p++) {                                 \
            const int pr = (p >= 4 && !b_hi_ok) ? p - 4 : p;                                \
            rb[p] = *reinterpret_cast<const u32x4*>(gB + (int64_t)pr * 32 * g.K + koff_);   \
        }                                                                                   \
    } while (0)
#define FP8K_STORE_TILE(stage)                                                              \
    do {                                                                                    \
        uint8_t* sA_ = smem + (stage) * STAGE;                                              \
        uint8_t* sB_ = sA_ + A_BYTES;                                                       \
        _Pragma("unroll") for (int p = 0; p < APASS; p++)                                   \
            *reinterpret_cast<u32x4*>(sA_ + (lrow + 32 * p) * kBK + sw_st) = ra[p];         \
        _Pragma("unroll") for (int p = 0; p < BPASS; p++)                                   \
            *reinterpret_cast<u32x4*>(sB_ + (lrow + 32 * p) * kBK + sw_st) = rb[p];         \
    } while (0)

    v16f acc[4][WNJ];
#pragma unroll
    for (int mi = 0; mi < 4; mi++)
#pragma unroll
        for (int nj = 0; nj < WNJ; nj++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[mi][nj][v] = 0.0f;

    const int arow = wi * 128 + (lane & 31);
    const int brow = wj * (WNJ * 32) + (lane & 31);
    // rows (i) and column runs (j) owned by this lane in the accumulators
    const int64_t my_i = i0 + arow;               // + mi*32
    const int64_t my_j = j0 + wj * (WNJ * 32) + 4 * (lane >> 5);   // + nj*32 + 8q + r

    // block-scale pointers
    const bool sb_per_row = BLOCK && g.sb.group == 1;

    if (kt_begin < kt_end) {
        FP8K_LOAD_TILE(kt_begin);
        FP8K_STORE_TILE(0);
    }
    __syncthreads();

    for (int kt = kt_begin; kt < kt_end; kt++) {
        const int cur = (kt - kt_begin) & 1;
        const bool more = kt + 1 < kt_end;
        float sa_v[4];
        float sb_u = 0.0f;
        float sb_v[WNJ][16];
        if constexpr (BLOCK) {
#pragma unroll
            for (int mi = 0; mi < 4; mi++)
            {
                // rows past I (upper half of a last, half-full tile) read row I-1's scale
                const int64_t ii = my_i + mi * 32 < g.I ? my_i + mi * 32 : g.I - 1;
                sa_v[mi] = g.sa.sinv[(ii / g.sa.group) * g.sa.stride_r + (int64_t)kt * g.sa.stride_kb];
            }
            if (sb_per_row) {
#pragma unroll
                for (int nj = 0; nj < WNJ; nj++)
#pragma unroll
                    for (int v = 0; v < 16; v++)
                    {
                        int64_t jj = my_j + nj * 32 + 8 * (v >> 2) + (v & 3);
                        jj = jj < g.J ? jj : g.J - 1;
                        sb_v[nj][v] = g.sb.sinv[jj * g.sb.stride_r + (int64_t)kt * g.sb.stride_kb];
                    }
            } else {
                sb_u = g.sb.sinv[((j0 + wj * (WNJ * 32)) / g.sb.group) * g.sb.stride_r + (int64_t)kt * g.sb.stride_kb];
            }
        }
        if (more) FP8K_LOAD_TILE(kt + 1);

        const uint8_t* sA = smem + cur * STAGE;
        const uint8_t* sB = sA + A_BYTES;
        if constexpr (!BLOCK) {
#pragma unroll
            for (int kk = 0; kk < 2; kk++) {
                v8i af[4], bf[WNJ];
#pragma unroll
                for (int mi = 0; mi < 4; mi++) af[mi] = lds_frag(sA, arow + mi * 32, kk, lane);
#pragma unroll
                for (int nj = 0; nj < WNJ; nj++) bf[nj] = lds_frag(sB, brow + nj * 32, kk, lane);
#pragma unroll
                for (int mi = 0; mi < 4; mi++)
#pragma unroll
                    for (int nj = 0; nj < WNJ; nj++) acc[mi][nj] = mfma<FA, FB>(bf[nj], af[mi], acc[mi][nj]);
            }
        } else {
            v8i af[2][4], bf[2][WNJ];
#pragma unroll
            for (int kk = 0; kk < 2; kk++) {
#pragma unroll
                for (int mi = 0; mi < 4; mi++) af[kk][mi] = lds_frag(sA, arow + mi * 32, kk, lane);
#pragma unroll
                for (int nj = 0; nj < WNJ; nj++) bf[kk][nj] = lds_frag(sB, brow + nj * 32, kk, lane);
            }
            const v16f zero = {};
#pragma unroll
            for (int mi = 0; mi < 4; mi++)
#pragma unroll
                for (int nj = 0; nj < WNJ; nj++) {
                    v16f p = mfma<FA, FB>(bf[0][nj], af[0][mi], zero);
                    p = mfma<FA, FB>(bf[1][nj], af[1][mi], p);
                    if (sb_per_row) {
#pragma unroll
                        for (int v = 0; v < 16; v++)
                            acc[mi][nj][v] = __builtin_fmaf(p[v], sa_v[mi] * sb_v[nj][v], acc[mi][nj][v]);
                    } else {
                        const float t = sa_v[mi] * sb_u;
#pragma unroll
                        for (int v = 0; v < 16; v++) acc[mi][nj][v] = __builtin_fmaf(p[v], t, acc[mi][nj][v]);
                    }
                }
        }
        if (more) FP8K_STORE_TILE(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue -------------------------------------------------------
    if (g.splits > 1) {
        float* out = g.part + (int64_t)z * g.I * g.J;
#pragma unroll
        for (int mi = 0; mi < 4; mi++) {
            const int64_t i = my_i + mi * 32;
            if (i >= g.I) continue;
#pragma unroll
            for (int nj = 0; nj < WNJ; nj++)
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const int64_t j = my_j + nj * 32 + 8 * q;
                    if (j < g.J)
                        *reinterpret_cast<float4*>(out + i * g.J + j) =
                            make_float4(acc[mi][nj][4 * q], acc[mi][nj][4 * q + 1], acc[mi][nj][4 * q + 2], acc[mi][nj][4 * q + 3]);
                }
        }
        return;
    }

    float t = 1.0f;
    if constexpr (!BLOCK) t = g.sa.sinv[0] * g.sb.sinv[0];
    // stage the bf16 tile in LDS: row stride BN*2 bytes, 16-byte chunk c of
    // row r stored at chunk c ^ (r % CH)
    constexpr int CH = BN / 8;
    uint8_t* sC = smem;
#pragma unroll
    for (int mi = 0; mi < 4; mi++)
#pragma unroll
        for (int nj = 0; nj < WNJ; nj++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int r = arow + mi * 32;
                const int col = wj * (WNJ * 32) + nj * 32 + 8 * q;       // chunk-aligned
                const int chunk = col >> 3;
                const int off = r * (BN * 2) + ((chunk ^ (r & (CH - 1))) << 4) + (lane >> 5) * 8;
                const __bf16 h0 = (__bf16)(acc[mi][nj][4 * q] * t);
                const __bf16 h1 = (__bf16)(acc[mi][nj][4 * q + 1] * t);
                const __bf16 h2 = (__bf16)(acc[mi][nj][4 * q + 2] * t);
                const __bf16 h3 = (__bf16)(acc[mi][nj][4 * q + 3] * t);
                uint2 w;
                w.x = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
                w.y = (uint32_t)__builtin_bit_cast(uint16_t, h2) | ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
                *reinterpret_cast<uint2*>(sC + off) = w;
            }
    __syncthreads();
    // write rows: CH chunks of 16 bytes per row
    constexpr int ROWS_PER_PASS = kThreads / CH;
#pragma unroll 4
    for (int r = tid / CH; r < kBM; r += ROWS_PER_PASS) {
        const int c = tid % CH;
        if (i0 + r >= g.I) break;
        if (j0 + c * 8 >= g.J) continue;
        const uint4 w = *reinterpret_cast<const uint4*>(sC + r * (BN * 2) + ((c ^ (r & (CH - 1))) << 4));
        *reinterpret_cast<uint4*>(g.c + (i0 + r) * g.J + j0 + c * 8) = w;
    }
}

#undef FP8K_LOAD_TILE
#undef FP8K_STORE_TILE

// Sum split-K partials in split order, apply the tensorwise factor, bf16.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits, int64_t n4,
                                                            int64_t IJ, const float* sa, const float* sb,
                                                            int tensorwise, uint16_t* __restrict__ c) {
    const float t = tensorwise ? sa[0] * sb[0] : 1.0f;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
        float4 s = reinterpret_cast<const float4*>(part)[i];
        for (int z = 1; z < splits; z++) {
            const float4 p = reinterpret_cast<const float4*>(part + (int64_t)z * IJ)[i];
            s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
        }
        if (tensorwise) { s.x *= t; s.y *= t; s.z *= t; s.w *= t; }
        const __bf16 h0 = (__bf16)s.x, h1 = (__bf16)s.y, h2 = (__bf16)s.z, h3 = (__bf16)s.w;
        uint2 w;
        w.x = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        w.y = (uint32_t)__builtin_bit_cast(uint16_t, h2) | ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
        reinterpret_cast<uint2*>(c)[i] = w;
    }
}

static int block_n(bool block) { return block ? 128 : 256; }

int gemm_splits(int64_t I, int64_t J, int64_t K, bool block) {
    const int64_t tiles = ((I + kBM - 1) / kBM) * ((J + block_n(block) - 1) / block_n(block));
    const int64_t ktiles = K / kBK;
    // aim for >= 2 workgroups per CU (256 CUs), keep >= 8 K tiles per split
    int64_t s = 1;
    while (tiles * s < 512 && ktiles / (s * 2) >= 8 && s < 64) s *= 2;
    return (int)s;
}

size_t gemm_ws_bytes(int64_t I, int64_t J, int64_t K) {
    const int s = gemm_splits(I, J, K, false) > gemm_splits(I, J, K, true) ? gemm_splits(I, J, K, false)
                                                                            : gemm_splits(I, J, K, true);
    return s > 1 ? (size_t)s * (size_t)I * (size_t)J * sizeof(float) : 0;
}

hipError_t launch_gemm(const GemmLaunch& l, hipStream_t stream) {
    const bool block = l.sa.group != 0;
    const int bn = block_n(block);
    GemmArgs g;
    g.a = static_cast<const uint8_t*>(l.a);
    g.b = static_cast<const uint8_t*>(l.b);
    g.sa = l.sa;
    g.sb = l.sb;
    g.I = l.I;
    g.J = l.J;
    g.K = l.K;
    g.c = static_cast<uint16_t*>(l.c);
    g.part = static_cast<float*>(l.ws);
    g.splits = gemm_splits(l.I, l.J, l.K, block);
    g.tiles_i = (int)((l.I + kBM - 1) / kBM);
    g.tiles_j = (int)((l.J + bn - 1) / bn);
    g.ktiles = (int)(l.K / kBK);
    const dim3 grid((unsigned)(g.tiles_i * g.tiles_j), (unsigned)g.splits);
#define FP8K_GEMM(FA, FB, BL) hipLaunchKernelGGL((gemm_kernel<FA, FB, BL>), grid, dim3(kThreads), 0, stream, g)
    if (l.fa == 0 && l.fb == 0) { if (block) FP8K_GEMM(0, 0, true); else FP8K_GEMM(0, 0, false); }
    else if (l.fa == 1 && l.fb == 0) { if (block) FP8K_GEMM(1, 0, true); else FP8K_GEMM(1, 0, false); }
    else if (l.fa == 0 && l.fb == 1) { if (block) FP8K_GEMM(0, 1, true); else FP8K_GEMM(0, 1, false); }
    else { if (block) FP8K_GEMM(1, 1, true); else FP8K_GEMM(1, 1, false); }
#undef FP8K_GEMM
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || g.splits == 1) return e;
    const int64_t n4 = l.I * l.J / 4;
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const float*)g.part, g.splits, n4, l.I * l.J, l.sa.sinv, l.sb.sinv, block ? 0 : 1, g.c);
    return hipGetLastError();
}

}  // namespace fp8k
