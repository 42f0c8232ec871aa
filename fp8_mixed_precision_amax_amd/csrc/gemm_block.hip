// Block-scaled FP8 GEMM with per-row factors on both operands (1x128 x 1x128
// blocks: the weight gradient of the Float8BlockScaling linear),
// C[i][j] = sum_kb (sA[i][kb] sB[j][kb]) P_kb[i][j], P_kb[i][j] = sum_{k in kb}
// A[i][k] B[j][k] over each 128-long contraction block kb, on the gfx950
// matrix cores (BF16 output, or fp32 partial sums for split-K).  A B operand
// with 128x128-block factors goes to gemm_block_wide.hip instead.
//
// Method: the Float8BlockScaling recipe (TransformerEngine issue 2852, the
// question and its expected behaviour) quantizes activations and gradients in
// 1x128 blocks and weights in 128x128 blocks; the GEMMs of the FP8 linear
// ("Native FP8 MLP reconstruction", implementation paragraph) take FP8
// operands and accumulate in fp32.  Every 128-block's fp32 partial sum P_kb
// is multiplied by the product of its two dequantisation factors and added to
// an fp32 accumulator ("promotion"): acc = fma(P_kb, sA * sB, acc).
//
// Design
//  - persistent: one workgroup per CU walks work items (256 x 128 output
//    tile, split-K slice) dealt XCD by XCD and rastered in groups of tile
//    rows, as the tensorwise kernel does.
//  - 8 waves, two per SIMD, wave tile 64 x 64 (2 x 2 blocks of
//    v_mfma_f32_32x32x64_f8f6f4): 64 accumulators plus 64 registers of block
//    partial sums fit two waves per SIMD.
//  - one stage = one 128-block: A 256 x 128 B, B 128 x 128 B and the fp32
//    factors of its 256 + 128 rows, streamed HBM -> LDS by LDS-DMA (buffer
//    loads through resources based at the tile: rows past I read as zero);
//    3 stages, 2 in flight.
//  - promotion overlaps the matrix cores: the partial sums of blocks (0, *)
//    are promoted right after the stage's last MFMAs issue, those of blocks
//    (1, *) while the next stage's first MFMAs run; every element is
//    promoted with its own sA * sB (a multiply and an FMA).  A 256 x 256 tile
//    (gemm_block_wide.hip's) measured no faster for this case: the two VALU
//    operations per element, not the memory path, bound it.
//  - stage hand-off and the inline-assembly LDS reads follow the tensorwise
//    kernel: exact s_waitcnt vmcnt(n) on the wave's own DMA, then s_barrier;
//    every read group is issued and waited for inside one asm statement.
//    The DMA two stages ahead goes out after the step's first three MFMAs,
//    not right after the barrier, so the SIMD's two waves leave the barrier
//    issuing MFMAs (8192 x 8192 x 16384 1.322 -> 1.270 ms).
#include "device.hpp"
#include "gemm_common.hpp"
#include "internal.hpp"

namespace fp8k {
namespace block {

constexpr int BM = 256, BN = 128, BK = 128;
constexpr int S = 3;                        // LDS stages
constexpr int D = 2;                        // stages in flight ahead of the one read
constexpr int NW = 8;                       // waves
constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;
constexpr int SC_A = A_BYTES + B_BYTES;     // fp32 factors of the A rows
constexpr int SC_B = SC_A + BM * 4;         // fp32 factors of the B rows
constexpr int STAGE = 51200;                // 49.5 KiB used, padded to 1 KiB
constexpr int LA = A_BYTES / 1024 / NW;     // LDS-DMA instructions per wave per stage (A)
constexpr int LB = B_BYTES / 1024 / NW;     // (B)
constexpr int L = LA + LB + 1;              // + one 4-byte DMA of factors
constexpr int RPK = 1024 / BK;              // rows per 1 KiB DMA block
constexpr int CPR = BK / 16;                // 16-byte chunks per LDS row
static_assert(SC_B + BN * 4 <= STAGE && STAGE % 1024 == 0, "stage");
constexpr int SLICE = 1024;                 // per-wave epilogue slice: 8 rows x 64 bf16
static_assert(S * STAGE + NW * SLICE <= 160 * 1024, "LDS");
static_assert(LA % 2 == 0 && LB % 2 == 0, "odd DMA blocks alternate the swizzle");

struct Args {
    const uint8_t* a;
    const uint8_t* b;
    GemmScale sa, sb;
    int64_t I, J, K;
    uint16_t* c;
    float* part;          // split-K partials [splits][I][J]
    int splits, tiles_i, tiles_j, ktiles, items;
    int gi;               // tile rows per raster group
};

struct Item {
    int ti, tj, z, kb, ke;   // kb, ke: 128-blocks of the contraction
};

__device__ __forceinline__ bool item_at(const Args& g, int r, Item& it) {
    const int G = gridDim.x, b = blockIdx.x;
    const int Lg = r * G + ((G & 7) == 0 ? (b & 7) * (G >> 3) + (b >> 3) : b);
    if (Lg >= g.items) return false;
    const int tiles = g.tiles_i * g.tiles_j;
    const int z = Lg / tiles, t = Lg - z * tiles;
    const int GI = g.gi;
    const int per_group = GI * g.tiles_j, grp = t / per_group, local = t - grp * per_group;
    int rows = g.tiles_i - grp * GI;
    rows = rows < GI ? rows : GI;
    it.ti = grp * GI + local % rows;
    it.tj = local / rows;
    it.z = z;
    // ktiles < 2^16 and splits <= 64 (contraction below 2^23): 32-bit math
    it.kb = g.ktiles * z / g.splits;
    it.ke = g.ktiles * (z + 1) / g.splits;
    return true;
}

// s_waitcnt vmcnt(n) for a runtime n (rounded down to a supported value)
__device__ __forceinline__ void wait_vm_n(int n) {
    if (n == L) wait_vm<L>();
    else if (n == L + 8) wait_vm<L + 8>();
    else if (n == L + 16) wait_vm<L + 16>();
    else if (n >= 63) wait_vm<63>();
    else if (n >= 32) wait_vm<32>();
    else if (n >= 16) wait_vm<16>();
    else if (n >= 8) wait_vm<8>();
    else wait_vm<0>();
}

// First half of a 128-block: A fragments of rows +0 / +32 and B fragments of
// rows +0 / +32 (32 bytes each: chunks at x0 and x1), and the A factors of
// the lane's two rows; issued and waited for in one asm statement.
__device__ __forceinline__ void read_half_sa(v8i (&fa)[2], v8i (&fb)[2], float& sa0, float& sa1, uint32_t a0,
                                             uint32_t a1, uint32_t b0, uint32_t b1, uint32_t pa) {
    u32x4 x0, x1, x2, x3, y0, y1, y2, y3;
    asm volatile(
        "ds_read_b128 %0, %10 offset:0\n\t"
        "ds_read_b128 %1, %11 offset:0\n\t"
        "ds_read_b128 %2, %10 offset:4096\n\t"
        "ds_read_b128 %3, %11 offset:4096\n\t"
        "ds_read_b128 %4, %12 offset:0\n\t"
        "ds_read_b128 %5, %13 offset:0\n\t"
        "ds_read_b128 %6, %12 offset:4096\n\t"
        "ds_read_b128 %7, %13 offset:4096\n\t"
        "ds_read_b32 %8, %14 offset:0\n\t"
        "ds_read_b32 %9, %14 offset:128\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3), "=&v"(y0), "=&v"(y1), "=&v"(y2), "=&v"(y3), "=&v"(sa0),
          "=&v"(sa1)
        : "v"(a0), "v"(a1), "v"(b0), "v"(b1), "v"(pa)
        : "memory");
    fa[0] = __builtin_bit_cast(v8i, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
    fa[1] = __builtin_bit_cast(v8i, __builtin_shufflevector(x2, x3, 0, 1, 2, 3, 4, 5, 6, 7));
    fb[0] = __builtin_bit_cast(v8i, __builtin_shufflevector(y0, y1, 0, 1, 2, 3, 4, 5, 6, 7));
    fb[1] = __builtin_bit_cast(v8i, __builtin_shufflevector(y2, y3, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Second half of a 128-block with the B factors of the lane's 32 columns
// (per-row B factors): float4 q of column block nj holds columns 8q .. 8q+3
// (lanes 0..31) or 8q+4 .. 8q+7 (lanes 32..63) of the block.
__device__ __forceinline__ void read_half_sb_rows(v8i (&fa)[2], v8i (&fb)[2], f32x4 (&sb)[2][4], uint32_t a0,
                                                  uint32_t a1, uint32_t b0, uint32_t b1, uint32_t pb) {
    u32x4 x0, x1, x2, x3, y0, y1, y2, y3;
    f32x4 g0, g1, g2, g3, g4, g5, g6, g7;
    asm volatile(
        "ds_read_b128 %0, %16 offset:0\n\t"
        "ds_read_b128 %1, %17 offset:0\n\t"
        "ds_read_b128 %2, %16 offset:4096\n\t"
        "ds_read_b128 %3, %17 offset:4096\n\t"
        "ds_read_b128 %4, %18 offset:0\n\t"
        "ds_read_b128 %5, %19 offset:0\n\t"
        "ds_read_b128 %6, %18 offset:4096\n\t"
        "ds_read_b128 %7, %19 offset:4096\n\t"
        "ds_read_b128 %8, %20 offset:0\n\t"
        "ds_read_b128 %9, %20 offset:32\n\t"
        "ds_read_b128 %10, %20 offset:64\n\t"
        "ds_read_b128 %11, %20 offset:96\n\t"
        "ds_read_b128 %12, %20 offset:128\n\t"
        "ds_read_b128 %13, %20 offset:160\n\t"
        "ds_read_b128 %14, %20 offset:192\n\t"
        "ds_read_b128 %15, %20 offset:224\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3), "=&v"(y0), "=&v"(y1), "=&v"(y2), "=&v"(y3), "=&v"(g0),
          "=&v"(g1), "=&v"(g2), "=&v"(g3), "=&v"(g4), "=&v"(g5), "=&v"(g6), "=&v"(g7)
        : "v"(a0), "v"(a1), "v"(b0), "v"(b1), "v"(pb)
        : "memory");
    fa[0] = __builtin_bit_cast(v8i, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
    fa[1] = __builtin_bit_cast(v8i, __builtin_shufflevector(x2, x3, 0, 1, 2, 3, 4, 5, 6, 7));
    fb[0] = __builtin_bit_cast(v8i, __builtin_shufflevector(y0, y1, 0, 1, 2, 3, 4, 5, 6, 7));
    fb[1] = __builtin_bit_cast(v8i, __builtin_shufflevector(y2, y3, 0, 1, 2, 3, 4, 5, 6, 7));
    sb[0][0] = g0;
    sb[0][1] = g1;
    sb[0][2] = g2;
    sb[0][3] = g3;
    sb[1][0] = g4;
    sb[1][1] = g5;
    sb[1][2] = g6;
    sb[1][3] = g7;
}

// acc += P * (sa * sb[column]) for one 32 x 32 block
__device__ __forceinline__ void promote_rows(v16f& acc, const v16f& p, float sa, const f32x4 (&sb)[4]) {
#pragma unroll
    for (int q = 0; q < 4; q++) {
        acc[4 * q + 0] = __builtin_fmaf(p[4 * q + 0], sa * sb[q].x, acc[4 * q + 0]);
        acc[4 * q + 1] = __builtin_fmaf(p[4 * q + 1], sa * sb[q].y, acc[4 * q + 1]);
        acc[4 * q + 2] = __builtin_fmaf(p[4 * q + 2], sa * sb[q].z, acc[4 * q + 2]);
        acc[4 * q + 3] = __builtin_fmaf(p[4 * q + 3], sa * sb[q].w, acc[4 * q + 3]);
    }
}
template <int FA, int FB, bool NT>
__global__ __launch_bounds__(NW * 64, 1) void gemm_block_kernel(Args g) {
    // separate objects: the epilogue's LDS traffic never aliases the stages
    __shared__ __attribute__((aligned(1024))) uint8_t smem[S * STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t sepi[NW * SLICE];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int wi = wave & 3, wj = wave >> 2;
    const uint32_t K = (uint32_t)g.K;

    // ---- load cursor (uniform) ---------------------------------------------
    int l_round = 0;
    Item l_it;
    bool l_ok = item_at(g, 0, l_it);
    __amdgpu_buffer_rsrc_t ra = make_rsrc(g.a, 0);
    __amdgpu_buffer_rsrc_t rb = ra;
    // lane offset inside an 8-row DMA block: row lane/8, swizzled chunk; the
    // odd blocks of a wave start at a row with bit 3 set, whose swizzle
    // differs in chunk bit 2
    const int lrow = lane / CPR;
    const uint32_t loff0 = (uint32_t)lrow * K + (uint32_t)(((lane % CPR) ^ swz<BK>(lrow)) * 16);
    const uint32_t loff1 = (uint32_t)lrow * K + (uint32_t)(((lane % CPR) ^ swz<BK>(lrow + RPK)) * 16);
    const uint32_t a_row0 = (uint32_t)(wave * LA * RPK), b_row0 = (uint32_t)(wave * LB * RPK);
    uint32_t l_kso = 0;   // byte offset of the next stage's 128-block along K
    int l_left = 0;       // stages left in the load item
    // factor DMA: waves 0-3 move A rows 64w .. 64w+63, waves 4-7 B rows
    // 64(w&1) .. (waves 6, 7 repeat 4, 5: same values to the same place)
    const bool sc_is_a = wave < 4;
    const GemmScale& gs = sc_is_a ? g.sa : g.sb;
    const int sc_row = (sc_is_a ? wave * 64 : (wave & 1) * 64) + lane;
    const uint32_t sc_lds = (uint32_t)(sc_is_a ? SC_A + wave * 256 : SC_B + (wave & 1) * 256);
    const float* l_ps = g.sa.sinv;
    auto set_load_item = [&]() __attribute__((always_inline)) {
        const int64_t i0 = (int64_t)l_it.ti * BM, j0 = (int64_t)l_it.tj * BN;
        ra = make_rsrc(g.a + i0 * g.K, (g.I - i0 < BM ? g.I - i0 : BM) * g.K);
        rb = make_rsrc(g.b + j0 * g.K, BN * g.K);
        l_kso = (uint32_t)l_it.kb * BK;
        l_left = l_it.ke - l_it.kb;
        int64_t r = (sc_is_a ? i0 : j0) + sc_row;
        const int64_t rmax = (sc_is_a ? g.I : g.J) - 1;
        r = r < rmax ? r : rmax;
        l_ps = gs.sinv + (gs.group == 1 ? r : r >> 7) * gs.stride_r + (int64_t)l_it.kb * gs.stride_kb;   // group 1 or 128
    };
    if (l_ok) set_load_item();
    const uint32_t smem0 = lds_off(smem);
    uint32_t dma_off = 0;   // stage buffer the next DMA fills
    auto issue_stage = [&]() __attribute__((always_inline)) {
        const uint32_t dA = smem0 + dma_off + (uint32_t)(wave * LA * 1024);
        const uint32_t dB = smem0 + dma_off + (uint32_t)(A_BYTES + wave * LB * 1024);
#pragma unroll
        for (int p = 0; p < LA; p++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (__attribute__((address_space(3))) void*)(uintptr_t)(dA + p * 1024), 16, (p & 1) ? loff1 : loff0,
                __builtin_amdgcn_readfirstlane((a_row0 + (uint32_t)(p * RPK)) * K + l_kso), 0, 0);
#pragma unroll
        for (int p = 0; p < LB; p++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (__attribute__((address_space(3))) void*)(uintptr_t)(dB + p * 1024), 16, (p & 1) ? loff1 : loff0,
                __builtin_amdgcn_readfirstlane((b_row0 + (uint32_t)(p * RPK)) * K + l_kso), 0, 0);
        __builtin_amdgcn_global_load_lds(l_ps, (__attribute__((address_space(3))) void*)(uintptr_t)(smem0 + dma_off + sc_lds),
                                         4, 0, 0);
        dma_off = dma_off + STAGE == S * STAGE ? 0 : dma_off + STAGE;
        if (--l_left == 0) {
            if (l_ok && item_at(g, l_round + 1, l_it)) {
                l_round++;
                set_load_item();
            } else {
                // past the last item: keep re-reading its last stage into
                // buffers nobody reads, so every step issues the same loads
                l_ok = false;
                l_left = 1;
            }
        } else {
            l_kso += BK;
            l_ps += gs.stride_kb;
        }
    };

    // ---- prologue: D stages in flight ----------------------------------------
#pragma unroll
    for (int s = 0; s < D; s++) issue_stage();

    int c_round = 0;
    Item c_it;
    bool c_ok = item_at(g, 0, c_it);
    int st_cur = 0;   // epilogue stores issued since the last stage wait

    const int frow = lane & 31;
    const int arow = wi * 64 + frow, brow = wj * 64 + frow;
    const int ch = (lane >> 5) * 2;
    // fragment rows in a stage: chunk ch (ch+1 at ^16; the second 64-long
    // half at ^64), +4096 bytes per 32 rows
    const uint32_t offA = (uint32_t)(arow * BK + ((ch ^ swz<BK>(arow)) << 4));
    const uint32_t offB = (uint32_t)(A_BYTES + brow * BK + ((ch ^ swz<BK>(brow)) << 4));
    const uint32_t offSA = (uint32_t)(SC_A + arow * 4);
    const uint32_t epi_slice = lds_off(sepi) + (uint32_t)(wave * SLICE);
    const uint32_t offSB = (uint32_t)(SC_B + (wj * 64 + 4 * (lane >> 5)) * 4);

    v16f acc[2][2], p[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; mi++)
#pragma unroll
        for (int nj = 0; nj < 2; nj++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                acc[mi][nj][v] = 0.0f;
                p[mi][nj][v] = 0.0f;
            }
    const v16f vzero = {};
    // factors of the stage whose blocks (1, *) still wait for promotion
    float sa1_prev = 0.0f;
    f32x4 sbr_prev[2][4];
#pragma unroll
    for (int nj = 0; nj < 2; nj++)
#pragma unroll
        for (int q = 0; q < 4; q++) sbr_prev[nj][q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    uint32_t rd_off = 0;   // stage buffer the next step reads

    // One 128-block.  Its stage must have landed everywhere: wait for this
    // wave's DMA of it (the ops issued after it are the next stage's DMA and
    // the epilogue stores since), then the barrier, which also retires every
    // wave's reads of the buffer the DMA below overwrites (all LDS reads are
    // waited for inside their asm statements).
#define FP8K_PROMOTE(MI, NJ, SA, SBR)                                  \
    do {                                                                    \
        promote_rows(acc[MI][NJ], p[MI][NJ], SA, SBR[NJ]);                  \
    } while (0)
#define FP8K_STEP(DEFER)                                                                           \
    do {                                                                                           \
        wait_vm_n(L + st_cur);                                                                     \
        st_cur = 0;                                                                                \
        asm volatile("s_barrier" ::: "memory");                                                    \
        const uint32_t sb_ = smem0 + rd_off;                                                       \
        rd_off = rd_off + STAGE == S * STAGE ? 0 : rd_off + STAGE;                                 \
        const uint32_t a0_ = sb_ + offA, a1_ = a0_ ^ 16u, b0_ = sb_ + offB, b1_ = b0_ ^ 16u;       \
        v8i fa_[2], fb_[2];                                                                        \
        float sa0_, sa1_;                                                                          \
        read_half_sa(fa_, fb_, sa0_, sa1_, a0_, a1_, b0_, b1_, sb_ + offSA);                       \
        __builtin_amdgcn_sched_barrier(0);                                                         \
        /* each promotion issues behind one MFMA (MFMA first) */                                   \
        p[0][0] = mfma<FA, FB>(fb_[0], fa_[0], vzero);                                             \
        if (DEFER) FP8K_PROMOTE(1, 0, sa1_prev, sbr_prev);                               \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                         \
        __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);                                        \
        __builtin_amdgcn_sched_barrier(0);                                                         \
        p[0][1] = mfma<FA, FB>(fb_[1], fa_[0], vzero);                                             \
        if (DEFER) FP8K_PROMOTE(1, 1, sa1_prev, sbr_prev);                               \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                         \
        __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);                                        \
        __builtin_amdgcn_sched_barrier(0);                                                         \
        p[1][0] = mfma<FA, FB>(fb_[0], fa_[1], vzero);                                             \
        issue_stage();                                                                             \
        p[1][1] = mfma<FA, FB>(fb_[1], fa_[1], vzero);                                             \
        __builtin_amdgcn_sched_barrier(0);                                                         \
        read_half_sb_rows(fa_, fb_, sbr_prev, a0_ ^ 64u, a1_ ^ 64u, b0_ ^ 64u, b1_ ^ 64u, sb_ + offSB);    \
        __builtin_amdgcn_sched_barrier(0);                                                         \
        p[0][0] = mfma<FA, FB>(fb_[0], fa_[0], p[0][0]);                                           \
        p[0][1] = mfma<FA, FB>(fb_[1], fa_[0], p[0][1]);                                           \
        __builtin_amdgcn_sched_barrier(0);                                                         \
        /* blocks (0, *) completed two MFMAs earlier */                                            \
        p[1][0] = mfma<FA, FB>(fb_[0], fa_[1], p[1][0]);                                           \
        FP8K_PROMOTE(0, 0, sa0_, sbr_prev);                                              \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                         \
        __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);                                        \
        __builtin_amdgcn_sched_barrier(0);                                                         \
        p[1][1] = mfma<FA, FB>(fb_[1], fa_[1], p[1][1]);                                           \
        FP8K_PROMOTE(0, 1, sa0_, sbr_prev);                                              \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                         \
        __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);                                        \
        __builtin_amdgcn_sched_barrier(0);                                                         \
        sa1_prev = sa1_;                                                                           \
    } while (0)

    // write one item's accumulators; returns the vector-memory stores issued
    auto epilogue = [&](const Item& it) __attribute__((always_inline)) -> int {
        const int64_t i0 = (int64_t)it.ti * BM, j0 = (int64_t)it.tj * BN;
        // validity is uniform per wave (I is a multiple of 128, J of BN)
        if (i0 + wi * 64 >= g.I) return 0;
        const int64_t my_i = i0 + arow, my_j = j0 + wj * 64 + 4 * (lane >> 5);
        if (g.splits > 1) {
            float* out = g.part + (int64_t)it.z * g.I * g.J + my_i * g.J + my_j;
#pragma unroll
            for (int mi = 0; mi < 2; mi++)
#pragma unroll
                for (int nj = 0; nj < 2; nj++)
#pragma unroll
                    for (int q = 0; q < 4; q++)
                        *reinterpret_cast<float4*>(out + (int64_t)mi * 32 * g.J + nj * 32 + 8 * q) =
                            make_float4(acc[mi][nj][4 * q], acc[mi][nj][4 * q + 1], acc[mi][nj][4 * q + 2],
                                        acc[mi][nj][4 * q + 3]);
            return 16;
        }
        // bf16 output through the wave's LDS slice, 8 rows at a time: row r
        // holds 64 columns as 16-byte chunks, chunk c at (c ^ r) (the writes
        // of 8 rows hit distinct banks); each store instruction then writes 8
        // whole 128-byte row segments.  A wave's LDS operations execute in
        // order, so a pass's read-back sees its writes and the next pass's
        // writes follow the read.
        uint2 w[2][2][4];
#pragma unroll
        for (int mi = 0; mi < 2; mi++)
#pragma unroll
            for (int nj = 0; nj < 2; nj++)
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    w[mi][nj][q].x = pack_bf16x2(acc[mi][nj][4 * q], acc[mi][nj][4 * q + 1]);
                    w[mi][nj][q].y = pack_bf16x2(acc[mi][nj][4 * q + 2], acc[mi][nj][4 * q + 3]);
                }
        const int rw = frow & 7, gw = frow >> 3;          // writer: row in the pass, pass of its row
        const uint32_t wbase = epi_slice + (uint32_t)(rw * 128 + (lane >> 5) * 8);
        const int rr = lane >> 3, kr = lane & 7;          // reader: row, 16-byte chunk
        const uint32_t raddr = epi_slice + (uint32_t)(rr * 128 + ((kr ^ rr) << 4));
        uint8_t* ob = reinterpret_cast<uint8_t*>(g.c + (i0 + wi * 64 + rr) * g.J + j0 + wj * 64) + kr * 16;
#pragma unroll
        for (int mi = 0; mi < 2; mi++)
#pragma unroll
            for (int pg = 0; pg < 4; pg++) {
                if (gw == pg) {
#pragma unroll
                    for (int nj = 0; nj < 2; nj++)
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            const uint32_t wa = wbase + (uint32_t)((((nj * 4 + q) ^ rw) << 4));
                            asm volatile("ds_write_b64 %0, %1" : : "v"(wa), "v"(w[mi][nj][q]) : "memory");
                        }
                }
                u32x4 r;
                asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(raddr) : "memory");
                st_out16<NT>(ob + (int64_t)(mi * 32 + pg * 8) * g.J * 2, r);
            }
        return 8;
    };

    while (c_ok) {
        Item n_it;
        const bool more = item_at(g, c_round + 1, n_it);
        const int nsteps = c_it.ke - c_it.kb;   // >= 1
        FP8K_STEP(false);
        for (int s = 1; s < nsteps; s++) FP8K_STEP(true);
        // the item's last blocks (1, *), then its output
        FP8K_PROMOTE(1, 0, sa1_prev, sbr_prev);
        FP8K_PROMOTE(1, 1, sa1_prev, sbr_prev);
        st_cur += epilogue(c_it);
#pragma unroll
        for (int mi = 0; mi < 2; mi++)
#pragma unroll
            for (int nj = 0; nj < 2; nj++) acc[mi][nj] = vzero;
        c_it = n_it;
        c_ok = more;
        c_round++;
    }
#undef FP8K_STEP
#undef FP8K_PROMOTE
    wait_vm<0>();
}

}  // namespace block

using namespace block;

int gemm_block_splits(int64_t I, int64_t J, int64_t K) {
    const int64_t tiles = ((I + BM - 1) / BM) * ((J + BN - 1) / BN);
    const int64_t kb = K / BK;
    // aim for one work item per CU, keep >= 8 blocks of 128 per slice
    int64_t s = 1;
    while (tiles * s < 256 && kb / (s * 2) >= 8 && s < 64) s *= 2;
    return (int)s;
}

hipError_t launch_gemm_block(const GemmLaunch& l, int splits, hipStream_t stream) {
    Args g;
    g.a = static_cast<const uint8_t*>(l.a);
    g.b = static_cast<const uint8_t*>(l.b);
    g.sa = l.sa;
    g.sb = l.sb;
    g.I = l.I;
    g.J = l.J;
    g.K = l.K;
    g.c = static_cast<uint16_t*>(l.c);
    g.part = static_cast<float*>(l.ws);
    g.splits = splits;
    g.tiles_i = (int)((l.I + BM - 1) / BM);
    g.tiles_j = (int)(l.J / BN);
    g.ktiles = (int)(l.K / BK);
    g.items = g.tiles_i * g.tiles_j * splits;
    // raster groups of 8 tile rows: best or within 2 % of the best of
    // 2, 4, 8, 16 on every measured shape (8192 x 8192 x 16384: 1216 -> 1139 us
    // against groups of 2)
    g.gi = 8;
    int grid = cu_count();
    if (grid > g.items) grid = g.items;
    const bool nt = l.K <= kNtMaxContraction;
#define FP8K_LAUNCH(FA, FB)                                                                                    \
    if (nt) hipLaunchKernelGGL((gemm_block_kernel<FA, FB, true>), dim3(grid), dim3(NW * 64), 0, stream, g);  \
    else hipLaunchKernelGGL((gemm_block_kernel<FA, FB, false>), dim3(grid), dim3(NW * 64), 0, stream, g)
    if (l.fa == 0 && l.fb == 0) { FP8K_LAUNCH(0, 0); }
    else if (l.fa == 1 && l.fb == 0) { FP8K_LAUNCH(1, 0); }
    else if (l.fa == 0 && l.fb == 1) { FP8K_LAUNCH(0, 1); }
    else { FP8K_LAUNCH(1, 1); }
#undef FP8K_LAUNCH
    return hipGetLastError();
}

}  // namespace fp8k
