// Block-scaled FP8 GEMM C[i][j] = sum_kb (sA[i][kb] sB[j][kb]) sum_{k in kb}
// A[i][k] B[j][k] on the gfx950 FP8 matrix cores, the split-K reduction shared
// with the tensorwise kernel, and the GEMM dispatcher.
//
// Method ("Native FP8 MLP reconstruction", implementation paragraph): the
// three GEMMs of the FP8 linear take FP8 operands (E4M3 x E4M3 forward,
// E5M2 x E4M3 for both gradients), accumulate at full fp32 precision (no
// fast accumulation) and write BF16.  Block scales (Float8BlockScaling,
// TransformerEngine issue 2852) are applied to every 128-long contraction
// block's partial sum, which is then added to an fp32 accumulator.  The
// tensorwise GEMM (one scale pair, applied in the epilogue) lives in
// gemm_tensor.hip.
//
// Design of the block-scaled kernel (every operand contraction-contiguous):
//  - persistent: one workgroup per CU walks a list of work items (output tile,
//    split-K slice); the software pipeline runs continuously across item
//    boundaries, so the next tile's first K stages stream in while the
//    current tile's epilogue stores go out.
//  - workgroup 256 threads = 4 waves in 2x2, output tile 256x128 (wave tile
//    128x64 = 4x2 v_mfma_f32_32x32x64_f8f6f4 blocks), BK=128 (one scale block
//    per K step), 3 LDS stages; per-block fp32 promotion keeps the
//    accumulators and the block partial sums in VGPRs.
//  - operands move HBM -> LDS with global_load_lds_dwordx4 (no VGPR staging):
//    each instruction fills 1 KiB of LDS at M0 + 16 * lane; the lane picks
//    its global 16-byte chunk so that the LDS rows come out XOR-swizzled
//    (16-byte chunk index ^ f(row)), which makes the fragment reads of 16
//    consecutive rows hit 16 distinct bank groups.  The stage also carries
//    the fp32 factors of its 128-block (4-byte LDS-DMA).
//  - stage hand-off: each wave waits with s_waitcnt vmcnt(n) for its own
//    loads of the stage, then a plain s_barrier (no fence: a workgroup
//    release fence would force vmcnt(0) and drain the prefetch queue).
//  - the B tile is the matrix cores' "A" operand, so each lane's accumulators
//    hold one output row i and runs of 4 consecutive columns j, stored as
//    8-byte bf16 runs.
//  - work items are dealt so that the workgroups on one XCD (the dispatcher
//    deals workgroups round-robin over the 8 XCDs) take consecutive items,
//    rastered in groups of 8 tile rows for L2 reuse of A.
//  - split-K (small outputs with long contractions, e.g. the weight
//    gradient): each slice writes fp32 partials; a reduce kernel sums the
//    slices in fixed order (deterministic), applies the tensorwise factor and
//    rounds to bf16.
#include <type_traits>

#include "gemm_common.hpp"
#include "internal.hpp"

namespace fp8k {

constexpr int kThreads = 256;

// Tile configuration: BM x BN output tile, BK contraction step, S LDS stages,
// WNJ 32-column blocks per wave (wave tile 128 x 32*WNJ), OCC workgroups per CU.
template <int BM_, int BN_, int BK_, int S_, int WNJ_, int OCC_>
struct GemmCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, S = S_, WNJ = WNJ_, OCC = OCC_;
    static_assert(BM == 256 && BN == 2 * WNJ * 32, "4 waves in 2 x 2, wave tile 128 x 32*WNJ");
    static_assert(BK == 64 || BK == 128, "BK");
};
using CfgBlock = GemmCfg<256, 128, 128, 3, 2, 1>;

struct GemmArgs {
    const uint8_t* a;
    const uint8_t* b;
    GemmScale sa, sb;
    int64_t I, J, K;
    uint16_t* c;
    float* part;      // split-K partials [splits][I][J]
    int splits;
    int tiles_i, tiles_j;
    int ktiles;       // K / BK
    int items;        // tiles_i * tiles_j * splits
};

struct Item {
    int ti, tj, z, kb, ke;
};

// r-th item of this workgroup.  Round r covers logical items
// [r*G, (r+1)*G); a workgroup on XCD x = b % 8 takes the x-th eighth of it.
__device__ __forceinline__ bool item_of(const GemmArgs& g, int r, Item& it) {
    const int G = gridDim.x;
    const int b = blockIdx.x;
    const int L = r * G + ((G & 7) == 0 ? (b & 7) * (G >> 3) + (b >> 3) : b);
    if (L >= g.items) return false;
    const int tiles = g.tiles_i * g.tiles_j;
    const int z = L / tiles;
    const int t = L - z * tiles;
    constexpr int GI = 8;
    const int per_group = GI * g.tiles_j;
    const int grp = t / per_group;
    const int local = t - grp * per_group;
    int rows = g.tiles_i - grp * GI;
    rows = rows < GI ? rows : GI;
    it.ti = grp * GI + local % rows;
    it.tj = local / rows;
    it.z = z;
    it.kb = (int)(((int64_t)g.ktiles * z) / g.splits);
    it.ke = (int)(((int64_t)g.ktiles * (z + 1)) / g.splits);
    return true;
}

template <int FA, int FB, bool BLOCK, class C>
__global__ __launch_bounds__(kThreads, C::OCC) void gemm_kernel(GemmArgs g) {
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, S = C::S, WNJ = C::WNJ;
    constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;
    // block mode: the stage also carries the fp32 factors of its 128-block,
    // A rows [BM] then B rows [BN], loaded by 4-byte LDS-DMA
    constexpr int SC_BYTES = BLOCK ? (BM + BN) * 4 : 0;
    constexpr int STAGE = A_BYTES + B_BYTES + SC_BYTES;
    constexpr int LA = A_BYTES / 1024 / 4, LB = B_BYTES / 1024 / 4;
    constexpr int L = LA + LB + (BLOCK ? 2 : 0);   // LDS-DMA instructions per wave per stage
    constexpr int RPK = 1024 / BK;   // rows per 1 KiB LDS block
    constexpr int CPR = BK / 16;     // 16-byte chunks per row
    static_assert(S * STAGE <= 160 * 1024, "LDS");
    static_assert(BLOCK && BK == 128 && WNJ == 2, "block-scaled kernel: BK 128, wave tile 128 x 64");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[S * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wi = wave >> 1, wj = wave & 1;

    // ---- load cursor (runs S-1 stages ahead of the compute cursor) -------
    int l_round = 0, l_kt = 0;
    Item l_it;
    bool l_ok = item_of(g, 0, l_it);
    // Per-lane load addresses.  Instruction p of this wave fills LDS block
    // (wave*LA + p); its rows are those of p = 0 plus p*RPK, and the swizzled
    // chunk is the same for every p (BK = 64) or alternates with p's parity
    // (BK = 128: chunk ^ 4), so one base pointer and one parity delta per
    // operand describe all of them.
    const uint8_t* pa0 = nullptr;   // A rows of p = 0
    const uint8_t* pb0 = nullptr;
    int64_t a_hi = 0, b_hi = 0;      // shift for the upper 128 rows of a half-full tile
    int dchunk = 0;                  // byte delta of odd p (BK = 128)
    const float* psa = nullptr;      // block mode: scale row pointers of this lane
    const float* psb = nullptr;
    {
        const int row0 = lane / CPR;
        const int c0 = (lane % CPR) ^ swz<BK>(row0);
        if (BK == 128) dchunk = (((lane % CPR) ^ swz<BK>(row0 + RPK)) - c0) * 16;
    }
#define FP8K_SET_LOAD_PTRS()                                                              \
    do {                                                                                  \
        const int64_t i0_ = (int64_t)l_it.ti * BM, j0_ = (int64_t)l_it.tj * BN;           \
        const int rowa_ = wave * LA * RPK + lane / CPR;                                   \
        const int rowb_ = wave * LB * RPK + lane / CPR;                                   \
        const int c_ = (lane % CPR) ^ swz<BK>(lane / CPR);                                \
        pa0 = g.a + (i0_ + rowa_) * g.K + c_ * 16;                                        \
        pb0 = g.b + (j0_ + rowb_) * g.K + c_ * 16;                                        \
        /* half-full last tile: rows >= 128 of the tile re-read rows - 128 */             \
        a_hi = (i0_ + 128 >= g.I) ? -128 * g.K : 0;                                       \
        b_hi = (j0_ + 128 >= g.J) ? -128 * g.K : 0;                                       \
        if constexpr (BLOCK) {                                                            \
            /* this lane's scale rows: A row wave*64+lane, B row (wave&1)*64+lane */       \
            int64_t ra_ = i0_ + wave * 64 + lane;                                         \
            ra_ = ra_ < g.I ? ra_ : g.I - 1;                                              \
            int64_t rb_ = j0_ + (wave & 1) * 64 + lane;                                   \
            rb_ = rb_ < g.J ? rb_ : g.J - 1;                                              \
            psa = g.sa.sinv + (ra_ / g.sa.group) * g.sa.stride_r;                         \
            psb = g.sb.sinv + (rb_ / g.sb.group) * g.sb.stride_r;                         \
        }                                                                                 \
    } while (0)
    if (l_ok) {
        l_kt = l_it.kb;
        FP8K_SET_LOAD_PTRS();
    }
    int issued = 0;   // stages issued so far
    // vmcnt bookkeeping (wave-uniform): ops = vector-memory instructions
    // issued so far (LDS-DMA loads and epilogue stores); pendK = value of ops
    // right after the K-th oldest not-yet-consumed stage was issued.
    int ops = 0, npend = 0, pend0 = 0, pend1 = 0, pend2 = 0;
    // row offset (in rows) of instruction p inside this wave's part of the tile
#define FP8K_ROWOFF(p, rows_per_wave, hi)                                                          \
    ((int64_t)(p) * RPK * g.K + (((wave * (rows_per_wave) + (p) * RPK) >= 128) ? (hi) : 0) +          \
     (((p) & 1) ? dchunk : 0))
#define FP8K_ISSUE_STAGE()                                                                         \
    do {                                                                                           \
        uint8_t* st_ = smem + (issued % S) * STAGE;                                                \
        const int64_t koff_ = (int64_t)l_kt * BK;                                                  \
        _Pragma("unroll") for (int p = 0; p < LA; p++)                                             \
            __builtin_amdgcn_global_load_lds(pa0 + koff_ + FP8K_ROWOFF(p, LA * RPK, a_hi),        \
                                             st_ + (wave * LA + p) * 1024, 16, 0, 0);              \
        _Pragma("unroll") for (int p = 0; p < LB; p++)                                             \
            __builtin_amdgcn_global_load_lds(pb0 + koff_ + FP8K_ROWOFF(p, LB * RPK, b_hi),        \
                                             st_ + A_BYTES + (wave * LB + p) * 1024, 16, 0, 0);    \
        if constexpr (BLOCK) {                                                                     \
            __builtin_amdgcn_global_load_lds(psa + (int64_t)l_kt * g.sa.stride_kb,                \
                                             st_ + A_BYTES + B_BYTES + wave * 256, 4, 0, 0);       \
            __builtin_amdgcn_global_load_lds(psb + (int64_t)l_kt * g.sb.stride_kb,                \
                                             st_ + A_BYTES + B_BYTES + BM * 4 + (wave & 1) * 256, 4, 0, 0); \
        }                                                                                          \
        issued++;                                                                                  \
        ops += L;                                                                                  \
        if (npend == 0) pend0 = ops;                                                               \
        else if (npend == 1) pend1 = ops;                                                          \
        else pend2 = ops;                                                                          \
        npend++;                                                                                   \
        if (++l_kt >= l_it.ke) {                                                                   \
            l_ok = item_of(g, ++l_round, l_it);                                                    \
            if (l_ok) {                                                                            \
                l_kt = l_it.kb;                                                                    \
                FP8K_SET_LOAD_PTRS();                                                              \
            }                                                                                      \
        }                                                                                          \
    } while (0)
    // prologue: S-1 stages in flight
#pragma unroll
    for (int s = 0; s < S - 1; s++)
        if (l_ok) FP8K_ISSUE_STAGE();

    // ---- compute cursor ----------------------------------------------------
    int c_round = 0;
    Item c_it;
    if (!item_of(g, 0, c_it)) return;
    int c_kt = c_it.kb;
    int consumed = 0;

    v16f acc[4][WNJ];
#pragma unroll
    for (int mi = 0; mi < 4; mi++)
#pragma unroll
        for (int nj = 0; nj < WNJ; nj++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[mi][nj][v] = 0.0f;

    const int frow = lane & 31;                    // fragment row within a 32-row block
    const int arow = wi * 128 + frow;
    const int brow = wj * (WNJ * 32) + frow;
    const bool sb_per_row = g.sb.group == 1;
    const int ch = (lane >> 5) * 2;
    const uint32_t smem0 = lds_off(smem);
    // fragment rows in a stage: chunk ch (ch+1 at ^16; the second 64-long half
    // at ^64), +4096 bytes per 32-row block
    const uint32_t offA = (uint32_t)(arow * BK + ((ch ^ swz<BK>(arow)) << 4));
    const uint32_t offB = (uint32_t)(A_BYTES + brow * BK + ((ch ^ swz<BK>(brow)) << 4));

#define FP8K_STEP(FIRST)                                                                   \
    do {                                                                                   \
 /* vmcnt completes in order: waiting until at most n ops are outstanding, \
   n = ops issued after this stage (capped at 63, rounded down to a multiple \
   of 4), guarantees the stage landed while later stages and epilogue stores \
   stay in flight. */ \
        { \
            const int n_after = ops - pend0; \
            pend0 = pend1; \
            pend1 = pend2; \
            npend--; \
            if (n_after >= 63) wait_vm<63>(); \
            else if (n_after >= 56) wait_vm<56>(); \
            else if (n_after >= 48) wait_vm<48>(); \
            else if (n_after >= 40) wait_vm<40>(); \
            else if (n_after >= 32) wait_vm<32>(); \
            else if (n_after >= 28) wait_vm<28>(); \
            else if (n_after >= 24) wait_vm<24>(); \
            else if (n_after >= 20) wait_vm<20>(); \
            else if (n_after >= 16) wait_vm<16>(); \
            else if (n_after >= 14) wait_vm<14>(); \
            else if (n_after >= 12) wait_vm<12>(); \
            else if (n_after >= 8) wait_vm<8>(); \
            else if (n_after >= 4) wait_vm<4>(); \
            else wait_vm<0>(); \
        } \
        barrier_lds(); \
        if (l_ok) FP8K_ISSUE_STAGE(); \
 \
        /* LDS reads in inline assembly (no compiler vmcnt(0) in front of
           them), each group issued and waited for inside one asm statement:
           the stage's fp32 factors, then the fragments of each 64-long half
           of the 128-block */ \
        const uint32_t sb_ = smem0 + (uint32_t)((consumed % S) * STAGE); \
        float sa_v[4]; \
        float sb_v[WNJ][16]; \
        float sb_u = 0.0f; \
        { \
            const uint32_t sc_ = sb_ + A_BYTES + B_BYTES; \
            const uint32_t pa_ = sc_ + (uint32_t)(arow * 4); \
            if (sb_per_row) { \
                const uint32_t pb_ = sc_ + (uint32_t)(BM * 4 + (wj * (WNJ * 32) + 4 * (lane >> 5)) * 4); \
                f32x4 g0_, g1_, g2_, g3_, g4_, g5_, g6_, g7_; \
                asm volatile("ds_read_b32 %0, %12 offset:0\n\t" \
                             "ds_read_b32 %1, %12 offset:128\n\t" \
                             "ds_read_b32 %2, %12 offset:256\n\t" \
                             "ds_read_b32 %3, %12 offset:384\n\t" \
                             "ds_read_b128 %4, %13 offset:0\n\t" \
                             "ds_read_b128 %5, %13 offset:32\n\t" \
                             "ds_read_b128 %6, %13 offset:64\n\t" \
                             "ds_read_b128 %7, %13 offset:96\n\t" \
                             "ds_read_b128 %8, %13 offset:128\n\t" \
                             "ds_read_b128 %9, %13 offset:160\n\t" \
                             "ds_read_b128 %10, %13 offset:192\n\t" \
                             "ds_read_b128 %11, %13 offset:224\n\t" \
                             "s_waitcnt lgkmcnt(0)" \
                             : "=&v"(sa_v[0]), "=&v"(sa_v[1]), "=&v"(sa_v[2]), "=&v"(sa_v[3]), \
                               "=&v"(g0_), "=&v"(g1_), "=&v"(g2_), "=&v"(g3_), \
                               "=&v"(g4_), "=&v"(g5_), "=&v"(g6_), "=&v"(g7_) \
                             : "v"(pa_), "v"(pb_) \
                             : "memory"); \
                /* element e of float4 q of column block nj: column 8q + e (+4 for lanes 32..63) */ \
                const f32x4 gq_[WNJ][4] = {{g0_, g1_, g2_, g3_}, {g4_, g5_, g6_, g7_}}; \
_Pragma("unroll") \
                for (int nj = 0; nj < WNJ; nj++) \
_Pragma("unroll") \
                    for (int q = 0; q < 4; q++) { \
                        sb_v[nj][4 * q + 0] = gq_[nj][q].x; \
                        sb_v[nj][4 * q + 1] = gq_[nj][q].y; \
                        sb_v[nj][4 * q + 2] = gq_[nj][q].z; \
                        sb_v[nj][4 * q + 3] = gq_[nj][q].w; \
                    } \
            } else { \
                const uint32_t pb_ = sc_ + (uint32_t)(BM * 4 + wj * (WNJ * 32) * 4); \
                asm volatile("ds_read_b32 %0, %5 offset:0\n\t" \
                             "ds_read_b32 %1, %5 offset:128\n\t" \
                             "ds_read_b32 %2, %5 offset:256\n\t" \
                             "ds_read_b32 %3, %5 offset:384\n\t" \
                             "ds_read_b32 %4, %6\n\t" \
                             "s_waitcnt lgkmcnt(0)" \
                             : "=&v"(sa_v[0]), "=&v"(sa_v[1]), "=&v"(sa_v[2]), "=&v"(sa_v[3]), "=&v"(sb_u) \
                             : "v"(pa_), "v"(pb_) \
                             : "memory"); \
            } \
        } \
        const uint32_t a0_ = sb_ + offA, a1_ = a0_ ^ 16u, b0_ = sb_ + offB, b1_ = b0_ ^ 16u; \
        v16f p[4][WNJ]; \
        { \
            v8i af[4], bf[WNJ]; \
            ds_frags6_wait(af, bf, a0_, a1_, b0_, b1_); \
            const v16f zero = {}; \
_Pragma("unroll") \
            for (int mi = 0; mi < 4; mi++) \
_Pragma("unroll") \
                for (int nj = 0; nj < WNJ; nj++) p[mi][nj] = mfma<FA, FB>(bf[nj], af[mi], zero); \
        } \
        { \
            /* second half of the block: chunks 4..7 of the same rows */ \
            v8i af[4], bf[WNJ]; \
            ds_frags6_wait(af, bf, a0_ ^ 64u, a1_ ^ 64u, b0_ ^ 64u, b1_ ^ 64u); \
_Pragma("unroll") \
            for (int mi = 0; mi < 4; mi++) \
_Pragma("unroll") \
                for (int nj = 0; nj < WNJ; nj++) p[mi][nj] = mfma<FA, FB>(bf[nj], af[mi], p[mi][nj]); \
        } \
_Pragma("unroll") \
        for (int mi = 0; mi < 4; mi++) \
_Pragma("unroll") \
            for (int nj = 0; nj < WNJ; nj++) { \
                if (sb_per_row) { \
_Pragma("unroll") \
                    for (int v = 0; v < 16; v++) \
                        acc[mi][nj][v] = FIRST ? p[mi][nj][v] * (sa_v[mi] * sb_v[nj][v]) : __builtin_fmaf(p[mi][nj][v], sa_v[mi] * sb_v[nj][v], acc[mi][nj][v]); \
                } else { \
                    const float t = sa_v[mi] * sb_u; \
_Pragma("unroll") \
                    for (int v = 0; v < 16; v++) acc[mi][nj][v] = FIRST ? p[mi][nj][v] * t : __builtin_fmaf(p[mi][nj][v], t, acc[mi][nj][v]); \
                } \
            } \
        consumed++;                                                                        \
    } while (0)

    while (true) {
        FP8K_STEP(true);
        for (int kt = c_it.kb + 1; kt < c_it.ke; kt++) {
            c_kt = kt;
            FP8K_STEP(false);
        }
        // ---- epilogue of the finished item ---------------------------------
        {
            const int64_t i0 = (int64_t)c_it.ti * BM, j0 = (int64_t)c_it.tj * BN;
            const int64_t my_i = i0 + arow;
            const int64_t jw = j0 + wj * (WNJ * 32);                  // first column of this wave
            const int64_t my_j = jw + 4 * (lane >> 5);
            // validity is uniform per 32x32 block (I, J are multiples of 128)
            const bool i_ok0 = i0 + wi * 128 < g.I;                   // mi blocks share it
            const int nj_ok = jw >= g.J ? 0 : WNJ;                    // wave's columns all valid or none
            // the wave issues all of the stores below or none of them
            if (i_ok0 && nj_ok) ops += 4 * WNJ * 4;
            if (g.splits > 1) {
                float* out = g.part + (int64_t)c_it.z * g.I * g.J + my_i * g.J + my_j;
                if (i_ok0 && nj_ok) {
#pragma unroll
                    for (int mi = 0; mi < 4; mi++)
#pragma unroll
                        for (int nj = 0; nj < WNJ; nj++)
#pragma unroll
                            for (int q = 0; q < 4; q++)
                                *reinterpret_cast<float4*>(out + (int64_t)mi * 32 * g.J + nj * 32 + 8 * q) =
                                    make_float4(acc[mi][nj][4 * q], acc[mi][nj][4 * q + 1], acc[mi][nj][4 * q + 2],
                                                acc[mi][nj][4 * q + 3]);
                }
            } else {
                // block-scaled: the factors are already in the accumulators
                uint16_t* out = g.c + my_i * g.J + my_j;
                if (i_ok0 && nj_ok) {
#pragma unroll
                    for (int mi = 0; mi < 4; mi++)
#pragma unroll
                        for (int nj = 0; nj < WNJ; nj++)
#pragma unroll
                            for (int q = 0; q < 4; q++) {
                                const __bf16 h0 = (__bf16)acc[mi][nj][4 * q];
                                const __bf16 h1 = (__bf16)acc[mi][nj][4 * q + 1];
                                const __bf16 h2 = (__bf16)acc[mi][nj][4 * q + 2];
                                const __bf16 h3 = (__bf16)acc[mi][nj][4 * q + 3];
                                uint2 w;
                                w.x = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                                      ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
                                w.y = (uint32_t)__builtin_bit_cast(uint16_t, h2) |
                                      ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
                                *reinterpret_cast<uint2*>(out + (int64_t)mi * 32 * g.J + nj * 32 + 8 * q) = w;
                            }
                }
            }
        }
        if (!item_of(g, ++c_round, c_it)) break;
        c_kt = c_it.kb;
    }
#undef FP8K_SET_LOAD_PTRS
#undef FP8K_ISSUE_STAGE
#undef FP8K_ROWOFF
#undef FP8K_STEP
}

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

int gemm_splits(int64_t I, int64_t J, int64_t K, bool block) {
    if (!block) return gemm_tensor_splits(I, J, K);
    const int64_t tiles = ((I + CfgBlock::BM - 1) / CfgBlock::BM) * ((J + CfgBlock::BN - 1) / CfgBlock::BN);
    const int64_t k128 = K / 128;
    // aim for one work item per resident workgroup (256 CUs x occupancy),
    // keep >= 8 blocks of 128 per split
    const int64_t slots = 256 * CfgBlock::OCC;
    int64_t s = 1;
    while (tiles * s < slots && k128 / (s * 2) >= 8 && s < 64) s *= 2;
    return (int)s;
}

size_t gemm_ws_bytes(int64_t I, int64_t J, int64_t K) {
    const int a = gemm_splits(I, J, K, false), b = gemm_splits(I, J, K, true);
    const int s = a > b ? a : b;
    return s > 1 ? (size_t)s * (size_t)I * (size_t)J * sizeof(float) : 0;
}

hipError_t launch_gemm(const GemmLaunch& l, hipStream_t stream) {
    const bool block = l.sa.group != 0;
    const int splits = gemm_splits(l.I, l.J, l.K, block);
    if (!block) {
        hipError_t e = launch_gemm_tensor(l, splits, stream);
        if (e != hipSuccess || splits == 1) return e;
    } else {
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
        g.splits = splits;
        g.tiles_i = (int)((l.I + CfgBlock::BM - 1) / CfgBlock::BM);
        g.tiles_j = (int)((l.J + CfgBlock::BN - 1) / CfgBlock::BN);
        g.ktiles = (int)(l.K / CfgBlock::BK);
        g.items = g.tiles_i * g.tiles_j * g.splits;
        int grid = cu_count() * CfgBlock::OCC;
        if (grid > g.items) grid = g.items;
#define FP8K_GEMM(FA, FB) \
    hipLaunchKernelGGL((gemm_kernel<FA, FB, true, CfgBlock>), dim3(grid), dim3(kThreads), 0, stream, g)
        if (l.fa == 0 && l.fb == 0) FP8K_GEMM(0, 0);
        else if (l.fa == 1 && l.fb == 0) FP8K_GEMM(1, 0);
        else if (l.fa == 0 && l.fb == 1) FP8K_GEMM(0, 1);
        else FP8K_GEMM(1, 1);
#undef FP8K_GEMM
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || splits == 1) return e;
    }
    const int64_t n4 = l.I * l.J / 4;
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const float*>(l.ws), splits, n4, l.I * l.J, l.sa.sinv, l.sb.sinv, block ? 0 : 1,
                       static_cast<uint16_t*>(l.c));
    return hipGetLastError();
}

}  // namespace fp8k
