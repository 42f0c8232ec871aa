// Tensorwise-scaled FP8 GEMM C[i][j] = t * sum_k A[i][k] B[j][k] on the gfx950
// matrix cores (t = product of the two operands' inverse scales, applied once
// in the epilogue; BF16 output, or fp32 partial sums for split-K).
//
// Method ("Native FP8 MLP reconstruction", implementation paragraph): the
// three GEMMs of the FP8 linear (E4M3 x E4M3 forward, E5M2 x E4M3 for both
// gradients) accumulate at full fp32 precision across the contraction and
// write BF16.  Every operand is contraction-contiguous ("NT").
//
// Design
//  - persistent: one workgroup per CU walks work items (256 x 256 output
//    tile, split-K slice) dealt XCD by XCD (the dispatcher puts workgroup b on
//    XCD b % 8) and rastered in groups of tile rows (8 for wide outputs, 2
//    for narrow ones), so the workgroups of one XCD share A and B tiles
//    through its L2.
//  - 8 waves, two per SIMD, wave tile 128 x 64 (4 x 2 blocks of
//    v_mfma_f32_32x32x64_f8f6f4, 128 accumulator registers), all waves in
//    lock step with one s_barrier per 128-long contraction stage.
//  - operands stream HBM -> LDS with buffer_load ... lds (LDS-DMA, no VGPR
//    staging): 2 stages of 64 KiB (A and B, 256 rows x 128 bytes each); each
//    DMA instruction fills 8 whole 128-byte rows, so every cache line it
//    touches is read in full (with 64-byte rows each instruction touched
//    twice the lines and the L1 stalled the address unit: 8192 x 8192 x 16384
//    830 -> 753 us).  Each wave moves 8 KiB per stage through a buffer
//    resource based at the tile (rows past I or J lie outside the resource
//    and read as zero).  LDS rows are XOR-swizzled.
//  - a stage is two 64-long half steps of 8 MFMAs; the fragments of the next
//    half step are read between the MFMAs (A fragment mi is reloaded right
//    after its last MFMA; the two B fragments alternate between two register
//    sets).  The first half reads the second half of the same rows; the
//    second half starts with the hand-off of the next stage and reads its
//    first half, and after the barrier the wave issues the DMA of the stage
//    after that into the buffer just consumed, in four chunks of one A and
//    one B block, one before each MFMA group of that half step (all eight at
//    once after the barrier: 8192^3 423 -> 398-404 us with the spread).
//  - the hand-off of a stage is one s_waitcnt vmcnt(n) on the wave's own DMA
//    (n counted exactly: the epilogue stores issued after it) plus the
//    barrier; fragment reads are inline assembly so the compiler adds no
//    vmcnt(0) in front of them.  Their destination registers stay live
//    operands of an lgkmcnt(0) wait (the next half step's, or the wait before
//    the final epilogue), so no register with a load in flight is reused.
//  - epilogue: each wave converts 32 rows at a time to bf16 into a private
//    4 KiB LDS slice (chunk-major, (row ^ 2 chunk) swizzle: conflict-free
//    writes and reads) and stores whole 128-byte row segments.
#include <type_traits>

#include "device.hpp"
#include "gelu_keys.hpp"
#include "gemm_common.hpp"
#include "internal.hpp"

namespace fp8k {
namespace tensor {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int S = 2;                      // LDS stages (power of two)
constexpr int D = S;                      // stages issued in the prologue
constexpr int NW = 8;                     // waves
constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK, STAGE = A_BYTES + B_BYTES;
constexpr int LA = A_BYTES / 1024 / NW;   // LDS-DMA instructions per wave per stage (A)
constexpr int LB = B_BYTES / 1024 / NW;   // (B)
constexpr int L = LA + LB;
constexpr int RPK = 1024 / BK;            // rows per 1 KiB DMA block (whole 128-byte lines)
constexpr int CPR = BK / 16;              // 16-byte chunks per LDS row
constexpr int ECH = 8;                    // 16-byte chunks per epilogue row (64 bf16)
constexpr int SLICE = 32 * ECH * 16;      // per-wave epilogue slice
static_assert(S * STAGE + NW * SLICE <= 160 * 1024, "LDS");
static_assert((S & (S - 1)) == 0, "S");
static_assert(LA % 2 == 0 && LB % 2 == 0, "odd DMA blocks alternate the swizzle");

struct Args {
    const uint8_t* a;
    const uint8_t* b;
    const float* sa;      // tensorwise inverse scales
    const float* sb;
    int64_t I, J, K;
    uint16_t* c;
    float* part;          // split-K partials [splits][I][J]
    int splits, tiles_i, tiles_j, kpairs, items;   // kpairs: contraction blocks of 128
    int gi;               // tile rows per raster group
    uint16_t* amax_part;  // optional: one partial max |bf16 C| per workgroup, zeros after
    uint16_t* gelu_keys;  // KEYS: the four GELU amax key arrays (gelu_keys.hpp), one slot
                          // per workgroup, zeros after
};

struct Item {
    int ti, tj, z, kb, ke;   // kb, ke: contraction stages of BK = 128
};

__device__ __forceinline__ bool item_at(const Args& g, int r, Item& it) {
    const int G = gridDim.x, b = blockIdx.x;
    const int Lg = r * G + ((G & 7) == 0 ? (b & 7) * (G >> 3) + (b >> 3) : b);
    if (Lg >= g.items) return false;
    const int tiles = g.tiles_i * g.tiles_j;
    const int z = Lg / tiles, t = Lg - z * tiles;
    // raster groups of g.gi tile rows: the workgroups of an XCD share B tiles
    // across the group and A tiles along it
    const int GI = g.gi;
    const int per_group = GI * g.tiles_j, grp = t / per_group, local = t - grp * per_group;
    int rows = g.tiles_i - grp * GI;
    rows = rows < GI ? rows : GI;
    it.ti = grp * GI + local % rows;
    it.tj = local / rows;
    it.z = z;
    // kpairs < 2^16 and splits <= 64 (contraction below 2^23): 32-bit math
    it.kb = g.kpairs * z / g.splits;
    it.ke = g.kpairs * (z + 1) / g.splits;
    return true;
}

// s_waitcnt vmcnt(n) for a runtime n (rounded down to a supported value)
__device__ __forceinline__ void wait_vm_n(int n) {
    if (n == L) wait_vm<L>();
    else if (n >= 63) wait_vm<63>();
    else if (n >= 48) wait_vm<48>();
    else if (n >= 32) wait_vm<32>();
    else if (n >= 24) wait_vm<24>();
    else if (n >= 16) wait_vm<16>();
    else if (n >= 8) wait_vm<8>();
    else if (n >= 4) wait_vm<4>();
    else wait_vm<0>();
}

template <int FA, int FB, bool NT, bool KEYS = false>
__global__ __launch_bounds__(NW * 64, 1) void gemm_tensor_kernel(Args g) {
    // separate objects: the epilogue's LDS traffic never aliases the stages
    __shared__ __attribute__((aligned(1024))) uint8_t smem[S * STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t sepi[NW * SLICE];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int wi = wave & 1, wj = wave >> 1;
    const uint32_t K = (uint32_t)g.K;
    const uint32_t KR = K * RPK;   // bytes of one DMA block's rows

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
    const uint32_t wrow_off = (uint32_t)(wave * LA * RPK) * K;   // this wave's first row of the tile
    uint32_t l_so = 0;   // buffer offset of the next stage to load
    int l_left = 0;      // stages left in the load item
    auto set_load_item = [&]() __attribute__((always_inline)) {
        const int64_t i0 = (int64_t)l_it.ti * BM, j0 = (int64_t)l_it.tj * BN;
        ra = make_rsrc(g.a + i0 * g.K, (g.I - i0 < BM ? g.I - i0 : BM) * g.K);
        rb = make_rsrc(g.b + j0 * g.K, (g.J - j0 < BN ? g.J - j0 : BN) * g.K);
        l_so = wrow_off + (uint32_t)l_it.kb * BK;
        l_left = l_it.ke - l_it.kb;
    };
    if (l_ok) set_load_item();
    const uint32_t smem0 = lds_off(smem);
    uint32_t dma_off = 0;   // stage buffer the next DMA fills
    // DMA of one stage in four chunks (A block c and B block c), so they can be
    // spread between matrix instructions; advance_stage() moves the load
    // cursor once all four are issued
    auto dma_chunk = [&](int c) __attribute__((always_inline)) {
        const uint32_t dA = smem0 + dma_off + (uint32_t)(wave * LA * 1024);
        const uint32_t dB = smem0 + dma_off + (uint32_t)(A_BYTES + wave * LB * 1024);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)(uintptr_t)(dA + c * 1024),
                                                 16, (c & 1) ? loff1 : loff0,
                                                 __builtin_amdgcn_readfirstlane(l_so + (uint32_t)c * KR), 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (__attribute__((address_space(3))) void*)(uintptr_t)(dB + c * 1024),
                                                 16, (c & 1) ? loff1 : loff0,
                                                 __builtin_amdgcn_readfirstlane(l_so + (uint32_t)c * KR), 0, 0);
    };
    auto advance_stage = [&]() __attribute__((always_inline)) {
        dma_off = (dma_off + STAGE) & (S * STAGE - 1);
        l_so += BK;
        if (--l_left == 0) {
            if (l_ok && item_at(g, l_round + 1, l_it)) {
                l_round++;
                set_load_item();
            } else {
                // past the last item: keep re-reading its last stage into
                // buffers nobody reads, so every step issues the same loads
                l_ok = false;
                l_so -= BK;
                l_left = 1;
            }
        }
    };
    auto issue_stage = [&]() __attribute__((always_inline)) {
        dma_chunk(0);
        dma_chunk(1);
        dma_chunk(2);
        dma_chunk(3);
        advance_stage();
    };

    // ---- prologue: both stages in flight, stage 0 landed, the fragments of
    // its first half read ------------------------------------------------------
#pragma unroll
    for (int s = 0; s < D; s++) issue_stage();
    wait_vm<(D - 1) * L>();
    barrier_lds();

    int c_round = 0;
    Item c_it;
    bool c_ok = item_at(g, 0, c_it);
    int st_cur = 0;   // epilogue stores issued since the last stage wait

    const int frow = lane & 31;
    const int arow = wi * 128 + frow, brow = wj * 64 + frow;
    const int ch = (lane >> 5) * 2;
    const float t_tensor = g.sa[0] * g.sb[0];
    // fragment rows in a stage: chunk ch (ch+1 at ^16; the second 64-long
    // half of the 128-byte row at ^64), +4096 per 32 rows
    const uint32_t offA = (uint32_t)(arow * BK + ((ch ^ swz<BK>(arow)) << 4));
    const uint32_t offB = (uint32_t)(A_BYTES + brow * BK + ((ch ^ swz<BK>(brow)) << 4));

    v16f acc[4][2];
    v8i fa[4], fb0[2], fb1[2];
#pragma unroll
    for (int mi = 0; mi < 4; mi++)
#pragma unroll
        for (int nj = 0; nj < 2; nj++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[mi][nj][v] = 0.0f;
    {
        const uint32_t a0 = smem0 + offA, a1 = a0 ^ 16u, b0 = smem0 + offB, b1 = b0 ^ 16u;
        fa[0] = ds_frag<0>(a0, a1);
        fa[1] = ds_frag<4096>(a0, a1);
        fa[2] = ds_frag<8192>(a0, a1);
        fa[3] = ds_frag<12288>(a0, a1);
        fb0[0] = ds_frag<0>(b0, b1);
        fb0[1] = ds_frag<4096>(b0, b1);
    }
    uint32_t cur_off = 0;   // stage buffer being consumed

    // epilogue slice: (row r, chunk c) at c*512 + ((r ^ 2c) << 4)
    const uint32_t slice = lds_off(sepi) + (uint32_t)(wave * SLICE);
    const uint32_t wbase = slice + (uint32_t)((lane >> 5) * 8);
    const uint32_t rc = (uint32_t)(lane & 7), rr = (uint32_t)(lane >> 3);
    const uint32_t goff = (uint32_t)(rr * (uint32_t)g.J * 2 + rc * 16);

    // max |bf16| of the outputs this lane wrote (two packed 16-bit
    // magnitudes; NaN magnitudes exceed +Inf's, so NaN propagates)
    uint32_t amx = 0;
    GeluKeys gk;   // KEYS: what the quantize of GELU(C) needs instead of an amax pass

    // write one item's accumulators; returns the vector-memory stores issued.
    // AMAX (a std::bool_constant): fold max |bf16| into amx -- only when the
    // caller asked for the partials, since it is 4 of the 10 VALU operations
    // per 4 outputs (131072 x 2048 x 512: a third of the epilogue's VALU).
    const bool want_amax = g.amax_part != nullptr;
    auto epilogue = [&](const Item& it, auto amax_on) __attribute__((always_inline)) -> int {
        constexpr bool AMAX = decltype(amax_on)::value;
        const int64_t i0 = (int64_t)it.ti * BM, j0 = (int64_t)it.tj * BN;
        const int64_t jw = j0 + wj * 64;
        // validity is uniform per wave (I and J are multiples of 128)
        if (!((i0 + wi * 128 < g.I) && (jw < g.J))) return 0;
        if (g.splits > 1) {
            float* out = g.part + (int64_t)it.z * g.I * g.J + (i0 + arow) * g.J + jw + 4 * (lane >> 5);
#pragma unroll
            for (int mi = 0; mi < 4; mi++)
#pragma unroll
                for (int nj = 0; nj < 2; nj++)
#pragma unroll
                    for (int q = 0; q < 4; q++)
                        *reinterpret_cast<float4*>(out + (int64_t)mi * 32 * g.J + nj * 32 + 8 * q) =
                            make_float4(acc[mi][nj][4 * q], acc[mi][nj][4 * q + 1], acc[mi][nj][4 * q + 2],
                                        acc[mi][nj][4 * q + 3]);
            return 4 * 2 * 4;
        }
        uint8_t* out_base = reinterpret_cast<uint8_t*>(g.c + (i0 + wi * 128) * g.J + jw);
#pragma unroll
        for (int mi = 0; mi < 4; mi++) {
#pragma unroll
            for (int nj = 0; nj < 2; nj++)
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    uint2 w;
                    w.x = pack_bf16x2(acc[mi][nj][4 * q] * t_tensor, acc[mi][nj][4 * q + 1] * t_tensor);
                    w.y = pack_bf16x2(acc[mi][nj][4 * q + 2] * t_tensor, acc[mi][nj][4 * q + 3] * t_tensor);
                    if constexpr (AMAX) amx = pkmax_u16(amx, pkmax_u16(mag2(w.x), mag2(w.y)));
                    if constexpr (KEYS) {
                        gk.add(w.x);
                        gk.add(w.y);
                    }
                    const int chunk = nj * 4 + q;
                    const uint32_t wa = wbase + (uint32_t)(chunk * 512 + ((frow ^ (2 * chunk)) << 4));
                    asm volatile("ds_write_b64 %0, %1" : : "v"(wa), "v"(w) : "memory");
                }
            // a wave's LDS operations execute in order: the read-back sees the
            // writes above, and the next block's writes follow these reads
            u32x4 r0, r1, r2, r3;
            const uint32_t ra0 = slice + rc * 512 + ((rr ^ (2 * rc)) << 4);
            const uint32_t ra1 = slice + rc * 512 + (((rr + 8) ^ (2 * rc)) << 4);
            const uint32_t ra2 = slice + rc * 512 + (((rr + 16) ^ (2 * rc)) << 4);
            const uint32_t ra3 = slice + rc * 512 + (((rr + 24) ^ (2 * rc)) << 4);
            asm volatile("ds_read_b128 %0, %1" : "=v"(r0) : "v"(ra0) : "memory");
            asm volatile("ds_read_b128 %0, %1" : "=v"(r1) : "v"(ra1) : "memory");
            asm volatile("ds_read_b128 %0, %1" : "=v"(r2) : "v"(ra2) : "memory");
            asm volatile("ds_read_b128 %0, %1" : "=v"(r3) : "v"(ra3) : "memory");
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r0), "+v"(r1), "+v"(r2), "+v"(r3));
            uint8_t* ob = out_base + (int64_t)mi * 32 * g.J * 2;
            st_out16<NT>(ob + goff, r0);
            st_out16<NT>(ob + (int64_t)8 * g.J * 2 + goff, r1);
            st_out16<NT>(ob + (int64_t)16 * g.J * 2 + goff, r2);
            st_out16<NT>(ob + (int64_t)24 * g.J * 2 + goff, r3);
        }
        return 4 * 4;
    };

    // A stage is two 64-long half steps of 8 MFMAs each; the fragments of
    // the next half step are read while the current one's MFMAs run (A
    // fragment mi is reloaded right after its last MFMA; the B fragments
    // alternate between two register sets).  First half: its fragments come
    // from the stage being consumed (second half of the rows, ^64).  Second
    // half: the next stage must have landed everywhere -- wait for this
    // wave's DMA of it (issued one stage earlier; only epilogue stores can
    // follow it) and the barrier, which also retires every wave's reads of
    // the consumed stage, whose buffer the DMA two stages ahead then fills.
#define FP8K_MF(MI, FBC, FIRST)                                                                    \
    do {                                                                                           \
        acc[MI][0] = mfma<FA, FB>(FBC[0], fa[MI], (FIRST) ? vzero : acc[MI][0]);                  \
        acc[MI][1] = mfma<FA, FB>(FBC[1], fa[MI], (FIRST) ? vzero : acc[MI][1]);                  \
    } while (0)
#define FP8K_HALF(FBC, FBN, FIRST, A0, B0, DMA)                                                    \
    do {                                                                                           \
        const uint32_t a0_ = (A0), a1_ = a0_ ^ 16u, b0_ = (B0), b1_ = b0_ ^ 16u;                   \
        if (DMA) dma_chunk(0);                                                                     \
        FP8K_MF(0, FBC, FIRST);                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                         \
        fa[0] = ds_frag<0>(a0_, a1_);                                                              \
        FBN[0] = ds_frag<0>(b0_, b1_);                                                             \
        if (DMA) dma_chunk(1);                                                                     \
        __builtin_amdgcn_sched_barrier(0);                                                         \
        FP8K_MF(1, FBC, FIRST);                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                         \
        fa[1] = ds_frag<4096>(a0_, a1_);                                                           \
        FBN[1] = ds_frag<4096>(b0_, b1_);                                                          \
        if (DMA) dma_chunk(2);                                                                     \
        __builtin_amdgcn_sched_barrier(0);                                                         \
        FP8K_MF(2, FBC, FIRST);                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                         \
        fa[2] = ds_frag<8192>(a0_, a1_);                                                           \
        if (DMA) dma_chunk(3);                                                                     \
        __builtin_amdgcn_sched_barrier(0);                                                         \
        FP8K_MF(3, FBC, FIRST);                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                         \
        fa[3] = ds_frag<12288>(a0_, a1_);                                                          \
        __builtin_amdgcn_sched_barrier(0);                                                         \
    } while (0)
#define FP8K_STAGE(FIRST)                                                                          \
    do {                                                                                           \
        asm volatile("s_waitcnt lgkmcnt(0)"                                                        \
                     : "+v"(fa[0]), "+v"(fa[1]), "+v"(fa[2]), "+v"(fa[3]), "+v"(fb0[0]), "+v"(fb0[1]) \
                     :                                                                             \
                     : "memory");                                                                  \
        FP8K_HALF(fb0, fb1, FIRST, (smem0 + cur_off + offA) ^ 64u, (smem0 + cur_off + offB) ^ 64u, false); \
        wait_vm_n(st_cur);                                                                         \
        st_cur = 0;                                                                                \
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier"                                           \
                     : "+v"(fa[0]), "+v"(fa[1]), "+v"(fa[2]), "+v"(fa[3]), "+v"(fb1[0]), "+v"(fb1[1]) \
                     :                                                                             \
                     : "memory");                                                                  \
        cur_off ^= (uint32_t)STAGE;                                                                \
        FP8K_HALF(fb1, fb0, false, smem0 + cur_off + offA, smem0 + cur_off + offB, true);          \
        advance_stage();                                                                           \
    } while (0)

    const v16f vzero = {};
    bool have_prev = false;
    Item p_it;
    while (c_ok) {
        Item n_it;
        const bool more = item_at(g, c_round + 1, n_it);
        const int nstages = c_it.ke - c_it.kb;   // >= 1
        if (have_prev)
            st_cur += want_amax ? epilogue(p_it, std::true_type{}) : epilogue(p_it, std::false_type{});
        FP8K_STAGE(true);
        // after the last item the fragments the last half step reads are
        // unused (their stage is a re-read of the last one); reading anyway
        // keeps a single definition of every fragment register
        for (int s = 1; s < nstages; s++) FP8K_STAGE(false);
        p_it = c_it;
        have_prev = true;
        c_it = n_it;
        c_ok = more;
        c_round++;
    }
#undef FP8K_STAGE
#undef FP8K_HALF
#undef FP8K_MF
    // The last step's fragment reads (of a re-read stage) are dead but still
    // in flight: let them land before the epilogue's temporaries can reuse
    // their registers.
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(fa[0]), "+v"(fa[1]), "+v"(fa[2]), "+v"(fa[3]), "+v"(fb0[0]), "+v"(fb0[1]), "+v"(fb1[0]),
                   "+v"(fb1[1])
                 :
                 : "memory");
    if (have_prev) {
        if (want_amax) epilogue(p_it, std::true_type{});
        else epilogue(p_it, std::false_type{});
    }
    wait_vm<0>();
    if (g.amax_part) {
        // workgroup max through the (now idle) epilogue slices, one partial
        // per workgroup; workgroup 0 zeroes the slots no workgroup owns
        const uint32_t m = wave_max_u32(hmax_u16(amx));
        uint32_t* red = reinterpret_cast<uint32_t*>(sepi);
        __syncthreads();
        if (lane == 0) red[wave] = m;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t r = red[0];
#pragma unroll
            for (int w = 1; w < NW; w++) r = r > red[w] ? r : red[w];
            g.amax_part[blockIdx.x] = (uint16_t)r;
        }
        if (blockIdx.x == 0)
            for (int p = (int)gridDim.x + (int)threadIdx.x; p < kMaxAmaxPartials; p += NW * 64) g.amax_part[p] = 0;
    }
    if constexpr (KEYS) {
        // the same reduction for the four GELU keys (all max-reducible)
        uint32_t k[kGeluKeyArrays];
        gk.fold(k);
#pragma unroll
        for (int q = 0; q < kGeluKeyArrays; q++) k[q] = wave_max_u32(k[q]);
        uint32_t* red = reinterpret_cast<uint32_t*>(sepi) + NW;
        __syncthreads();
        if (lane == 0)
#pragma unroll
            for (int q = 0; q < kGeluKeyArrays; q++) red[q * NW + wave] = k[q];
        __syncthreads();
        if (threadIdx.x < kGeluKeyArrays) {
            const int q = (int)threadIdx.x;
            uint32_t r = red[q * NW];
#pragma unroll
            for (int w = 1; w < NW; w++) r = r > red[q * NW + w] ? r : red[q * NW + w];
            g.gelu_keys[q * kMaxAmaxPartials + blockIdx.x] = (uint16_t)r;
        }
        if (blockIdx.x == 0)
            for (int p = (int)gridDim.x + (int)threadIdx.x; p < kMaxAmaxPartials; p += NW * 64)
#pragma unroll
                for (int q = 0; q < kGeluKeyArrays; q++) g.gelu_keys[q * kMaxAmaxPartials + p] = 0;
    }
}

}  // namespace tensor

using namespace tensor;

int gemm_tensor_splits(int64_t I, int64_t J, int64_t K) {
    const int64_t tiles = ((I + BM - 1) / BM) * ((J + BN - 1) / BN);
    const int64_t kp = K / 128;
    // aim for one work item per CU, keep >= 8 blocks of 128 per slice
    int64_t s = 1;
    while (tiles * s < 256 && kp / (s * 2) >= 8 && s < 64) s *= 2;
    return (int)s;
}

hipError_t launch_gemm_tensor(const GemmLaunch& l, int splits, hipStream_t stream) {
    Args g;
    g.a = static_cast<const uint8_t*>(l.a);
    g.b = static_cast<const uint8_t*>(l.b);
    g.sa = l.sa.sinv;
    g.sb = l.sb.sinv;
    g.I = l.I;
    g.J = l.J;
    g.K = l.K;
    g.c = static_cast<uint16_t*>(l.c);
    g.part = static_cast<float*>(l.ws);
    g.splits = splits;
    g.tiles_i = (int)((l.I + BM - 1) / BM);
    g.tiles_j = (int)((l.J + BN - 1) / BN);
    g.kpairs = (int)(l.K / 128);
    g.items = g.tiles_i * g.tiles_j * splits;
    // the split-K reduce emits the amax of a split output
    g.amax_part = splits == 1 ? l.c_amax : nullptr;
    g.gelu_keys = splits == 1 ? l.gelu_keys : nullptr;
    // an XCD's 32 concurrent items cover 8 tile rows x 4 columns when the
    // output is wide (8192 x 8192 x 16384: 955 -> 820 us against groups of
    // 2), 16 x 2 when it has few tile columns (131072 x 512 x 2048: 139 us
    // against 147 with groups of 8)
    g.gi = g.tiles_j >= 16 ? 8 : 2;
    int grid = cu_count();
    if (grid > g.items) grid = g.items;
    const bool nt = l.K <= kNtMaxContraction;
#define FP8K_LAUNCH(FA, FB)                                                                                     \
    if (nt) hipLaunchKernelGGL((gemm_tensor_kernel<FA, FB, true>), dim3(grid), dim3(NW * 64), 0, stream, g);  \
    else hipLaunchKernelGGL((gemm_tensor_kernel<FA, FB, false>), dim3(grid), dim3(NW * 64), 0, stream, g)
    if (g.gelu_keys) {
        // the keys are emitted for E4M3 x E4M3 only (the forward GEMM)
        if (l.fa != 0 || l.fb != 0) return hipErrorInvalidValue;
        if (nt) hipLaunchKernelGGL((gemm_tensor_kernel<0, 0, true, true>), dim3(grid), dim3(NW * 64), 0, stream, g);
        else hipLaunchKernelGGL((gemm_tensor_kernel<0, 0, false, true>), dim3(grid), dim3(NW * 64), 0, stream, g);
        return hipGetLastError();
    }
    if (l.fa == 0 && l.fb == 0) { FP8K_LAUNCH(0, 0); }
    else if (l.fa == 1 && l.fb == 0) { FP8K_LAUNCH(1, 0); }
    else if (l.fa == 0 && l.fb == 1) { FP8K_LAUNCH(0, 1); }
    else { FP8K_LAUNCH(1, 1); }
#undef FP8K_LAUNCH
    return hipGetLastError();
}

}  // namespace fp8k
