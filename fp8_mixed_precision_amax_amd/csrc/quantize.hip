// Current-scaling FP8 quantizers for gfx950.
//
// Method ("Native FP8 MLP reconstruction", implementation paragraph): the
// scale of every tensor comes from its current amax, and one fused cast
// emits the ordinary and the transposed FP8 layouts.  Block scaling follows
// the Float8BlockScaling recipe named in TransformerEngine issue 2852
// (opening post): blockwise amax, no amax history.
//
// Kernels
//   amax_partial_kernel<STREAM>
//                         tensorwise amax, pass 1: grid-stride 16-byte loads,
//                         packed 16-bit max on bf16 magnitude bits, wave and
//                         workgroup reduction, one partial max per workgroup.
//   cast_kernel<FMT,MODE> one wave per 128x128 tile, no LDS: lane (rb, cb)
//                         owns columns cb*8..+7 of rows rb*16..+15 and
//                         64+rb*16..+15 (16-byte loads, 256 contiguous bytes
//                         per row per instruction); codes from the hardware
//                         converters (v_cvt_pk_fp8/bf8_f32, clamped first);
//                         the transposed layout comes from in-register 4x4
//                         byte transposes (v_perm_b32).  The two 16-row
//                         groups make every transposed store instruction
//                         write whole 64-byte spans (4 lanes x 16 bytes),
//                         issued as ordinary write-back stores so the L2
//                         merges them; the row layout goes out with 8-byte
//                         stores (16 lanes = 128 bytes), ordinary ones when
//                         it fits the memory-side cache (the GEMM that
//                         follows reads it back from there), non-temporal
//                         otherwise.
//     MODE 0 tensorwise: the scale is rebuilt in each wave from the amax
//            partials of pass 1 (so the cast needs no separate launch).
//     MODE 1 1x128 blocks: row blocks reduce over the 16 lanes of a DPP row;
//            column blocks reduce the lane's 32 rows, then across the 4 lane
//            rows with two xor shuffles.  The column layout is requantized
//            with the column-block scales.
//     MODE 2 128x128 blocks: one scale per tile (wave-wide reduction).
//     MODE 3 tensorwise, delayed: the scale from an amax history; per-tile
//            amaxes for history_update_kernel.
//   act_amax_kernel<ACT>, act_cast_kernel<FMT,MODE,ACT>
//                         the same passes on GELU(x) (ACT 1) or on
//                         dy * GELU'(x) (ACT 2), the activation between the
//                         two linears of an MLP block, computed from LDS
//                         tables as the data arrives (act.hpp) and never
//                         written out: each workgroup copies its table to
//                         LDS once and then loops over tiles.
#include "act.hpp"
#include "gelu_keys.hpp"
#include "device.hpp"
#include "internal.hpp"

namespace fp8k {

constexpr int kAmaxThreads = 256;
constexpr int kAmaxStreamThreads = 1024;   // the streamed sweep: 4x the threads, same partial count

// Partial maxima are bf16 magnitude bits (16 bits): the workgroup's maximum
// of the threads' packed magnitude maxima m goes to partial[blockIdx.x], and
// workgroup 0 zero-fills the unused tail of the kMaxAmaxPartials slots so
// readers may scan all of them.
__device__ __forceinline__ void amax_store_partial(uint32_t m, uint16_t* __restrict__ partial, int block,
                                                   int nblocks) {
    m = wave_max_u32(hmax_u16(m));
    __shared__ uint32_t red[kAmaxStreamThreads / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = red[0];
        for (int w = 1; w < (int)(blockDim.x >> 6); w++) r = r > red[w] ? r : red[w];
        partial[block] = (uint16_t)r;
    }
    if (block == 0)
        for (int p = nblocks + threadIdx.x; p < kMaxAmaxPartials; p += (int)blockDim.x) partial[p] = 0;
}
__device__ __forceinline__ void amax_store_partial(uint32_t m, uint16_t* __restrict__ partial) {
    amax_store_partial(m, partial, (int)blockIdx.x, (int)gridDim.x);
}

__device__ __forceinline__ uint32_t mag8_max(uint32_t m, uint4 v) {
    return pkmax_u16(m, pkmax_u16(pkmax_u16(mag2(v.x), mag2(v.y)), pkmax_u16(mag2(v.z), mag2(v.w))));
}

// One sweep of the tensor from front to back (grid-stride, one 16-byte load
// per thread per step).  A tensor that fits the memory-side cache is read
// with ordinary loads, so the cast that follows (last tile first) finds the
// most recently read data still cached.  A larger one cannot stay cached
// (the cast gains nothing from the cache: measured) and is streamed with
// non-temporal loads, which also spare the cache's dirty lines (left by the
// kernel before) the write-back an allocating read would force: after a
// 512 MiB write, ordinary loads read at 3.2-3.6 TB/s and non-temporal ones at
// 6.2-6.9 TB/s.  One load in flight per thread (2048 x 1024 threads: 32 MiB
// outstanding, all within one contiguous window of the tensor) measured
// faster than four spaced a grid stride apart: 131072 x 2048 quantize
// 294.5 -> 284.3 us, 262144 x 2048 596 -> 574 us.
// The packed magnitude maximum of this thread's share of x when `nblocks`
// workgroups sweep it and this one is number `block`.
template <bool STREAM>
__device__ __forceinline__ uint32_t amax_sweep(const uint4* __restrict__ x, int64_t n16, int block, int nblocks) {
    uint32_t m = 0;
    const int64_t stride = (int64_t)nblocks * blockDim.x;
    for (int64_t i = (int64_t)block * blockDim.x + threadIdx.x; i < n16; i += stride)
        m = mag8_max(m, STREAM ? ld_nt16(x + i) : x[i]);
    return m;
}

template <bool STREAM>
__global__ __launch_bounds__(kAmaxStreamThreads) void amax_partial_kernel(const uint4* __restrict__ x, int64_t n16,
                                                                          uint16_t* __restrict__ partial) {
    amax_store_partial(amax_sweep<STREAM>(x, n16, (int)blockIdx.x, (int)gridDim.x), partial);
}

// Pass 1 of two tensorwise quantizes in one launch (a layer's input a and
// its weight b): workgroups [0, gb) sweep the small b first, so they run
// beside a's rather than after them, the rest sweep a; each part writes its
// own partials as a launch of its own would.
template <bool STREAM_A>
__global__ __launch_bounds__(kAmaxStreamThreads) void amax_pair_kernel(const uint4* __restrict__ xa, int64_t na16,
                                                                       uint16_t* __restrict__ pa,
                                                                       const uint4* __restrict__ xb, int64_t nb16,
                                                                       uint16_t* __restrict__ pb, int gb) {
    const int b = (int)blockIdx.x;
    if (b < gb) amax_store_partial(amax_sweep<false>(xb, nb16, b, gb), pb, b, gb);
    else amax_store_partial(amax_sweep<STREAM_A>(xa, na16, b - gb, (int)gridDim.x - gb), pa, b - gb, (int)gridDim.x - gb);
}

// Table bytes of an activation: the bf16 GELU table (ACT 1) or the fp32 GELU'
// table (ACT 2).
template <int ACT> constexpr uint32_t act_table_bytes() { return ACT == 2 ? kActEntries * 4 : kActEntries * 2; }

// amax of GELU(x) (ACT 1) or of dGELU(x, x2) (ACT 2): the transform is
// applied as in the cast, so both passes see the same bf16 values.  One
// load per input in flight per thread (as amax_sweep; four spaced a grid
// stride apart measured 4-5 us slower on 131072 x 2048); non-temporal ones
// (STREAM) for inputs larger than the memory-side cache.
template <int ACT, bool STREAM>
__device__ __forceinline__ uint4 amax_ld(const uint4* p) {
    if constexpr (STREAM) return ld_nt16(p);
    else return *p;
}

template <int ACT, bool STREAM>
__global__ __launch_bounds__(kAmaxStreamThreads) void act_amax_kernel(const uint4* __restrict__ x,
                                                                const uint4* __restrict__ x2, int64_t n16,
                                                                uint16_t* __restrict__ partial, const void* gtab) {
    __shared__ __align__(16) uint32_t tab[act_table_bytes<ACT>() / 4];
    act_table_to_lds(tab, gtab, sizeof(tab));
    __syncthreads();
    uint32_t m = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i < n16; i += stride) {
        const uint4 v = amax_ld<ACT, STREAM>(x + i);
        if constexpr (ACT == 1) m = mag8_max(m, gelu8(v, reinterpret_cast<const uint16_t*>(tab)));
        else m = mag8_max(m, dgelu8(v, amax_ld<ACT, STREAM>(x2 + i), reinterpret_cast<const float*>(tab)));
    }
    amax_store_partial(m, partial);
}

struct CastArgs {
    const uint16_t* x;  // [R, C] bf16
    int64_t R, C;
    uint8_t* q_row;     // [R, C] or null
    uint8_t* q_col;     // [C, R] or null
    float* scale;       // tensor: [1]; 1x128: [C/128, R] (block (r, cb) at cb*R + r); 128x128: [R/128, C/128]
    float* scale_inv;
    float* scale_col;   // 1x128 only: [R/128, C] (block (c, rb) at rb*C + c)
    float* scale_inv_col;
    float* amax_out;    // tensor only, optional
    const uint16_t* partial;  // tensor only: kMaxAmaxPartials amax partials of pass 1 (unused slots 0)
    const float* hist;        // delayed only: amax history [hist_len]
    int hist_len;
    uint16_t* tile_amax;      // delayed only: amax of each 128x128 tile (bf16 magnitude bits)
    const uint16_t* x2;       // dGELU only: GELU's input [R, C]; x is the gradient of its output
    const void* act_tab;      // GELU / GELU' table (global memory), act_cast_kernel only
    const uint16_t* gelu_keys; // GELU, tensorwise, optional: the GELU amax keys of x (the amax
                               // comes from them instead of `partial`)
    int row_cached;           // row layout with ordinary (cached) stores instead of non-temporal
};

// 8 bytes of the row layout.  The GEMM that follows a quantize reads its row
// layout at once: up to 128 MiB it is written with ordinary stores and read
// back from the memory-side cache (131072 x 2048 x 512 GEMM after the
// quantize of its 64 MiB operand: 186 -> 155 us), larger ones would evict
// more than they keep (the two 256 MiB cases slowed by 6-9 us) and stream.
__device__ __forceinline__ void st_row8(const CastArgs& a, uint8_t* p, uint2 w) {
    if (a.row_cached) *reinterpret_cast<uint2*>(p) = w;
    else st_nt8(p, w);
}

// One 128x128 tile, by one wave.  slot < number of tiles.  ACT 1 / 2 encode
// GELU(x) / dGELU(x, x2) instead of x (tab: the table in LDS).
template <int FMT, int MODE, int ACT>
__device__ __forceinline__ void cast_tile(const CastArgs& a, int64_t slot, const void* tab) {
    // lane, rowA and col0 are made opaque: in a loop over tiles the
    // compiler would otherwise hoist everything derived from the lane (row
    // offsets, shuffle addresses, lane masks) out of the loop, each value
    // holding a register for the whole kernel
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int64_t tiles_c = a.C >> 7;
    const int64_t ntiles = (a.R >> 7) * tiles_c;
    // tensorwise: last tile first (the amax pass swept front to back, so the
    // tail of the tensor is the part most likely still cached)
    const int64_t tile = MODE == 0 ? ntiles - 1 - slot : slot;
    const int64_t tr = tile / tiles_c, tc = tile - tr * tiles_c;
    const int rb = lane >> 4, cb = lane & 15;
    // this lane's rows: i < 16 -> rowA + i, i >= 16 -> rowB + (i - 16)
    int64_t rowA = tr * 128 + rb * 16;
    int64_t col0 = tc * 128 + cb * 8;    // first of this lane's 8 columns
    asm volatile("" : "+v"(rowA), "+v"(col0));
    const int64_t rowB = rowA + 64;
#define FP8K_ROW(i) ((i) < 16 ? rowA + (i) : rowB + ((i) - 16))

    // tensorwise: the amax partials (issued first, they return first)
    uint4 pw[kMaxAmaxPartials / 512];
    if constexpr (MODE == 0) {
#pragma unroll
        for (int r = 0; r < kMaxAmaxPartials / 512; r++)
            pw[r] = reinterpret_cast<const uint4*>(a.partial)[r * 64 + lane];
    }
    // delayed: the amax history, likewise first
    float hv[kMaxHistory / 64];
    if constexpr (MODE == 3) {
#pragma unroll
        for (int r = 0; r < kMaxHistory / 64; r++) {
            const int idx = r * 64 + lane;
            hv[r] = idx < a.hist_len ? a.hist[idx] : 0.0f;
        }
    }

    // ---- load 32 rows x 8 bf16 ------------------------------------------
    uint4 v[32];
    if constexpr (ACT == 2) {
        // the gradient and GELU's input, 16 rows at a time (all 32 rows of
        // both would need every register of the wave)
        const float* t = static_cast<const float*>(tab);
        us2_t far = {0, 0};
        uint32_t dm = 0;
#pragma unroll
        for (int hf = 0; hf < 2; hf++) {
            uint4 u[16];
#pragma unroll
            for (int i = 0; i < 16; i++) {
                v[16 * hf + i] = ld_nt16(a.x + FP8K_ROW(16 * hf + i) * a.C + col0);
                u[i] = ld_nt16(a.x2 + FP8K_ROW(16 * hf + i) * a.C + col0);
            }
            // 4 rows between scheduling barriers: otherwise every table read
            // of the tile is hoisted to the top, each holding a register
#pragma unroll
            for (int i = 0; i < 16; i++) {
                v[16 * hf + i] = dgelu8_fast(v[16 * hf + i], u[i], t, far, dm);
                if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);
            }
        }
        // a tile with an input outside the table or a non-finite gradient:
        // read it again and take the exact path, 4 rows at a time
        if (act_need_full(far, dm)) {
#pragma unroll
            for (int i = 0; i < 32; i++) {
                v[i] = dgelu8_full(ld_nt16(a.x + FP8K_ROW(i) * a.C + col0), ld_nt16(a.x2 + FP8K_ROW(i) * a.C + col0), t);
                if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; i++) v[i] = ld_nt16(a.x + FP8K_ROW(i) * a.C + col0);
        if constexpr (ACT == 1) {
            const uint16_t* t = static_cast<const uint16_t*>(tab);
            us2_t far = {0, 0};
            // 4 rows between scheduling barriers: otherwise every table read
            // of the tile is hoisted to the top, each holding a register
#pragma unroll
            for (int i = 0; i < 32; i++) {
                v[i] = gelu8_fast(v[i], t, far);
                if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);
            }
            if (act_need_full(far)) {
#pragma unroll
                for (int i = 0; i < 32; i++) {
                    v[i] = gelu8_full(ld_nt16(a.x + FP8K_ROW(i) * a.C + col0), t);
                    if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }

    // ---- scales ---------------------------------------------------------
    float s_tile = 1.0f;          // MODE 0, 2 and 3
    bool nan_any = false;
    if constexpr (MODE == 0) {
        uint32_t m = 0;
#pragma unroll
        for (int r = 0; r < kMaxAmaxPartials / 512; r++)
            m = pkmax_u16(m, pkmax_u16(pkmax_u16(pw[r].x, pw[r].y), pkmax_u16(pw[r].z, pw[r].w)));
        m = wave_max_u32(hmax_u16(m));
        float si;
        scale_from_amax_bits<FMT>(m, s_tile, si);
        nan_any = m > 0x7F80u;
        if (slot == 0 && lane == 0) {
            a.scale[0] = s_tile;
            a.scale_inv[0] = si;
            if (a.amax_out) a.amax_out[0] = m > 0x7F80u ? __uint_as_float(0x7FC00000u) : __uint_as_float(m << 16);
        }
    } else if constexpr (MODE == 3) {
        // scale from the largest history entry (NaN if any entry is NaN)
        float hm = 0.0f;
        bool hn = false;
#pragma unroll
        for (int r = 0; r < kMaxHistory / 64; r++) {
            hn |= hv[r] != hv[r];
            hm = hv[r] > hm ? hv[r] : hm;
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) hm = fmaxf(hm, __shfl_xor(hm, o, 64));
        float si;
        scale_from_amax_f32<FMT>(__ballot(hn) != 0 ? __uint_as_float(0x7FC00000u) : hm, s_tile, si);
        // this tile's amax, for the history update and the NaN patch
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 32; i++)
            m = pkmax_u16(m, pkmax_u16(pkmax_u16(mag2(v[i].x), mag2(v[i].y)), pkmax_u16(mag2(v[i].z), mag2(v[i].w))));
        m = wave_max_u32(hmax_u16(m));
        nan_any = m > 0x7F80u;
        if (lane == 0) a.tile_amax[tile] = (uint16_t)m;
        if (slot == 0 && lane == 0) {
            a.scale[0] = s_tile;
            a.scale_inv[0] = si;
        }
    } else if constexpr (MODE == 2) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 32; i++)
            m = pkmax_u16(m, pkmax_u16(pkmax_u16(mag2(v[i].x), mag2(v[i].y)), pkmax_u16(mag2(v[i].z), mag2(v[i].w))));
        m = wave_max_u32(hmax_u16(m));
        float si;
        scale_from_amax_bits<FMT>(m, s_tile, si);
        nan_any = m > 0x7F80u;
        if (lane == 0) {
            a.scale[tr * tiles_c + tc] = s_tile;
            a.scale_inv[tr * tiles_c + tc] = si;
        }
    }

    if constexpr (MODE == 0 || MODE == 2 || MODE == 3) {
        // One scale for the whole tile: the column layout is the transpose
        // of the row layout.
        uint2 code[32];
#pragma unroll
        for (int i = 0; i < 32; i++) {
            code[i] = enc8<FMT>(v[i], s_tile);
            if (nan_any) code[i] = patch_nan8(v[i], code[i]);
        }
        if (a.q_row) {
#pragma unroll
            for (int i = 0; i < 32; i++) st_row8(a, a.q_row + FP8K_ROW(i) * a.C + col0, code[i]);
        }
        if (a.q_col) {
            uint32_t t[8][8];   // t[column j][row group h]
#pragma unroll
            for (int h = 0; h < 8; h++) {
                transpose4x4(code[4 * h].x, code[4 * h + 1].x, code[4 * h + 2].x, code[4 * h + 3].x,
                             t[0][h], t[1][h], t[2][h], t[3][h]);
                transpose4x4(code[4 * h].y, code[4 * h + 1].y, code[4 * h + 2].y, code[4 * h + 3].y,
                             t[4][h], t[5][h], t[6][h], t[7][h]);
            }
#pragma unroll
            for (int j = 0; j < 8; j++) {
                uint8_t* dst = a.q_col + (col0 + j) * a.R;
                *reinterpret_cast<uint4*>(dst + rowA) = make_uint4(t[j][0], t[j][1], t[j][2], t[j][3]);
                *reinterpret_cast<uint4*>(dst + rowB) = make_uint4(t[j][4], t[j][5], t[j][6], t[j][7]);
            }
        }
    } else {
        // ---- MODE 1: 1x128 row blocks and 128x1 column blocks ------------
        if (a.q_row) {
            // row maxima: two rows per packed dword, reduced over the DPP row
            uint32_t rm[16];
#pragma unroll
            for (int p = 0; p < 16; p++) {
                uint32_t m0 = pkmax_u16(pkmax_u16(mag2(v[2 * p].x), mag2(v[2 * p].y)), pkmax_u16(mag2(v[2 * p].z), mag2(v[2 * p].w)));
                uint32_t m1 = pkmax_u16(pkmax_u16(mag2(v[2 * p + 1].x), mag2(v[2 * p + 1].y)), pkmax_u16(mag2(v[2 * p + 1].z), mag2(v[2 * p + 1].w)));
                rm[p] = hmax_u16(m0) | (hmax_u16(m1) << 16);
                rm[p] = row16_pkmax(rm[p]);
            }
            // every lane of a 16-lane row group holds the maxima of the group's
            // 32 rows; lane cb computes the scales of rows 2cb and 2cb+1 (the
            // fp32 divisions once per row, not once per lane) and stores them:
            // the tile's 128 row scales are one contiguous run of the
            // block-column-major scale array
            uint32_t mine = 0;
#pragma unroll
            for (int p = 0; p < 16; p++) mine = (p == cb) ? rm[p] : mine;
            float s0, si0, s1, si1;
            scale_from_amax_bits<FMT>(mine & 0xFFFFu, s0, si0);
            scale_from_amax_bits<FMT>(mine >> 16, s1, si1);
            {
                const int64_t r0 = FP8K_ROW(2 * cb);   // rows 2cb, 2cb+1 are adjacent, r0 even
                *reinterpret_cast<float2*>(a.scale + tc * a.R + r0) = make_float2(s0, s1);
                *reinterpret_cast<float2*>(a.scale_inv + tc * a.R + r0) = make_float2(si0, si1);
            }
            // NaN patching only in tiles that hold a NaN (wave-uniform branch;
            // patch_nan8 tests each element itself)
            uint32_t mrow = rm[0];
#pragma unroll
            for (int p = 1; p < 16; p++) mrow = pkmax_u16(mrow, rm[p]);
            const bool nan_rows = __ballot(hmax_u16(mrow) > 0x7F80u) != 0;
            const int src0 = (lane & ~15) * 4;   // byte address of lane 0 of this row group
#pragma unroll
            for (int p = 0; p < 16; p++) {
                // scales of rows 2p, 2p+1 from lane p of the row group
                const float sp0 = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src0 + 4 * p, __builtin_bit_cast(int, s0)));
                const float sp1 = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src0 + 4 * p, __builtin_bit_cast(int, s1)));
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const int i = 2 * p + h;
                    uint2 c = enc8<FMT>(v[i], h ? sp1 : sp0);
                    if (nan_rows) c = patch_nan8(v[i], c);
                    st_row8(a, a.q_row + FP8K_ROW(i) * a.C + col0, c);
                }
            }
        }
        if (a.q_col) {
            // column maxima over the lane's 32 rows, then over the 4 lane rows
            uint32_t cm[4];
            cm[0] = mag2(v[0].x); cm[1] = mag2(v[0].y); cm[2] = mag2(v[0].z); cm[3] = mag2(v[0].w);
#pragma unroll
            for (int i = 1; i < 32; i++) {
                cm[0] = pkmax_u16(cm[0], mag2(v[i].x));
                cm[1] = pkmax_u16(cm[1], mag2(v[i].y));
                cm[2] = pkmax_u16(cm[2], mag2(v[i].z));
                cm[3] = pkmax_u16(cm[3], mag2(v[i].w));
            }
#pragma unroll
            for (int g = 0; g < 4; g++) {
                cm[g] = pkmax_u16(cm[g], (uint32_t)__shfl_xor((int)cm[g], 16, 64));
                cm[g] = pkmax_u16(cm[g], (uint32_t)__shfl_xor((int)cm[g], 32, 64));
            }
            float sc[8], si[8];
            bool nan_lane = false;
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const uint32_t m = (j & 1) ? (cm[j >> 1] >> 16) : (cm[j >> 1] & 0xFFFFu);
                scale_from_amax_bits<FMT>(m, sc[j], si[j]);
                nan_lane |= m > 0x7F80u;
            }
            // the tile's 128 column scales: one contiguous run of the
            // block-row-major array; lanes of row group 0 store the scales,
            // those of row group 1 the inverses, 8 columns (32 bytes) each
            if (rb < 2) {
                float* d = (rb == 0 ? a.scale_col : a.scale_inv_col) + tr * a.C + col0;
                const float* w = rb == 0 ? sc : si;
                *reinterpret_cast<float4*>(d) = make_float4(w[0], w[1], w[2], w[3]);
                *reinterpret_cast<float4*>(d + 4) = make_float4(w[4], w[5], w[6], w[7]);
            }
            const bool nan_col = __ballot(nan_lane) != 0;   // wave-uniform, as for the rows
            uint32_t t[8][8];
#pragma unroll
            for (int h = 0; h < 8; h++) {
                uint2 c0 = enc8_cols<FMT>(v[4 * h], sc);
                uint2 c1 = enc8_cols<FMT>(v[4 * h + 1], sc);
                uint2 c2 = enc8_cols<FMT>(v[4 * h + 2], sc);
                uint2 c3 = enc8_cols<FMT>(v[4 * h + 3], sc);
                if (nan_col) {
                    c0 = patch_nan8(v[4 * h], c0);
                    c1 = patch_nan8(v[4 * h + 1], c1);
                    c2 = patch_nan8(v[4 * h + 2], c2);
                    c3 = patch_nan8(v[4 * h + 3], c3);
                }
                transpose4x4(c0.x, c1.x, c2.x, c3.x, t[0][h], t[1][h], t[2][h], t[3][h]);
                transpose4x4(c0.y, c1.y, c2.y, c3.y, t[4][h], t[5][h], t[6][h], t[7][h]);
            }
#pragma unroll
            for (int j = 0; j < 8; j++) {
                uint8_t* dst = a.q_col + (col0 + j) * a.R;
                *reinterpret_cast<uint4*>(dst + rowA) = make_uint4(t[j][0], t[j][1], t[j][2], t[j][3]);
                *reinterpret_cast<uint4*>(dst + rowB) = make_uint4(t[j][4], t[j][5], t[j][6], t[j][7]);
            }
        }
    }
#undef FP8K_ROW
}

template <int FMT, int MODE>
__global__ __launch_bounds__(256) void cast_kernel(CastArgs a) {
    const int64_t ntiles = (a.R >> 7) * (a.C >> 7);
    const int64_t slot = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (slot >= ntiles) return;
    cast_tile<FMT, MODE, 0>(a, slot, nullptr);
}

// The casts of two tensorwise quantizes in one launch: workgroups [0, gb)
// take the small b's tiles (four per workgroup) first, the rest a's.
template <int FMT>
__global__ __launch_bounds__(256) void cast_pair_kernel(CastArgs a, CastArgs b, int gb) {
    const bool small = (int)blockIdx.x < gb;
    const CastArgs& c = small ? b : a;
    const int64_t ntiles = (c.R >> 7) * (c.C >> 7);
    const int64_t slot = (int64_t)((int)blockIdx.x - (small ? 0 : gb)) * 4 + (threadIdx.x >> 6);
    if (slot >= ntiles) return;
    if (small) cast_tile<FMT, 0, 0>(b, slot, nullptr);
    else cast_tile<FMT, 0, 0>(a, slot, nullptr);
}

// MODE 0 or 1 on GELU(x) / dGELU(x, x2): the table goes to LDS once per
// workgroup, then each wave casts one tile (the tensorwise loop below takes
// further tiles only if a launch has fewer workgroups than tiles / 4; in
// 1x128 blocks a loop would make the compiler interleave the row- and
// column-block parts and need twice the registers).
template <int FMT, int MODE, int ACT>
__global__ __launch_bounds__(256) void act_cast_kernel(CastArgs a) {
    __shared__ __align__(16) uint32_t tab[act_table_bytes<ACT>() / 4];
    act_table_to_lds(tab, a.act_tab, sizeof(tab));
    if constexpr (MODE == 0 && ACT == 1) {
        if (a.gelu_keys) {
            // the amax of GELU(x) from the keys x's producer wrote: every
            // workgroup reduces the four key arrays (16 KiB), evaluates GELU
            // at the values they name from the table in LDS, and the tiles
            // read that amax as a partials array whose slot 0 holds it
            __shared__ __align__(16) uint16_t kpart[kMaxAmaxPartials];
            __shared__ uint32_t kred[kGeluKeyArrays][4];
            uint32_t k[kGeluKeyArrays];
#pragma unroll
            for (int q = 0; q < kGeluKeyArrays; q++) {
                const uint4 w = reinterpret_cast<const uint4*>(a.gelu_keys + q * kMaxAmaxPartials)[threadIdx.x];
                k[q] = wave_max_u32(hmax_u16(pkmax_u16(pkmax_u16(w.x, w.y), pkmax_u16(w.z, w.w))));
            }
            for (int s = (int)threadIdx.x; s < kMaxAmaxPartials / 8; s += 256)
                reinterpret_cast<uint4*>(kpart)[s] = make_uint4(0, 0, 0, 0);
            if ((threadIdx.x & 63) == 0)
#pragma unroll
                for (int q = 0; q < kGeluKeyArrays; q++) kred[q][threadIdx.x >> 6] = k[q];
            __syncthreads();    // also the table copy
            if (threadIdx.x == 0) {
#pragma unroll
                for (int q = 0; q < kGeluKeyArrays; q++) {
                    uint32_t m = kred[q][0];
                    for (int w = 1; w < 4; w++) m = m > kred[q][w] ? m : kred[q][w];
                    k[q] = m;
                }
                const uint16_t* t = reinterpret_cast<const uint16_t*>(tab);
                kpart[0] = (uint16_t)gelu_amax_from_keys(k, [t](uint32_t b) { return gelu_one(b, t); });
            }
            a.partial = kpart;
        }
    }
    __syncthreads();
    const int64_t ntiles = (a.R >> 7) * (a.C >> 7);
    const int64_t slot0 = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if constexpr (MODE == 1) {
        if (slot0 < ntiles) cast_tile<FMT, MODE, ACT>(a, slot0, tab);
    } else {
        for (int64_t slot = slot0; slot < ntiles; slot += (int64_t)gridDim.x * 4) cast_tile<FMT, MODE, ACT>(a, slot, tab);
    }
}

// Delayed scaling, after the cast: this call's amax from the per-tile maxima,
// then the history rolls by one (oldest entry dropped) and takes it in front.
__global__ __launch_bounds__(256) void history_update_kernel(const uint16_t* __restrict__ tile_amax, int64_t ntiles,
                                                             float* __restrict__ hist, int H, float* amax_out) {
    uint32_t m = 0;
    for (int64_t i = threadIdx.x; i < ntiles; i += 256) m = m > tile_amax[i] ? m : tile_amax[i];
    m = wave_max_u32(m);
    __shared__ uint32_t red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = red[0];
    for (int w = 1; w < 4; w++) m = m > red[w] ? m : red[w];
    const float amax = m > 0x7F80u ? __uint_as_float(0x7FC00000u) : __uint_as_float(m << 16);
    float v[kMaxHistory / 256];
#pragma unroll
    for (int k = 0; k < kMaxHistory / 256; k++) {
        const int i = (int)threadIdx.x + 256 * k;
        v[k] = i + 1 < H ? hist[i] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMaxHistory / 256; k++) {
        const int i = (int)threadIdx.x + 256 * k;
        if (i + 1 < H) hist[i + 1] = v[k];
    }
    if (threadIdx.x == 0) {
        hist[0] = amax;
        if (amax_out) amax_out[0] = amax;
    }
}

int amax_partial_count(int64_t numel) {
    // about eight workgroups per CU, one 16-byte load per thread per sweep
    // step; a small tensor (a weight) gets up to 512 workgroups of one load
    // per thread instead of a few workgroups of sixteen dependent steps
    const int64_t n16 = numel / 8;
    int64_t g = (n16 + (int64_t)kAmaxThreads * 16 - 1) / ((int64_t)kAmaxThreads * 16);
    int64_t g1 = (n16 + kAmaxThreads - 1) / kAmaxThreads;
    if (g1 > 512) g1 = 512;
    if (g < g1) g = g1;
    if (g < 1) g = 1;
    if (g > kMaxAmaxPartials) g = kMaxAmaxPartials;
    return (int)g;
}

// Quantize GELU(x) (q.act 1) or dGELU(x, x2) (q.act 2), tensorwise (two
// passes) or in 1x128 blocks (one pass).
hipError_t launch_act_quantize(const QuantizeLaunch& q, CastArgs& a, hipStream_t stream) {
    ActTables t;
    hipError_t e = act_tables(stream, t);
    if (e != hipSuccess) return e;
    a.act_tab = q.act == 1 ? static_cast<const void*>(t.gelu) : static_cast<const void*>(t.dgelu);
    a.gelu_keys = q.gelu_keys;
    if (q.scaling == 0 && !q.partial_given && !q.gelu_keys) {
        // about two workgroups per CU: each one copies the table to LDS first
        const int64_t n16 = q.rows * q.cols / 8;
        int64_t g = (n16 + (int64_t)kAmaxThreads * 16 - 1) / ((int64_t)kAmaxThreads * 16);
        g = g < 1 ? 1 : (g > 512 ? 512 : g);
        const bool big = q.rows * q.cols * 2 * (q.act == 2 ? 2 : 1) > (int64_t(256) << 20);
        const uint4* x = static_cast<const uint4*>(q.x);
        const uint4* x2 = static_cast<const uint4*>(q.x2);
#define FP8K_AMAX(A, S) \
    hipLaunchKernelGGL((act_amax_kernel<A, S>), dim3((unsigned)g), dim3(kAmaxStreamThreads), 0, stream, x, x2, n16, \
                       q.partial, a.act_tab)
        if (q.act == 1) {
            if (big) FP8K_AMAX(1, true); else FP8K_AMAX(1, false);
        } else {
            if (big) FP8K_AMAX(2, true); else FP8K_AMAX(2, false);
        }
#undef FP8K_AMAX
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // one tile per wave, four per workgroup, each workgroup copying its table
    // first: tensorwise, this beat 512 (and 1024) workgroups looping over
    // tiles, which copied the table fewer times (MLP block forward + backward
    // 1.7838 -> 1.7487 ms; the GELU quantize of 131072 x 2048 345 -> 327 us,
    // the dGELU one 509 -> 488 us)
    const int64_t ntiles = (q.rows / 128) * (q.cols / 128);
    const dim3 grid((unsigned)((ntiles + 3) / 4));
#define FP8K_ACT(F, M, A) hipLaunchKernelGGL((act_cast_kernel<F, M, A>), grid, dim3(256), 0, stream, a)
#define FP8K_ACT_F(M, A) \
    if (q.format == 0) FP8K_ACT(0, M, A); \
    else FP8K_ACT(1, M, A)
    if (q.scaling == 0) {
        if (q.act == 1) { FP8K_ACT_F(0, 1); } else { FP8K_ACT_F(0, 2); }
    } else {
        if (q.act == 1) { FP8K_ACT_F(1, 1); } else { FP8K_ACT_F(1, 2); }
    }
#undef FP8K_ACT_F
#undef FP8K_ACT
    return hipGetLastError();
}

static CastArgs cast_args(const QuantizeLaunch& q) {
    CastArgs a;
    a.x = static_cast<const uint16_t*>(q.x);
    a.R = q.rows;
    a.C = q.cols;
    a.q_row = static_cast<uint8_t*>(q.q_row);
    a.q_col = static_cast<uint8_t*>(q.q_col);
    a.scale = q.scale;
    a.scale_inv = q.scale_inv;
    a.scale_col = q.scale_col;
    a.scale_inv_col = q.scale_inv_col;
    a.amax_out = q.amax;
    a.partial = q.partial;
    a.hist = q.hist;
    a.hist_len = q.hist_len;
    a.tile_amax = q.partial;
    a.x2 = static_cast<const uint16_t*>(q.x2);
    a.act_tab = nullptr;
    a.gelu_keys = nullptr;
    a.row_cached = q.rows * q.cols <= (int64_t(128) << 20);
    return a;
}

hipError_t launch_quantize(const QuantizeLaunch& q, hipStream_t stream) {
    CastArgs a = cast_args(q);
    if (q.act) return launch_act_quantize(q, a, stream);
    if (q.scaling == 0 && !q.partial_given) {
        const int g = amax_partial_count(q.rows * q.cols);
        // above 256 MiB of bf16 the tensor outgrows the memory-side cache
        if (q.rows * q.cols * 2 > (int64_t(256) << 20))
            hipLaunchKernelGGL(amax_partial_kernel<true>, dim3(g), dim3(kAmaxStreamThreads), 0, stream,
                               static_cast<const uint4*>(q.x), q.rows * q.cols / 8, q.partial);
        else
            hipLaunchKernelGGL(amax_partial_kernel<false>, dim3(g), dim3(kAmaxThreads), 0, stream,
                               static_cast<const uint4*>(q.x), q.rows * q.cols / 8, q.partial);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // four waves (tiles) per workgroup; a small tensor (a weight: 64 tiles
    // for 2048 x 512) takes one wave per workgroup, so its tiles spread over
    // as many CUs as there are tiles
    const int64_t ntiles = (q.rows / 128) * (q.cols / 128);
    const int wpg = ntiles < 1024 ? 1 : 4;
    const dim3 grid((unsigned)((ntiles + wpg - 1) / wpg));
#define FP8K_CAST(F, M) hipLaunchKernelGGL((cast_kernel<F, M>), grid, dim3(64 * wpg), 0, stream, a)
    if (q.format == 0) {
        if (q.scaling == 0) FP8K_CAST(0, 0);
        else if (q.scaling == 1) FP8K_CAST(0, 1);
        else if (q.scaling == 2) FP8K_CAST(0, 2);
        else FP8K_CAST(0, 3);
    } else {
        if (q.scaling == 0) FP8K_CAST(1, 0);
        else if (q.scaling == 1) FP8K_CAST(1, 1);
        else if (q.scaling == 2) FP8K_CAST(1, 2);
        else FP8K_CAST(1, 3);
    }
#undef FP8K_CAST
    if (q.scaling == 3) {
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(history_update_kernel, dim3(1), dim3(256), 0, stream, q.partial, ntiles, q.hist,
                           q.hist_len, q.amax);
    }
    return hipGetLastError();
}

}  // namespace fp8k

namespace fp8k {

// Two tensorwise quantizes (same format, plain input, amax pass included)
// as one amax launch and one cast launch: a layer's input x (a) and its
// weight (b), whose separate launches would each leave the GPU mostly idle
// for a small tensor.  The bytes written are those of two launch_quantize
// calls.
hipError_t launch_quantize_pair(const QuantizeLaunch& qa, const QuantizeLaunch& qb, hipStream_t stream) {
    const int64_t na16 = qa.rows * qa.cols / 8, nb16 = qb.rows * qb.cols / 8;
    const int ga = amax_partial_count(qa.rows * qa.cols);
    int64_t gb = (nb16 + kAmaxStreamThreads - 1) / kAmaxStreamThreads;
    if (gb > 512) gb = 512;
    if (gb < 1) gb = 1;
    const dim3 agrid((unsigned)(ga + gb));
    if (qa.rows * qa.cols * 2 > (int64_t(256) << 20))
        hipLaunchKernelGGL(amax_pair_kernel<true>, agrid, dim3(kAmaxStreamThreads), 0, stream,
                           static_cast<const uint4*>(qa.x), na16, qa.partial, static_cast<const uint4*>(qb.x), nb16,
                           qb.partial, (int)gb);
    else
        hipLaunchKernelGGL(amax_pair_kernel<false>, agrid, dim3(kAmaxStreamThreads), 0, stream,
                           static_cast<const uint4*>(qa.x), na16, qa.partial, static_cast<const uint4*>(qb.x), nb16,
                           qb.partial, (int)gb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const CastArgs a = cast_args(qa), b = cast_args(qb);
    const int64_t ta = (qa.rows / 128) * (qa.cols / 128), tb = (qb.rows / 128) * (qb.cols / 128);
    const int wa = (int)((ta + 3) / 4), wb = (int)((tb + 3) / 4);
    if (qa.format == 0)
        hipLaunchKernelGGL((cast_pair_kernel<0>), dim3((unsigned)(wa + wb)), dim3(256), 0, stream, a, b, wb);
    else
        hipLaunchKernelGGL((cast_pair_kernel<1>), dim3((unsigned)(wa + wb)), dim3(256), 0, stream, a, b, wb);
    return hipGetLastError();
}

}  // namespace fp8k
