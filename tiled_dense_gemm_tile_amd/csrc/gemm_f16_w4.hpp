// Four-wave kernel for D = A.B + C with 16-bit inputs, gfx950: the default
// for grids of at least half a wave of 256 x 256 output tiles.
//
// The workgroup computes a 256 x 256 output tile with 4 waves, one per SIMD,
// each owning a 128 x 128 quadrant as 8 x 8 blocks of 16 x 16 accumulators
// (v_mfma_f32_16x16x32: 256 accumulator registers per lane).  Large wave
// tiles keep LDS traffic low (per 64-wide K tile each wave reads 32 KiB of
// fragments against 64 KiB of tile data written by the direct global->LDS
// loads), and the 16x16 MFMA form draws less power per flop than 32x32, so
// the clock holds higher under load.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "gemm_f16.hpp"
#include "pipeline.hpp"

namespace tg {

// In-place MFMA on an AGPR accumulator block: acc = A.B + acc.
template <bool FP16>
__device__ __forceinline__ void mfma16_acc_asm(f32x4 &acc, const u32x4 &a, const u32x4 &b) {
    if constexpr (FP16)
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// acc = A.B (C operand the inline constant 0).
template <bool FP16>
__device__ __forceinline__ void mfma16_zero_asm(f32x4 &acc, const u32x4 &a, const u32x4 &b) {
    if constexpr (FP16)
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
}

// Wait states between the last MFMA writing the accumulators and any other
// instruction touching them (far more than the dependent-read hazard of a
// 16x16x32 MFMA needs).  Every accumulator passes through one of these
// statements, which issue in order, so no use can be scheduled before the
// s_nops.
template <int TM, int TN>
__device__ __forceinline__ void mfma_result_fence(f32x4 (&acc)[TM][TN]) {
    static_assert(TN == 8, "eight blocks per statement");
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        if (i == 0)
            asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 3"
                         : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]), "+a"(acc[i][4]),
                           "+a"(acc[i][5]), "+a"(acc[i][6]), "+a"(acc[i][7]));
        else
            asm volatile(""
                         : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]), "+a"(acc[i][4]),
                           "+a"(acc[i][5]), "+a"(acc[i][6]), "+a"(acc[i][7]));
    }
}

// K tiles are 64 wide: 128-byte LDS rows, so every global->LDS load
// instruction moves whole 128-byte lines (8 rows of a tile); A and B each
// have two ring slots of 32 KiB.  Per tile a wave issues 128 MFMAs in two K
// steps of 32, and the second step of tile t-1 runs after the barrier that
// opens tile t, so the matrix pipe does not drain at the barrier:
//   after barrier t:  the 64 MFMAs of tile t-1 step 1, with the fragment
//                     reads of tile t step 0 (one per 4 MFMAs) and the loads
//                     of A(t+1), B(t+1) (one per 4 MFMAs)
//                     the 64 MFMAs of tile t step 0, with the fragment reads
//                     of tile t step 1 (one per 3 MFMAs)
//                     wait for A(t+1), B(t+1); barrier t+1
// A tile's slots are read only between its own barrier and the next one, so
// the loads of tile t+1 go to the slots tile t-1 used, freed at barrier t.
//
// With C given and at least 18 K tiles, C is streamed into the accumulators
// during the first 18 tiles and the epilogue only writes D.  Those tiles are
// unrolled so the accumulator blocks they update have fixed register names:
// C part c -- the four blocks 4c .. 4c+3 -- is loaded at the end of tile c
// (after the tile's global->LDS loads, into register set c % 3) and added in
// tile c + 2, at a point where no MFMA on those blocks is in flight and many
// MFMAs separate the add from the block's previous and next update (blocks
// of rows 0..63 early in the tile, rows 64..127 in its second phase).  The
// barrier wait at the end of tile c leaves the part's loads in flight, so
// they have a whole tile to arrive from memory.  C thus arrives over 16
// tiles instead of all at the end.
//
// SPLIT (split-K): workgroup (split s, tile) multiplies K tiles
// [s * kt_split, (s + 1) * kt_split) of its output tile -- the A and B tile
// bases move by the range's first K element and the K loop runs over the
// range as if it were the whole K -- and writes the fp32 partial tile to
// workspace slice s through the same epilogue, with no C; the reduction
// kernel adds the slices and C.
//
// AT / BT: A (B) is stored MN-contiguous -- a(m,k) = A[k*lda + m] (b(k,n) =
// B[k*ldb + n]), i.e. K rows of M (N) elements -- instead of K-contiguous.
// Such an operand's K tile is loaded as it lies, 64 LDS rows of the tile's
// 256 M (N) elements (512 bytes), and its MFMA fragments (eight K-consecutive
// values of one column per lane) are read with ds_read_b64_tr_b16: within a
// 16-lane group, output lane i receives element i % 4 of the 8-byte reads of
// lanes 4 r + i / 4, r = 0..3 (probed on gfx950), so lanes reading four
// K-consecutive rows x 16 columns hand each lane one column's four K values;
// two such reads make a fragment.  The 32-byte chunk c of LDS row r sits at
// chunk c ^ (r & 3) ^ 4 * ((r >> 3) & 1): the four rows of one read and the
// two 16-lane groups read together fall on distinct banks.  The tile's K
// offset moves the base of a per-tile buffer resource whose extent ends at
// row K, so rows past K read as zeros; columns past M (N) feed only outputs
// that are never stored.
// With the balanced schedule, the step-0 fragments of tile t are read in the
// first half of window t and used by its second half.  Reads issued as asm
// (the transpose reads) are not tracked by the compiler, so before block row
// i of the second half the kernel waits explicitly until at most
// tr_row_wait(i) LDS operations remain: those issued after the reads row i
// needs -- A rows i + 1 .. 7 of the first half, and the step-1 reads the
// second half has issued before its MFMA 8 i (one per three MFMAs) -- where
// a transposed operand's read counts two operations (CA, CB).  A count above
// the field's 15 only makes the wait stricter.
template <int CA, int CB>
constexpr int tr_row_wait(int i) {
    int n = (7 - i) * CA;
    const int issued = (8 * i + 2) / 3;
    for (int m = 0; m < issued && m < 16; ++m) n += (m >= 1 && m <= 8) ? CB : CA;
    return n > 15 ? 15 : n;
}

// TM_: blocks of 16 rows per wave along M -- 8 (256 x 256 tiles) or 6
// (192 x 256 tiles, for grids whose 256 x 256 tiles fill only part of the
// last wave: 4000 x 3000 is 192 such tiles but 252 of 192 x 256).
//
// PERSIST: one workgroup per CU walks the tiles w, w + grid, w + 2 grid, ...
// (virtual workgroup ids, so the XCD-aware order is that of a full grid).
// After a tile's last K step it issues the next tile's K tile 0 loads (into
// the slots K tile 0 always uses) and only then stages and stores the
// finished tile's D, from the other slots, so those loads run while D
// drains.  Taken for calls without C, with 16-byte rows and D rows of whole
// 16-byte segments.
template <bool FP16, bool OUT_BF16, bool SH = false, bool SPLIT = false, bool AT = false, bool BT = false,
          int TM_ = 8, bool PERSIST = false>
__global__ void __launch_bounds__(256) gemm_f16_w4t_kernel(F16Args p, F16Epi e) {
    constexpr int NA = 2, NB = 2;                      // ring slots of A and B
    constexpr int DAUX = kStoreStream;                 // D store policy
    constexpr int TM = TM_, TN = 8;
    constexpr int BM = 32 * TM, BN = 256, KT = 64;     // tile
    constexpr int WTM = 16 * TM, WTN = 128;
    constexpr int Q = TM * TN;                         // MFMAs per wave per K step
    // SH: rows only 8-byte aligned (see the row layout below): 144-byte rows
    constexpr int ROWB = SH ? KT * 2 + 16 : KT * 2;    // 128-byte LDS rows
    constexpr int IB = 1024;                           // one load instruction: 8 rows (SH: 64 chunks)
    // load instructions per wave per tile (SH: a row is 9 chunks; the last
    // instruction of A may reach past row BM, into spare slot space)
    constexpr int LPTA = SH ? (BM * 9 + 255) / 256 : BM / 32, LPTB = SH ? 9 : 8;
    constexpr int SLOTA = LPTA * 4 * IB, SLOTB = LPTB * 4 * IB;    // >= rows x ROWB
    constexpr int B_BASE = NA * SLOTA;
    constexpr int RING_BYTES = NA * SLOTA + NB * SLOTB;
    constexpr int EPI_BYTES = 4 * 32 * (WTN + 8) * 4;
    constexpr int LDS_BYTES = RING_BYTES > EPI_BYTES ? RING_BYTES : EPI_BYTES;
    static_assert(SLOTA >= BM * ROWB && SLOTB >= BN * ROWB, "slots");
    static_assert(LDS_BYTES <= 160 * 1024, "ring");
    static_assert(TM == 8 || TM == 6, "wave tile");
    static_assert(!SPLIT || !OUT_BF16, "split-K partial tiles are fp32");
    static_assert(!(AT || BT) || (!SH && !SPLIT && TM == 8), "MN-contiguous operands: 16-byte rows, 256 x 256");
    static_assert(!PERSIST || (!SH && !SPLIT && !AT && !BT && TM == 8), "persistent: 16-byte rows, 256 x 256");

    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    int tmi, tni, split = 0;
    int vt = blockIdx.x;                               // PERSIST: the virtual workgroup id
    if constexpr (SPLIT)
        tile_order_split(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tmi, tni, split);
    else
        tile_order(vt, PERSIST ? p.tiles_m * p.tiles_n : (int)gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tmi, tni);
    int m0 = tmi * BM, n0 = tni * BN;
    const int k_lo = SPLIT ? split * p.kt_split * KT : 0;          // first K element of this range
    const int M = p.M, N = p.N;
    const int K = SPLIT ? (p.K - k_lo < p.kt_split * KT ? p.K - k_lo : p.kt_split * KT) : p.K;

    // Tile bases.  With SH the resources start at the 16-byte boundary at or
    // below the tile's first element (at most 8 bytes earlier, never across a
    // page boundary, since the element itself lies 8 bytes into its 16).
    // (SPLIT: k_lo is a multiple of 64 elements, 128 bytes: the alignment of
    // the rows within 16 bytes does not change)
    const char *a_tile = (const char *)p.A + (int64_t)m0 * p.lda * 2 + (int64_t)k_lo * 2;
    const char *b_tile = (const char *)p.B + (int64_t)n0 * p.ldb * 2 + (int64_t)k_lo * 2;
    const int a_mis0 = SH ? (int)((uintptr_t)a_tile & 15) : 0;
    const int b_mis0 = SH ? (int)((uintptr_t)b_tile & 15) : 0;
    __amdgpu_buffer_rsrc_t rA = make_rsrc(a_tile - a_mis0, span_bytes(M - m0, K, p.lda, 2) + a_mis0);
    __amdgpu_buffer_rsrc_t rB = make_rsrc(b_tile - b_mis0, span_bytes(N - n0, K, p.ldb, 2) + b_mis0);

    // 16-byte rows (no SH): load instruction j of a wave fills slot rows
    // (4 j + wave) * 8 + lane / 8: lane L writes physical chunk L % 8 and
    // fetches logical chunk (L % 8) ^ swz16(row) = (L % 8) ^ (L / 8), the same
    // for every j.
    // 8-byte rows (SH): row r starts s = mis0 + r * ld * 2 bytes after the
    // resource base, s % 16 = 0 or 8.  Its 64-element K tile is fetched as
    // the nine aligned 16-byte chunks from s & ~15 on, stored as a 144-byte
    // LDS row, so the tile's data starts (s % 16) bytes into the row.  Load
    // instruction j of a wave fills slot chunks (4 j + wave) * 64 + lane (row
    // chunk / 9, chunk chunk % 9), written linearly.  The 144-byte pitch
    // spreads the 16 rows of a fragment read over all banks without a swizzle.
    const int chunk = (lane & 7) ^ (lane >> 3);
    const int kel = chunk * 8;
    uint32_t a_off[LPTA], b_off[LPTB];
    auto sh_row = [&](int j) __attribute__((always_inline)) { return ((4 * j + wave) * 64 + lane) / 9; };
    auto sh_chk = [&](int j) __attribute__((always_inline)) { return ((4 * j + wave) * 64 + lane) % 9; };
    // MN-contiguous operand: load instruction j of a wave fills LDS rows
    // 2 (4 j + wave) + lane / 32 of the tile (1 KiB: two 512-byte rows);
    // lane L writes 16 bytes at physical chunk (L % 32) / 2, half L % 2, and
    // fetches the columns of the logical chunk that lands there.
    auto mn_off = [&](int64_t ld, int j) __attribute__((always_inline)) {
        const int row = 2 * (4 * j + wave) + (lane >> 5);
        const int lchk = ((lane & 31) >> 1) ^ (row & 3) ^ (((row >> 3) & 1) << 2);
        return (uint32_t)((row * ld + lchk * 16 + (lane & 1) * 8) * 2);
    };
#pragma unroll
    for (int j = 0; j < LPTA; ++j) {
        if constexpr (SH) {
            // (a row that starts on a 16-byte boundary has its 64 elements in
            // chunks 0 .. 7: its ninth chunk, never read, is not fetched --
            // an offset past the resource makes no memory request)
            const uint32_t s_ = (uint32_t)(a_mis0 + sh_row(j) * p.lda * 2);
            a_off[j] = (sh_chk(j) == 8 && (s_ & 15u) == 0) ? kOOB : (s_ & ~15u) + sh_chk(j) * 16;
        } else {
            const int row = (4 * j + wave) * 8 + (lane >> 3);
            a_off[j] = AT ? mn_off(p.lda, j) : (uint32_t)(row * p.lda * 2) + chunk * 16;
        }
    }
#pragma unroll
    for (int j = 0; j < LPTB; ++j) {
        if constexpr (SH) {
            const uint32_t s_ = (uint32_t)(b_mis0 + sh_row(j) * p.ldb * 2);
            b_off[j] = (sh_chk(j) == 8 && (s_ & 15u) == 0) ? kOOB : (s_ & ~15u) + sh_chk(j) * 16;
        } else {
            const int row = (4 * j + wave) * 8 + (lane >> 3);
            b_off[j] = BT ? mn_off(p.ldb, j) : (uint32_t)(row * p.ldb * 2) + chunk * 16;
        }
    }
    // SH: K element (relative to the tile's K offset) at which chunk c of
    // row r starts: 8 c - (s % 16) / 2, i.e. -4 for the first chunk of a
    // shifted row.
    auto sh_kel = [&](int mis0, int64_t ld, int j) __attribute__((always_inline)) {
        const int s_ = mis0 + sh_row(j) * (int)ld * 2;
        return 8 * sh_chk(j) - ((s_ & 15) >> 1);
    };
    // Loads of K tile t: whole 16-byte chunks, the K offset in the scalar
    // offset (no vector instruction per load).  The last tile reads past K
    // (into the next row, or zeros past the resource) and clear_past_k then
    // zeroes those bytes in LDS; tiles past K are read through a resource of
    // size zero, which returns zeros.
    const __amdgpu_buffer_rsrc_t rZ = make_rsrc(p.D, 0u);
    auto dma = [&](__amdgpu_buffer_rsrc_t r, char *d, uint32_t voff, int t) __attribute__((always_inline)) {
        const int k0 = t * KT;
        const __amdgpu_buffer_rsrc_t rr = k0 < K ? r : rZ;
        const int sk = __builtin_amdgcn_readfirstlane(k0 * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (__attribute__((address_space(3))) void *)d, 16, voff, sk, 0, 0);
    };
    // MN-contiguous operand, K tile t: a resource based at row 64 t, column
    // e0 of the K x (M or N) storage, ending with the 16-byte block that
    // holds the last row's last element.  (The range check is per dword: an
    // odd M or N would otherwise lose the last element of row K - 1 with the
    // dword it shares.  The base is 16-byte aligned -- aligned operand, ld
    // a multiple of 8, e0 a multiple of 256 -- so the block lies in the same
    // page as that element.)
    auto dma_mn = [&](const void *base, int64_t ld, int e0, int ext, char *d, uint32_t voff, int t)
        __attribute__((always_inline)) {
        const int k0 = t * KT;
        const uint32_t span = (span_bytes(K - k0, ext - e0, ld, 2) + 15u) & ~15u;
        const __amdgpu_buffer_rsrc_t r = make_rsrc((const char *)base + ((int64_t)k0 * ld + e0) * 2, span);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)d, 16, voff, 0, 0, 0);
    };
    auto dma_a = [&](int t, int j) __attribute__((always_inline)) {
        char *d = smem + (t % NA) * SLOTA + (j * 4 + wave) * IB;
        if constexpr (AT)
            dma_mn(p.A, p.lda, m0, M, d, a_off[j], t);
        else
            dma(rA, d, a_off[j], t);
    };
    auto dma_b = [&](int t, int j) __attribute__((always_inline)) {
        char *d = smem + B_BASE + (t % NB) * SLOTB + (j * 4 + wave) * IB;
        if constexpr (BT)
            dma_mn(p.B, p.ldb, n0, N, d, b_off[j], t);
        else
            dma(rB, d, b_off[j], t);
    };
    // Last K tile t (after this lane's loads of it landed, before the
    // barrier that publishes it): the lane zeroes what its own direct-to-LDS
    // loads brought from past K -- whole chunks past K, and with SH the
    // second half of a chunk that straddles K (K % 4 == 0, so a chunk holds
    // 0, 4 or 8 elements inside K).  MN-contiguous operands read zeros past
    // K already.
    auto clear_past_k = [&](int t) __attribute__((always_inline)) {
        const int kr = K - t * KT;                     // elements of the tile inside K
        if (kr >= KT) return;
        auto clear = [&](char *d, int inside) __attribute__((always_inline)) {
            if (inside <= 0)
                *(u32x4 *)d = u32x4{0u, 0u, 0u, 0u};
            else if (inside < 8)
                *(u32x2 *)(d + 8) = u32x2{0u, 0u};
        };
#pragma unroll
        for (int j = 0; j < LPTA; ++j) {
            if constexpr (!AT)
                clear(smem + (t % NA) * SLOTA + (j * 4 + wave) * IB + lane * 16,
                      kr - (SH ? sh_kel(a_mis0, p.lda, j) : kel));
        }
#pragma unroll
        for (int j = 0; j < LPTB; ++j) {
            if constexpr (!BT)
                clear(smem + B_BASE + (t % NB) * SLOTB + (j * 4 + wave) * IB + lane * 16,
                      kr - (SH ? sh_kel(b_mis0, p.ldb, j) : kel));
        }
        wait_lgkmcnt0();
    };

    // Fragment reads: lane l reads row l % 16 of each block and chunk
    // 4 step + l / 16 of that row.  With SH the row's data starts (s % 16)
    // bytes into its LDS row -- the same for all rows of a lane (they are 16
    // apart) -- and a chunk is read as two 8-byte halves.
    const int fr = lane & 15, fq = lane >> 4;
    const int fswz = SH ? 0 : swz16(fr);               // the same for every block (16 rows apart)
    const int a_read = (wm * WTM + fr) * ROWB + (SH ? (a_mis0 + fr * (int)p.lda * 2) & 15 : 0);
    const int b_read = (wn * WTN + fr) * ROWB + (SH ? (b_mis0 + fr * (int)p.ldb * 2) & 15 : 0);
    auto ldfrag = [&](int addr) __attribute__((always_inline)) {
        if constexpr (SH) {
            // two 8-byte reads, kept apart (volatile): merged into one
            // 16-byte read at an 8-byte-aligned address they cost far more
            typedef __attribute__((address_space(3))) volatile const u32x2 lds_u32x2;
            const u32x2 lo = *(lds_u32x2 *)(smem + addr), hi = *(lds_u32x2 *)(smem + addr + 8);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
            return *(const u32x4 *)(smem + addr);
        }
    };

    // MN-contiguous operand: lane (group q, i = lane % 16) reads, for block b
    // (columns 16 b .. 16 b + 15 of the wave's 128), rows 32 st + 8 q + 4 h +
    // i / 4 (h = 0, 1: K 8 q .. 8 q + 3 and 8 q + 4 .. 8 q + 7 of step st) at
    // columns 4 (i % 4) .. + 3.  The chunk's swizzle depends only on i / 4
    // and q % 2, so per block one lane-dependent base holds the XOR and the
    // slot, step and half go in the read's immediate offset.
    auto mn_base = [&](int wb, int b) __attribute__((always_inline)) {
        const int g = (fr >> 2) ^ ((fq & 1) << 2);
        return (8 * fq + (fr >> 2)) * 512 + (wb * 8 + (b ^ g)) * 32 + (fr & 3) * 8;
    };
    int a_mn[AT ? TM : 1], b_mn[BT ? TN : 1];
#pragma unroll
    for (int b = 0; b < (AT ? TM : 1); ++b) a_mn[b] = AT ? mn_base(wm, b) : 0;
#pragma unroll
    for (int b = 0; b < (BT ? TN : 1); ++b) b_mn[b] = BT ? B_BASE + mn_base(wn, b) : 0;
    // The transpose reads are asm: through the compiler builtin every read
    // waited for all direct-to-LDS loads in flight (the compiler cannot tell
    // it from a write into the slots being loaded), which serialised the
    // loads of tile t + 1 with the reads of tile t.  Uncounted, they make the
    // compiler's own lgkmcnt waits only stricter; their own results are
    // waited for explicitly (tr_row_wait, and lgkmcnt(0) at each window's
    // end).
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)smem;
    auto ldfrag_tr = [&](int addr) __attribute__((always_inline)) {
        u32x2 lo, hi;
        const uint32_t a = lds0 + (uint32_t)addr;
        asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(lo) : "v"(a));
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:2048" : "=v"(hi) : "v"(a));
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };

    // Accumulators in AGPRs, updated in place by volatile asm MFMAs; a
    // scheduling barrier after each keeps the issue order of the source.
    f32x4 acc[TM][TN];
    u32x4 fa[2][TM], fb[2][TN];                        // [K step][block]

    // C streamed into the accumulators (see above).
    constexpr int OS = OUT_BF16 ? 2 : 4;
    constexpr int CPARTS = TM * TN / 4;                // parts of 4 blocks
    const int nt = (K + KT - 1) / KT;
    // (whole 4-column vectors: every C row segment a lane reads is either in
    // range or past N)
    // (and the stream's tiles load only whole K tiles: see the loop below)
    constexpr bool CSTREAM = !SPLIT && !PERSIST;       // (persistent calls have no C)
    const bool c_loop = CSTREAM && p.C != nullptr && nt >= CPARTS + 2 + NB && e.vec_c && N % 4 == 0;
    const __amdgpu_buffer_rsrc_t rC =
        make_rsrc(c_loop ? (const char *)p.C + (int64_t)m0 * p.ldc * OS : (const char *)p.D,
                  c_loop ? span_bytes(M - m0, N, p.ldc, OS) : 0u);
    f32x4 cv[3][4];                                    // [set][block of the part]: 4 columns of a row
    auto load_c = [&](int part, int u) __attribute__((always_inline)) {               // block u of a part: one load
        const int b = 4 * part + u;
        const int row = wm * WTM + (b / TN) * 16 + fr;   // rows past M lie past the resource
        const int col = n0 + wn * WTN + (b % TN) * 16 + 4 * fq;
        const uint32_t off = col < N ? (uint32_t)(row * p.ldc + col) * OS : kOOB;
        if constexpr (OUT_BF16) {
            const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rC, off, 0, 0));
            cv[part % 3][u] = f32x4{__builtin_bit_cast(float, v[0] << 16), __builtin_bit_cast(float, v[0] & 0xffff0000u),
                                   __builtin_bit_cast(float, v[1] << 16), __builtin_bit_cast(float, v[1] & 0xffff0000u)};
        } else {
            cv[part % 3][u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rC, off, 0, 0));
        }
    };
    // Block u of a part += its C.  The empty tied statements pin where the
    // accumulators are read and written back: the compiler cannot see that
    // the asm MFMAs around them read and write these registers, so without
    // them it may move the write-back right in front of the next MFMA on the
    // block and break the required distance between the two.
    auto add_c = [&](int part, int u) __attribute__((always_inline)) {
        const int b = 4 * part + u;
        f32x4 &a = acc[b / TN][b % TN];
        asm volatile("" : "+a"(a));
        f32x4 t = a;
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] += cv[part % 3][u][r];
        asm volatile("" : "+a"(t));
        a = t;
    };

    // Fragment read k of K step st of tile t: k = 0 is A block 0, k = 1..TN
    // B blocks 0..TN-1, then A blocks 1..TM-1 -- the order the MFMAs use them.
    auto read_frag = [&](int t, int st, int k) __attribute__((always_inline)) {
        const int coff = ((4 * st + fq) ^ fswz) << 4;
        if (k == 0 || k > TN) {
            const int i = k == 0 ? 0 : k - TN;
            if constexpr (AT)
                fa[st][i] = ldfrag_tr(a_mn[i] + (t % NA) * SLOTA + st * 32 * 512);
            else
                fa[st][i] = ldfrag((t % NA) * SLOTA + a_read + i * 16 * ROWB + coff);
        } else {
            const int j = k - 1;
            if constexpr (BT)
                fb[st][j] = ldfrag_tr(b_mn[j] + (t % NB) * SLOTB + st * 32 * 512);
            else
                fb[st][j] = ldfrag(B_BASE + (t % NB) * SLOTB + b_read + j * 16 * ROWB + coff);
        }
    };
    // B is the MFMA's first operand and A its second, so block (i, j) holds
    // the transpose of the D block: lane l has row 16 i + l % 16 of the
    // quadrant and its four consecutive columns 16 j + 4 (l / 16) .. + 3.
    auto mfma = [&](auto zero, int st, int i, int j) __attribute__((always_inline)) {
        if constexpr (decltype(zero)::value)
            mfma16_zero_asm<FP16>(acc[i][j], fb[st][j], fa[st][i]);
        else
            mfma16_acc_asm<FP16>(acc[i][j], fb[st][j], fa[st][i]);
        __builtin_amdgcn_sched_barrier(0);
    };
    // One tile; FIRST: no previous tile (no deferred MFMAs, accumulators
    // start from zero).  LP: the C part this tile loads (-1: none); AP: the
    // C part it adds (-1: none); SO: the K tiles it loads are whole.
    auto tile = [&](auto first, auto lp, auto ap, int t) __attribute__((always_inline)) {
        constexpr int LP = decltype(lp)::value, AP = decltype(ap)::value;
        // The whole step 1 of tile t-1 runs after barrier t while step 0 of
        // tile t is read (TM + TN reads spread evenly) and A(t+1), B(t+1)
        // are loaded (also spread), then step 0 of tile t while step 1 is
        // read (one per 3 MFMAs).  Block b gets its C at slot (b + Q/2) % Q
        // of the first half, Q/2 MFMAs from its updates on either side.
        // (issue slots: read k at MFMA k Q / (TM + TN); SH: loads j of A and B
        // at 7 j Q / 64 + 1 and + 4, 16 loads of 9 over 64 MFMAs; else A load
        // j at j Q / LPTA + 2, B load j at j Q / LPTB + Q / (2 LPTB) + 2)
        constexpr int RD = TM + TN;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            if constexpr (!decltype(first)::value) mfma(std::false_type(), 1, q / TN, q % TN);
            const int kr = (q * RD + Q - 1) / Q;
            if (kr < RD && kr * Q / RD == q) read_frag(t, 0, kr);
            if constexpr (SH) {
                const int ja = (64 * (q - 1) + 7 * Q - 1) / (7 * Q), jb = (64 * (q - 4) + 7 * Q - 1) / (7 * Q);
                if (q >= 1 && ja < LPTA && 7 * ja * Q / 64 + 1 == q) dma_a(t + 1, ja);
                if (q >= 4 && jb < LPTB && 7 * jb * Q / 64 + 4 == q) dma_b(t + 1, jb);
            } else {
                const int ja = ((q - 2) * LPTA + Q - 1) / Q, ob = Q / LPTB / 2 + 2;
                const int jb = ((q - ob) * LPTB + Q - 1) / Q;
                if (q >= 2 && ja < LPTA && ja * Q / LPTA + 2 == q) dma_a(t + 1, ja);
                if (q >= ob && jb < LPTB && jb * Q / LPTB + ob == q) dma_b(t + 1, jb);
            }
            if constexpr (AP >= 0) {
                constexpr int s0 = (4 * AP + Q / 2) % Q;
                if (q >= s0 && q < s0 + 4) add_c(AP, q - s0);
            }
        }
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            if constexpr (AT || BT) {
                constexpr int CA = AT ? 2 : 1, CB = BT ? 2 : 1;
                if (q % TN == 0) {
                    switch (q / TN) {
#define TG_TR_WAIT(i) \
    case i: __builtin_amdgcn_s_waitcnt(0xC07F | (tr_row_wait<CA, CB>(i) << 8)); break;
                        TG_TR_WAIT(0) TG_TR_WAIT(1) TG_TR_WAIT(2) TG_TR_WAIT(3)
                        TG_TR_WAIT(4) TG_TR_WAIT(5) TG_TR_WAIT(6) TG_TR_WAIT(7)
#undef TG_TR_WAIT
                    }
                }
            }
            mfma(first, 0, q / TN, q % TN);
            if (q % 3 == 0 && q / 3 < TM + TN) read_frag(t, 1, q / 3);
            if constexpr (LP >= 0) {
                const int u = (q - 6) * 4 / Q;
                if (q >= 6 && u < 4 && u * Q / 4 + 6 == q) load_c(LP, u);
            }
        }
        // A(t+1), B(t+1) landed; this tile's C loads (one per block of the
        // part) may still run
        wait_vmcnt<(LP >= 0 ? 4 : 0)>();
        wait_lgkmcnt0();
        if (t + 1 == nt - 1) clear_past_k(t + 1);
        barrier();
    };
    // tiles 1 .. CPARTS + 1 of the C stream, unrolled: tile t loads part t
    // (while t < CPARTS) and adds part t - 2 (from tile 2 on)
    auto c_tiles = [&](auto self, auto tc) __attribute__((always_inline)) {
        constexpr int T = decltype(tc)::value;
        if constexpr (T <= CPARTS + 1) {
            tile(std::false_type(), std::integral_constant<int, (T < CPARTS ? T : -1)>(),
                 std::integral_constant<int, T - 2>(), T);
            self(self, std::integral_constant<int, T + 1>());
        }
    };

    // PERSIST: the next tile's A(0), B(0), with the wave index passed
    // through an empty asm so that these loads' LDS destinations are
    // computed here, not held through the main loop
    auto next_tile_loads = [&]() __attribute__((always_inline)) {
        int wv = wave;
        asm volatile("" : "+s"(wv));
#pragma unroll
        for (int j = 0; j < LPTA; ++j) dma(rA, smem + (j * 4 + wv) * IB, a_off[j], 0);
#pragma unroll
        for (int j = 0; j < LPTB; ++j) dma(rB, smem + B_BASE + (j * 4 + wv) * IB, b_off[j], 0);
    };
    // PERSIST: this wave's D staging area, in the slots K tile 0 does not use
    float *stage = (float *)(smem + (wave < 2 ? SLOTA : B_BASE + SLOTB) + (wave & 1) * 16 * (WTN + 4) * 4);
    static_assert(!PERSIST || 2 * 16 * (WTN + 4) * 4 <= SLOTA, "staging areas");
    constexpr int D_STORES = (WTM / 16) * (16 * WTN / 4 / 64);

    if (nt > 0) {
        // A(0), B(0): the loads the first tile's iteration does not issue
#pragma unroll
        for (int j = 0; j < LPTA; ++j) dma_a(0, j);
#pragma unroll
        for (int j = 0; j < LPTB; ++j) dma_b(0, j);
        wait_vmcnt<0>();                               // A(0), B(0) landed
        if (nt == 1) clear_past_k(0);
        barrier();
    }
    while (true) {
        if (nt > 0) {
            using none = std::integral_constant<int, -1>;
            using yes = std::true_type;
            using no = std::false_type;
            int t0 = 1;
            if constexpr (CSTREAM) {
                if (c_loop) {
                    tile(yes(), std::integral_constant<int, 0>(), none(), 0);   // loads C part 0
                    c_tiles(c_tiles, std::integral_constant<int, 1>());         // tiles 1 .. CPARTS + 1
                    t0 = CPARTS + 2;
                } else {
                    tile(yes(), none(), none(), 0);
                }
            } else {
                tile(yes(), none(), none(), 0);
            }
            for (int t = t0; t < nt; ++t) tile(no(), none(), none(), t);
            // the deferred part of the last tile's step 1
#pragma unroll
            for (int q = 0; q < Q; ++q) mfma(std::false_type(), 1, q / TN, q % TN);
            mfma_result_fence<TM, TN>(acc);
        } else {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }

        wait_vmcnt<0>();
        wait_lgkmcnt0();
        barrier();
        if constexpr (SPLIT) {
            // partial tiles stay cacheable: the reduction reads them right after
            float *part = p.ws + (int64_t)split * M * p.ldw;
            epilogue_lds16t<false, TM, TN, WTM, WTN, 0>(acc, smem, wave, lane, wm, wn, m0, n0, M, N, nullptr, 0, part,
                                                        p.ldw, e);
            break;
        } else if constexpr (!PERSIST) {
            epilogue_lds16t<OUT_BF16, TM, TN, WTM, WTN, DAUX>(acc, smem, wave, lane, wm, wn, m0, n0, M, N,
                                                              c_loop ? nullptr : p.C, p.ldc, p.D, p.ldd, e);
            break;
        } else {
            const F16Args r = kernel_arg0_reloaded<F16Args>();
            const int dm0 = m0, dn0 = n0;              // the finished tile
            const int ntl = r.tiles_m * r.tiles_n;
            vt += gridDim.x;
            const bool more = vt < ntl;
            if (more) {
                tile_order(vt, ntl, r.tiles_m, r.tiles_n, r.group_m, tmi, tni);
                m0 = tmi * BM;
                n0 = tni * BN;
                rA = make_rsrc((const char *)r.A + (int64_t)m0 * r.lda * 2, span_bytes(r.M - m0, K, r.lda, 2));
                rB = make_rsrc((const char *)r.B + (int64_t)n0 * r.ldb * 2, span_bytes(r.N - n0, K, r.ldb, 2));
                if (nt > 0) next_tile_loads();
            }
            epilogue_rows16_vec<OUT_BF16, TM, TN, DAUX, true>(acc, stage, lane, wm, wn, dm0, dn0, r.M, r.N, r.D,
                                                              r.ldd);
            if (!more) break;
            // the next tile's first loads landed; up to 63 of the D stores issued after them may still run
            static_assert(D_STORES >= 63, "vmcnt");
            wait_vmcnt<63>();
            wait_lgkmcnt0();
            if (nt == 1) clear_past_k(0);
            barrier();                                 // staging reads done before tile 0 refills those slots
        }
    }
}

}  // namespace tg
