// Four-wave schedule for D = A.B + C with 16-bit inputs whose rows are
// 16-byte aligned (K a multiple of 8), gfx950.
//
// The workgroup computes a 256 x 256 output tile with 4 waves, one per SIMD,
// each owning a 128 x 128 quadrant as 8 x 8 blocks of 16 x 16 accumulators
// (v_mfma_f32_16x16x32: 256 accumulator registers per lane).  Large wave
// tiles keep LDS traffic low: per 32-wide K slab each wave reads 16 KiB of
// fragments (64 KiB for the workgroup) against 32 KiB of tile data written
// by the direct global->LDS loads, and the 16x16 MFMA form draws less power
// per flop than 32x32, so the clock holds higher under load.
//
// K advances in slabs of 32 (one MFMA step).  A and B each have a ring of NS
// LDS slots of 256 rows x 64 bytes.  In iteration s a wave
//   - issues the 64 MFMAs of slab s from fragments already in registers,
//   - reads slab s + 1's fragments into the other register buffer,
//   - issues its quarter of the global->LDS loads of slab s + NS into the
//     slot slab s used (every wave finished reading it before the barrier
//     that opened iteration s),
// then waits until its own loads of slab s + 2 have landed and joins the
// barrier that opens iteration s + 1.  A slab's loads thus have NS - 1
// iterations to land.  Loads past K read nothing (out-of-range offsets give
// zeros) so the wait counts stay fixed to the end.
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

// 64-byte LDS rows (four 16-byte chunks): logical chunk c of row r sits at
// physical chunk c ^ ((r >> 2) & 3).  A 16x16x32 fragment read has each
// group of 16 lanes read one chunk of 16 consecutive rows; rows r and r + 4
// share banks, and the swizzle gives those four rows four different chunks,
// so every 16-lane (and 8-lane) group hits distinct banks.
__device__ __forceinline__ int swz64(int r) { return (r >> 2) & 3; }

template <int NS, bool FP16, bool OUT_BF16>
__global__ void __launch_bounds__(256) gemm_f16_w4_kernel(F16Args p, F16Epi e) {
    constexpr int BM = 256, BN = 256, KS = 32;         // tile and K slab
    constexpr int WTM = 128, WTN = 128, TM = 8, TN = 8;
    constexpr int ROWB = KS * 2;                       // 64-byte LDS rows
    constexpr int SLOT = 256 * ROWB;                   // 16 KiB per operand slot
    constexpr int B_BASE = NS * SLOT;
    constexpr int RING_BYTES = 2 * NS * SLOT;
    constexpr int EPI_BYTES = 4 * 32 * (WTN + 8) * 4;
    constexpr int LDS_BYTES = RING_BYTES > EPI_BYTES ? RING_BYTES : EPI_BYTES;
    constexpr int IB = 1024;                           // one load instruction: 16 rows
    constexpr int LPS = 4;                             // load instructions per wave per operand per slab
    constexpr int WAIT_N = (NS - 2) * 2 * LPS;         // loads still in flight at a barrier
    static_assert(NS >= 3 && LDS_BYTES <= 160 * 1024 && WAIT_N < 64, "ring");

    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    int tmi, tni;
    tile_order(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tmi, tni);
    const int m0 = tmi * BM, n0 = tni * BN;
    const int M = p.M, N = p.N, K = p.K;

    const __amdgpu_buffer_rsrc_t rA =
        make_rsrc((const char *)p.A + (int64_t)m0 * p.lda * 2, span_bytes(M - m0, K, p.lda, 2));
    const __amdgpu_buffer_rsrc_t rB =
        make_rsrc((const char *)p.B + (int64_t)n0 * p.ldb * 2, span_bytes(N - n0, K, p.ldb, 2));

    // Load instruction j of a wave fills slot rows (4 j + wave) * 16 + lane / 4:
    // lane L writes physical chunk L % 4 and fetches logical chunk
    // (L % 4) ^ swz64(row) = (L % 4) ^ ((L / 16) % 4), the same for every j.
    const int chunk = (lane & 3) ^ ((lane >> 4) & 3);
    const int kel = chunk * 8;
    uint32_t a_off[LPS], b_off[LPS];
#pragma unroll
    for (int j = 0; j < LPS; ++j) {
        const int row = (4 * j + wave) * 16 + (lane >> 2);
        a_off[j] = (uint32_t)(row * p.lda * 2) + chunk * 16;
        b_off[j] = (uint32_t)(row * p.ldb * 2) + chunk * 16;
    }
    // Load k (0..7) of this wave for slab sl: k < 4 is A instruction k, else B.
    auto dma = [&](int sl, int k) {
        const int k0 = sl * KS;
        const uint32_t oob = (uint32_t)(k0 + kel >= K) << 31;   // offsets stay below 2^31
        char *d = smem + (sl % NS) * SLOT + (k >= LPS ? B_BASE : 0) + ((k % LPS) * 4 + wave) * IB;
        const uint32_t off = ((k < LPS ? a_off[k % LPS] : b_off[k % LPS]) + (uint32_t)k0 * 2) | oob;
        dma_load<16>(k < LPS ? rA : rB, d, off);
    };

    // Fragment reads: lane l reads row l % 16 of each block, chunk l / 16.
    const int fr = lane & 15, fq = lane >> 4;
    const int coff = (fq ^ swz64(fr)) << 4;            // the same for every block (16 rows apart)
    const int a_read = (wm * WTM + fr) * ROWB + coff;
    const int b_read = B_BASE + (wn * WTN + fr) * ROWB + coff;

    // The accumulators live in AGPRs and every MFMA updates its block in
    // place (tied asm operand), so the register allocator never moves them.
    // The asm is volatile and a scheduling barrier follows each MFMA, so
    // MFMAs, LDS reads, global->LDS loads and their address arithmetic issue
    // in source order: nothing is hoisted in front of a slab's first MFMA.
    f32x4 acc[TM][TN];
    u32x4 fa[2][TM], fb[2][TN];
    auto read_frag = [&](int buf, int sl, int k) {     // k < 8: A block k, else B block k - 8
        const char *s0 = smem + (sl % NS) * SLOT;
        if (k < TM)
            fa[buf][k] = *(const u32x4 *)(s0 + a_read + k * 16 * ROWB);
        else
            fb[buf][k - TM] = *(const u32x4 *)(s0 + b_read + (k - TM) * 16 * ROWB);
    };
    auto slab_end = [&]() {
        wait_vmcnt<WAIT_N>();
        wait_lgkmcnt0();
        barrier();
    };
    // Slab sl: its 64 MFMAs on fragment buffer buf; after every second of the
    // first 32 MFMAs one fragment read of slab sl + 1 into buf ^ 1, and after
    // every fourth of MFMAs 28..56 one load of slab sl + NS.  FIRST: the
    // accumulators start from zero (the MFMA's C operand is the constant 0).
    auto iteration = [&](auto first, int buf, int sl) {
#pragma unroll
        for (int q = 0; q < TM * TN; ++q) {
            const int i = q / TN, j = q % TN;
            if constexpr (decltype(first)::value)
                mfma16_zero_asm<FP16>(acc[i][j], fa[buf][i], fb[buf][j]);
            else
                mfma16_acc_asm<FP16>(acc[i][j], fa[buf][i], fb[buf][j]);
            __builtin_amdgcn_sched_barrier(0);
            if (q % 2 == 1 && q / 2 < TM + TN) read_frag(buf ^ 1, sl + 1, q / 2);
            if (q >= 28 && q % 4 == 0 && (q - 28) / 4 < 2 * LPS) dma(sl + NS, (q - 28) / 4);
        }
        slab_end();
    };

    const int ns = (K + KS - 1) / KS;
    if (ns > 0) {
#pragma unroll
        for (int q = 0; q < NS; ++q)                   // slabs 0 .. NS-1
#pragma unroll
            for (int k = 0; k < 2 * LPS; ++k) dma(q, k);
        wait_vmcnt<(NS - 1) * 2 * LPS>();              // slab 0 landed
        barrier();
#pragma unroll
        for (int k = 0; k < TM + TN; ++k) read_frag(0, 0, k);
        slab_end();                                    // slab 1 landed, slab 0 fragments in registers
        iteration(std::true_type(), 0, 0);
        // Slabs in pairs: with ns even the last pass multiplies the all-zero
        // slab ns (loaded out of range) and adds nothing.
        for (int s = 1; s < ns; s += 2) {
            iteration(std::false_type(), 1, s);
            iteration(std::false_type(), 0, s + 1);
        }
        // The epilogue reads the accumulators with VALU instructions; the
        // compiler cannot see that they were last written by MFMAs, so wait
        // out that hazard here, ahead of every accumulator use.
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
    epilogue_lds16<OUT_BF16, TM, TN, WTM, WTN>(acc, smem, wave, lane, wm, wn, m0, n0, M, N, p.C, p.ldc, p.D, p.ldd, e);
}


// The same four-wave, 128 x 128-per-wave layout with 64-wide K tiles:
// 128-byte LDS rows, so every global->LDS load instruction moves whole
// 128-byte lines (8 rows of a tile), and rings of NA slots for A and NB for
// B (32 KiB a slot).  Per tile a wave issues 128 MFMAs in two K steps of
// 32.  Half of the second step's MFMAs are issued after the barrier that
// opens the next tile, while that tile's first fragments are read, so the
// matrix pipe does not drain at the barrier:
//   after barrier t:  MFMAs of tile t-1 step 1 (blocks i = 4..7)
//                     + fragment reads of tile t step 0 + loads of A(t+NA-1)
//                     MFMAs of tile t step 0
//                     + fragment reads of tile t step 1 + loads of B(t+NB-1)
//                     MFMAs of tile t step 1 (blocks i = 0..3)
//                     wait for A(t+1), B(t+1); barrier t+1
// A tile's slots are read only between its own two barriers, so the loads
// of A(t+NA-1) and B(t+NB-1) go to slots freed at barrier t; A has one
// tile of time to land, B (with NB = NA + 1) two.
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

template <int NA, int NB, bool FP16, bool OUT_BF16, int SCHED = 0, int DAUX = kStoreStream, bool SH = false,
          bool SPLIT = false, bool AT = false, bool BT = false>
__global__ void __launch_bounds__(256) gemm_f16_w4t_kernel(F16Args p, F16Epi e) {
    constexpr int BM = 256, BN = 256, KT = 64;         // tile
    constexpr int WTM = 128, WTN = 128, TM = 8, TN = 8;
    // SH: rows only 8-byte aligned (see the row layout below): 144-byte rows
    constexpr int ROWB = SH ? KT * 2 + 16 : KT * 2;    // 128-byte LDS rows
    constexpr int SLOT = 256 * ROWB;                   // 32 KiB per operand slot (36 KiB with SH)
    constexpr int B_BASE = NA * SLOT;
    constexpr int RING_BYTES = (NA + NB) * SLOT;
    constexpr int EPI_BYTES = 4 * 32 * (WTN + 8) * 4;
    constexpr int LDS_BYTES = RING_BYTES > EPI_BYTES ? RING_BYTES : EPI_BYTES;
    constexpr int IB = 1024;                           // one load instruction: 8 rows
    constexpr int LPT = SH ? 9 : 8;                    // load instructions per wave per operand per tile
    constexpr int WAIT_N = (NB - NA) * LPT;            // B loads still in flight at a barrier
    static_assert(NA == 2 && (NB == 2 || NB == 3) && LDS_BYTES <= 160 * 1024, "ring");
    static_assert(!SH || (NB == 2 && SCHED == 1), "shifted rows: balanced schedule, two B slots");
    static_assert(!SPLIT || !OUT_BF16, "split-K partial tiles are fp32");
    static_assert(!(AT || BT) || (!SH && !SPLIT && SCHED == 1 && NB == 2), "MN-contiguous operands: 16-byte rows");

    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    int tmi, tni, split = 0;
    if constexpr (SPLIT)
        tile_order_split(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tmi, tni, split);
    else
        tile_order(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tmi, tni);
    const int m0 = tmi * BM, n0 = tni * BN;
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
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(a_tile - a_mis0, span_bytes(M - m0, K, p.lda, 2) + a_mis0);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(b_tile - b_mis0, span_bytes(N - n0, K, p.ldb, 2) + b_mis0);

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
    uint32_t a_off[LPT], b_off[LPT];
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
    for (int j = 0; j < LPT; ++j) {
        if constexpr (SH) {
            const int row = sh_row(j), c = sh_chk(j);
            a_off[j] = ((uint32_t)(a_mis0 + row * p.lda * 2) & ~15u) + c * 16;
            b_off[j] = ((uint32_t)(b_mis0 + row * p.ldb * 2) & ~15u) + c * 16;
        } else {
            const int row = (4 * j + wave) * 8 + (lane >> 3);
            a_off[j] = AT ? mn_off(p.lda, j) : (uint32_t)(row * p.lda * 2) + chunk * 16;
            b_off[j] = BT ? mn_off(p.ldb, j) : (uint32_t)(row * p.ldb * 2) + chunk * 16;
        }
    }
    // SH: K element (relative to the tile's K offset) at which chunk c of
    // row r starts: 8 c - (s % 16) / 2, i.e. -4 for the first chunk of a
    // shifted row.  A chunk reaching past K is read as zeros (a partly
    // out-of-range load is never issued); if its first half is valid, the
    // ragged tile's fix-up writes that half afterwards.
    auto sh_kel = [&](int mis0, int64_t ld, int j) __attribute__((always_inline)) {
        const int s_ = mis0 + sh_row(j) * (int)ld * 2;
        return 8 * sh_chk(j) - ((s_ & 15) >> 1);
    };
    // Loads of K tile t.  SO: the tile is wholly inside K or wholly past it,
    // so the K offset is uniform and goes in the scalar offset (bit 31 set
    // past K: every lane reads zeros) and no vector instruction is spent per
    // load; otherwise (the tile holding a ragged end of K) each lane adds the
    // K offset and sets bit 31 itself when its chunk lies past K.
    auto dma = [&](auto so, __amdgpu_buffer_rsrc_t r, char *d, uint32_t voff, int t, int kelj) __attribute__((always_inline)) {
        const int k0 = t * KT;
        if constexpr (decltype(so)::value) {
            const int sk = __builtin_amdgcn_readfirstlane((k0 * 2) | ((int)(k0 >= K) << 31));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)d, 16, voff, sk, 0, 0);
        } else {
            const uint32_t oob = (uint32_t)(SH ? k0 + kelj + 8 > K : k0 + kelj >= K) << 31;   // offsets stay below 2^31
            const uint32_t off = (voff + (uint32_t)k0 * 2) | oob;
            dma_load<16>(r, d, off);
        }
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
    auto dma_a = [&](auto so, int t, int j) __attribute__((always_inline)) {
        char *d = smem + (t % NA) * SLOT + (j * 4 + wave) * IB;
        if constexpr (AT) {
            dma_mn(p.A, p.lda, m0, M, d, a_off[j], t);
        } else {
            const int kelj = SH ? sh_kel(a_mis0, p.lda, j) : kel;
            dma(so, rA, d, a_off[j], t, kelj);
        }
    };
    auto dma_b = [&](auto so, int t, int j) __attribute__((always_inline)) {
        char *d = smem + B_BASE + (t % NB) * SLOT + (j * 4 + wave) * IB;
        if constexpr (BT) {
            dma_mn(p.B, p.ldb, n0, N, d, b_off[j], t);
        } else {
            const int kelj = SH ? sh_kel(b_mis0, p.ldb, j) : kel;
            dma(so, rB, d, b_off[j], t, kelj);
        }
    };
    // SH, last K tile nt - 1 (after its loads landed, before the barrier
    // that publishes it): each chunk whose first half is inside K and second
    // half past it was read as zeros; load its valid 8 bytes with an in-range
    // 8-byte load and write them into the chunk's first half.  Such chunks
    // exist whether or not K is a multiple of 64 (the ninth chunk of a row
    // shifted by 8 bytes ends 4 elements past its tile).
    auto sh_fixup = [&](int t) __attribute__((always_inline)) {
        const int k0 = t * KT;
        u32x2 v[2 * LPT];
#pragma unroll
        for (int j = 0; j < 2 * LPT; ++j) {
            const bool isb = j >= LPT;
            const int jj = isb ? j - LPT : j;
            const int kelj = isb ? sh_kel(b_mis0, p.ldb, jj) : sh_kel(a_mis0, p.lda, jj);
            const bool half = kelj >= 0 && k0 + kelj + 4 <= K && k0 + kelj + 8 > K;
            const uint32_t off = half ? (isb ? b_off[jj] : a_off[jj]) + (uint32_t)k0 * 2 : kOOB;
            v[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(isb ? rB : rA, off, 0, 0));
        }
        wait_vmcnt<0>();
#pragma unroll
        for (int j = 0; j < 2 * LPT; ++j) {
            const bool isb = j >= LPT;
            const int jj = isb ? j - LPT : j;
            const int kelj = isb ? sh_kel(b_mis0, p.ldb, jj) : sh_kel(a_mis0, p.lda, jj);
            const bool half = kelj >= 0 && k0 + kelj + 4 <= K && k0 + kelj + 8 > K;
            char *d = smem + (isb ? B_BASE + (t % NB) * SLOT : (t % NA) * SLOT) + (jj * 4 + wave) * IB + lane * 16;
            if (half) *(u32x2 *)d = v[j];
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
    constexpr int CPARTS = TM * TN / 4;                // 16 parts of 4 blocks
    const int nt = (K + KT - 1) / KT;
    // (whole 4-column vectors: every C row segment a lane reads is either in
    // range or past N)
    // (and the stream's tiles load only whole K tiles: see the loop below)
    const bool c_loop = !SPLIT && p.C != nullptr && nt >= CPARTS + 2 + NB && e.vec_c && N % 4 == 0;
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

    // Fragment read k of K step st of tile t: k = 0 is A block 0, k = 1..8
    // B blocks 0..7, k = 9..15 A blocks 1..7 -- the order the MFMAs use them.
    auto read_frag = [&](int t, int st, int k) __attribute__((always_inline)) {
        const int coff = ((4 * st + fq) ^ fswz) << 4;
        if (k == 0 || k >= 9) {
            const int i = k == 0 ? 0 : k - 8;
            if constexpr (AT)
                fa[st][i] = ldfrag_tr(a_mn[i] + (t % NA) * SLOT + st * 32 * 512);
            else
                fa[st][i] = ldfrag((t % NA) * SLOT + a_read + i * 16 * ROWB + coff);
        } else {
            const int j = k - 1;
            if constexpr (BT)
                fb[st][j] = ldfrag_tr(b_mn[j] + (t % NB) * SLOT + st * 32 * 512);
            else
                fb[st][j] = ldfrag(B_BASE + (t % NB) * SLOT + b_read + j * 16 * ROWB + coff);
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
    auto tile = [&](auto first, auto lp, auto ap, auto so, int t) __attribute__((always_inline)) {
        constexpr int LP = decltype(lp)::value, AP = decltype(ap)::value;
        if constexpr (SCHED == 1) {
            // Balanced: the whole step 1 of tile t-1 runs after barrier t
            // while step 0 of tile t is read (one read per 4 MFMAs), then
            // step 0 of tile t while step 1 is read (one per 3).  NB = 2: A
            // and B of tile t+1 load in the first half (one per 4 MFMAs);
            // NB = 3: A(t+1) in the first half, B(t+2) and C in the second.
            // Block b gets its C at slot (b + 32) % 64 of the first half,
            // 32 MFMAs from its updates on either side.
#pragma unroll
            for (int q = 0; q < 64; ++q) {
                if constexpr (!decltype(first)::value) mfma(std::false_type(), 1, q / TN, q % TN);
                if (q % 4 == 0) read_frag(t, 0, q / 4);
                if constexpr (SH) {
                    if (q % 7 == 1 && q / 7 < LPT) dma_a(so, t + 1, q / 7);
                    if (q % 7 == 4 && q / 7 < LPT) dma_b(so, t + 1, q / 7);
                } else if constexpr (NB == 3) {
                    if (q % 8 == 2) dma_a(so, t + 1, q / 8);
                } else {
                    if (q % 8 == 2) dma_a(so, t + 1, q / 8);
                    if (q % 8 == 6) dma_b(so, t + 1, q / 8);
                }
                if constexpr (AP >= 0) {
                    constexpr int s0 = (4 * AP + 32) % 64;
                    if (q >= s0 && q < s0 + 4) add_c(AP, q - s0);
                }
            }
#pragma unroll
            for (int q = 0; q < 64; ++q) {
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
                if (q % 3 == 0 && q / 3 < 16) read_frag(t, 1, q / 3);
                if constexpr (NB == 3) {
                    if (q % 8 == 2) dma_b(so, t + 2, q / 8);
                }
                if constexpr (LP >= 0) {
                    if (q % 16 == 6) load_c(LP, q / 16);
                }
            }
            wait_vmcnt<WAIT_N + (LP >= 0 ? 4 : 0)>();
            wait_lgkmcnt0();
            if constexpr (SH && !decltype(so)::value) {
                if (t + 1 == nt - 1) sh_fixup(t + 1);
            }
            barrier();
            return;
        }
        // step 1 of tile t-1, blocks i = 4..7, with tile t step 0 reads and A loads
#pragma unroll
        for (int q = 0; q < 32; ++q) {
            if constexpr (!decltype(first)::value) mfma(std::false_type(), 1, 4 + q / TN, q % TN);
            if (q % 2 == 0) read_frag(t, 0, q / 2);
            if (q % 4 == 1) dma_a(so, t + NA - 1, q / 4);
            if constexpr (AP >= 0 && AP < CPARTS / 2) {
                if (q >= 16 && q < 20) add_c(AP, q - 16);       // blocks of rows 0..63
            }
        }
        // step 0 of tile t, with step 1 reads (first half) and B loads (second half)
#pragma unroll
        for (int q = 0; q < 64; ++q) {
            mfma(first, 0, q / TN, q % TN);
            if (q % 2 == 1 && q < 32) read_frag(t, 1, q / 2);
            if (q % 4 == 1 && q >= 32) dma_b(so, t + NB - 1, (q - 32) / 4);
            if constexpr (AP >= CPARTS / 2) {
                if (q >= 16 && q < 20) add_c(AP, q - 16);       // blocks of rows 64..127
            }
        }
        // step 1 of tile t, blocks i = 0..3, with the loads of C part LP
#pragma unroll
        for (int q = 0; q < 32; ++q) {
            mfma(std::false_type(), 1, q / TN, q % TN);
            if constexpr (LP >= 0) {
                if (q % 8 == 1) load_c(LP, q / 8);
            }
        }
        // A(t+1), B(t+1) landed; B(t+NB-1) and this tile's C loads (one per
        // block of the part) may still run
        wait_vmcnt<WAIT_N + (LP >= 0 ? 4 : 0)>();
        wait_lgkmcnt0();
        barrier();
    };
    // tiles 1 .. CPARTS + 1 of the C stream, unrolled: tile t loads part t
    // (while t < CPARTS) and adds part t - 2 (from tile 2 on)
    auto c_tiles = [&](auto self, auto tc) __attribute__((always_inline)) {
        constexpr int T = decltype(tc)::value;
        if constexpr (T <= CPARTS + 1) {
            tile(std::false_type(), std::integral_constant<int, (T < CPARTS ? T : -1)>(),
                 std::integral_constant<int, T - 2>(), std::true_type(), T);
            self(self, std::integral_constant<int, T + 1>());
        }
    };

    if (nt > 0) {
        // A(0); B(0) .. B(NB-2): the loads the first tiles' iterations do not issue
#pragma unroll
        for (int j = 0; j < LPT; ++j) dma_a(std::false_type(), 0, j);
#pragma unroll
        for (int b = 0; b < NB - 1; ++b)
#pragma unroll
            for (int j = 0; j < LPT; ++j) dma_b(std::false_type(), b, j);
        wait_vmcnt<(NB - 2) * LPT>();                  // A(0), B(0) landed
        if constexpr (SH) {
            if (nt == 1) sh_fixup(0);
        }
        barrier();
        using none = std::integral_constant<int, -1>;
        using yes = std::true_type;
        using no = std::false_type;
        // Tile t loads K tiles up to t + NB - 1; only the last K tile can be
        // ragged, so tiles 0 .. nt - NB - 1 take scalar-offset loads and the
        // last NB tiles the per-lane form.
        if (nt > NB) {
            int t0 = 1;
            if (c_loop) {
                tile(yes(), std::integral_constant<int, 0>(), none(), yes(), 0);   // loads C part 0
                c_tiles(c_tiles, std::integral_constant<int, 1>());               // tiles 1 .. CPARTS + 1
                t0 = CPARTS + 2;
            } else {
                tile(yes(), none(), none(), yes(), 0);
            }
            for (int t = t0; t < nt - NB; ++t) tile(no(), none(), none(), yes(), t);
            for (int t = nt - NB; t < nt; ++t) tile(no(), none(), none(), no(), t);
        } else {
            tile(yes(), none(), none(), no(), 0);
            for (int t = 1; t < nt; ++t) tile(no(), none(), none(), no(), t);
        }
        // the deferred part of the last tile's step 1
        if constexpr (SCHED == 1) {
#pragma unroll
            for (int q = 0; q < 64; ++q) mfma(std::false_type(), 1, q / TN, q % TN);
        } else {
#pragma unroll
            for (int q = 0; q < 32; ++q) mfma(std::false_type(), 1, 4 + q / TN, q % TN);
        }
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
    } else {
        epilogue_lds16t<OUT_BF16, TM, TN, WTM, WTN, DAUX>(acc, smem, wave, lane, wm, wn, m0, n0, M, N,
                                                          c_loop ? nullptr : p.C, p.ldc, p.D, p.ldd, e);
    }
}

}  // namespace tg
