// Block-scaled fp8 D = A.B + C with four waves and
// v_mfma_scale_f32_16x16x128_f8f6f4, gfx950 (K a multiple of 512).
//
// The workgroup computes a 256 x 256 output tile with 4 waves, one per SIMD,
// each owning a 128 x 128 quadrant as 8 x 8 blocks of 16 x 16 fp32
// accumulators in AGPRs.  Against the eight-wave ping-pong layout (128 x 64
// per wave) this reads a third less fragment data from LDS per K tile: per
// 128-wide K tile a wave reads 32 KiB (A and B rows of its quadrant), the
// workgroup 128 KiB, next to the 64 KiB the direct global->LDS loads write.
//
// Operand placement of the 16x16x128 MFMA (measured with one-hot operands
// and distinct per-lane scales): lane l supplies row (A) or column (B)
// l % 16; its bytes 0..15 are K elements [16 q, 16 q + 16) and bytes 16..31
// are [64 + 16 q, 64 + 16 q + 16) of the 128-wide K tile, q = l / 16; the
// 32-wide K block b of row r takes its scale from lane 16 b + r.  So lane l
// reads 16-byte chunks q and 4 + q of its row and the scale byte of (its
// row, K block q); four blocks' scale bytes share a register, the MFMA's
// op_sel picks the byte.
//
// LDS: A and B rings of two 32 KiB slots (256 rows x 128 bytes, 16-byte
// chunk c of row r at chunk c ^ (r & 7)), and scales per "epoch" of four K
// tiles -- 16 bytes per row, the row's 16 blocks of 32 over 512 K -- in two
// slots per operand (one 16-byte load per row and epoch).
//
// Schedule.  Window t is the time between the barriers that open tiles t and
// t + 1.  In it a wave
//   - runs the 64 MFMAs of tile t - 1 (row i of blocks: MFMAs 8 i .. 8 i + 7),
//   - reads tile t's B fragments and scales into the other of two register
//     buffers, and its A fragments of block row i into the registers of row
//     i as soon as tile t - 1's row i is done; row 7 alternates between two
//     registers so its read never waits for the last row,
//   - issues its quarter of the loads of tile t + 1 (and, in the third window
//     of an epoch, of the next epoch's scales) into slots freed at barrier t,
// then waits for its loads and reads and joins barrier t + 1.  K tiles and
// scale groups past K read from a resource of size zero.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "gemm_f16_w4.hpp"
#include "gemm_mxfp8.hpp"
#include "pipeline.hpp"

namespace tg {

// Extent of a tile's scale resource: through the 16-byte word (a scale
// load's unit) holding the last row's last block.  Range checks are per
// dword and a dword partly past the end reads as zero, so an extent ending
// inside the word would lose the last row's final scales when a row's
// block count is not a multiple of 16.  The tile base is 16-byte aligned,
// so the word never reaches past the 16-byte block -- and the page --
// holding that block.
__device__ __forceinline__ uint32_t scale_span(int rows_left, int nblk, int64_t ld) {
    return (span_bytes(rows_left, nblk, ld, 1) + 15u) & ~15u;
}

// K tails (K not a multiple of 512): the last scale group's 16-byte word per
// row holds bytes past the row's last block (padding, or a later row's
// scales) which must not be applied: the data of those blocks is zero, but
// a NaN scale code times zero is NaN.  Lane l of wave w holds row 64 w + l's
// word of each operand (where the scale loads put it); its bytes rem .. 15
// (rem: valid blocks, 1 .. 15) are cleared.  Called after the group's loads
// have landed, before the barrier that publishes them; byte stores, so that
// it needs no registers beyond an address where the fragments are live.
__device__ __forceinline__ void mx_scale_tail_fixup(char *smem, int sa_off, int sb_off, int lane, int rem) {
    char *wa = smem + sa_off + lane * 16, *wb = smem + sb_off + lane * 16;
    for (int b = rem; b < 16; ++b) {
        wa[b] = 0;
        wb[b] = 0;
    }
    wait_lgkmcnt0();
}

// Work item of a four-wave block-scaled workgroup: its 256 x 256 output
// tile and, with SPLIT (split-K), its K range [k_lo, k_lo + K) -- split s of
// ranges of p.kt_split scale epochs (512 K each), the last one shorter.
template <bool SPLIT>
__device__ __forceinline__ void mx_work_item(const F16Args &p, int &m0, int &n0, int &split, int &k_lo, int &K) {
    int tmi, tni;
    split = 0;
    if constexpr (SPLIT)
        tile_order_split(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tmi, tni, split);
    else
        tile_order(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tmi, tni);
    m0 = tmi * 256;
    n0 = tni * 256;
    k_lo = SPLIT ? split * p.kt_split * 512 : 0;
    K = SPLIT ? (p.K - k_lo < p.kt_split * 512 ? p.K - k_lo : p.kt_split * 512) : p.K;
}

// Epilogue of the four-wave block-scaled kernels: D = acc + C, or with SPLIT
// the fp32 partial tile of split `split` into the workspace (no C: the
// reduction adds the slices and C; partial tiles stay cacheable, the
// reduction reads them right after).
template <bool OUT_BF16, int DAUX, bool SPLIT, int TM, int TN>
__device__ __forceinline__ void mx_epilogue(const f32x4 (&acc)[TM][TN], char *smem, int wave, int lane, int wm,
                                            int wn, int m0, int n0, const F16Args &p, int split, const F16Epi &e) {
    constexpr int WTM = TM * 16, WTN = TN * 16;        // the wave's quadrant
    if constexpr (SPLIT) {
        static_assert(!OUT_BF16, "split-K partial tiles are fp32");
        float *part = p.ws + (int64_t)split * p.M * p.ldw;
        epilogue_lds16<false, TM, TN, WTM, WTN, 0>(acc, smem, wave, lane, wm, wn, m0, n0, p.M, p.N, nullptr, 0, part,
                                                   p.ldw, e);
    } else {
        epilogue_lds16<OUT_BF16, TM, TN, WTM, WTN, DAUX>(acc, smem, wave, lane, wm, wn, m0, n0, p.M, p.N, p.C, p.ldc,
                                                         p.D, p.ldd, e);
    }
}

// One 16x16x128 e4m3 MFMA on an AGPR accumulator block, in place; SA / SB:
// the byte of each scale register used (encoded in op_sel / op_sel_hi).
template <int SA, int SB>
__device__ __forceinline__ void mfma_mx16_acc(f32x4 &acc, const i32x8 &a, const i32x8 &b, uint32_t sa, uint32_t sb) {
#define TG_STR2(x) #x
#define TG_STR(x) TG_STR2(x)
    asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[" TG_STR(%c5) "," TG_STR(%c6)
                 ",0] op_sel_hi:[" TG_STR(%c7) "," TG_STR(%c8) ",0]"
                 : "+a"(acc)
                 : "v"(a), "v"(b), "v"(sa), "v"(sb), "n"(SA & 1), "n"(SB & 1), "n"(SA >> 1), "n"(SB >> 1));
#undef TG_STR
#undef TG_STR2
}

// PERSIST: one workgroup per CU walks the tiles w, w + grid, w + 2 grid, ...
// (virtual workgroup ids, so the XCD-aware tile order is the one a full
// grid would have).  After a tile's last K step it issues the next tile's
// first loads (K tile 0 and its scales, into the slots K tile 0 always
// uses) and only then stages and stores the finished tile's D, from the
// other slots, so those loads run while D drains; the next tile then waits
// for its loads only, not for the stores issued after them.  Taken for
// calls without C whose D rows allow whole 16-byte row segments.
template <bool OUT_BF16, int DAUX = kStoreStream, bool SPLIT = false, bool PERSIST = false>
__global__ void __launch_bounds__(256) gemm_mx_w4_kernel(MxArgs q, F16Epi e) {
    static_assert(!(PERSIST && SPLIT), "persistent: whole tiles");
    const F16Args &p = q.g;
    constexpr int BK = 128, ROWB = 128;                // fp8: one byte per element
    constexpr int TM = 8, TN = 8, WTM = 128, WTN = 128;
    constexpr int SLOT = 256 * ROWB;                   // 32 KiB per operand slot
    constexpr int SS = 256 * 16;                       // one scale slot: 256 rows x 16 bytes
    constexpr int A_BASE = 0, B_BASE = 2 * SLOT, SA_BASE = 4 * SLOT, SB_BASE = SA_BASE + 2 * SS;
    constexpr int RING_BYTES = SB_BASE + 2 * SS;
    constexpr int EPI_BYTES = epilogue_lds_bytes(4, WTN);
    constexpr int LDS_BYTES = RING_BYTES > EPI_BYTES ? RING_BYTES : EPI_BYTES;
    constexpr int IB = 1024;                           // one load instruction: 8 rows
    static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");

    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    int m0, n0, split, k_lo, K;
    mx_work_item<SPLIT>(p, m0, n0, split, k_lo, K);
    const int nblk = K / 32;
    const int nk = K / BK, nep = K / 512;
    int vt = blockIdx.x;                               // PERSIST: the virtual workgroup id
    if constexpr (PERSIST) {
        int tmi, tni;
        tile_order(vt, p.tiles_m * p.tiles_n, p.tiles_m, p.tiles_n, p.group_m, tmi, tni);
        m0 = tmi * 256;
        n0 = tni * 256;
    }

    __amdgpu_buffer_rsrc_t rA, rB, rSA, rSB;
    auto tile_resources = [&](const MxArgs &a) __attribute__((always_inline)) {
        const F16Args &g = a.g;
        rA = make_rsrc((const char *)g.A + (int64_t)m0 * g.lda + k_lo, span_bytes(g.M - m0, K, g.lda, 1));
        rB = make_rsrc((const char *)g.B + (int64_t)n0 * g.ldb + k_lo, span_bytes(g.N - n0, K, g.ldb, 1));
        rSA = make_rsrc((const char *)a.SFA + (int64_t)m0 * a.ldsfa + k_lo / 32, span_bytes(g.M - m0, nblk, a.ldsfa, 1));
        rSB = make_rsrc((const char *)a.SFB + (int64_t)n0 * a.ldsfb + k_lo / 32, span_bytes(g.N - n0, nblk, a.ldsfb, 1));
    };
    tile_resources(q);
    const __amdgpu_buffer_rsrc_t rZ = make_rsrc(p.A, 0u);

    // Operand loads: instruction j of wave w fills slot rows (4 j + w) * 8 +
    // lane / 8; lane L writes physical chunk L % 8 and fetches logical chunk
    // (L % 8) ^ (L / 8).  Row step (32 j rows) and K offset go in the scalar
    // offset.  Scale loads: lane L of wave w brings row 64 w + L's 16 bytes.
    const int lchunk = ((lane & 7) ^ (lane >> 3)) << 4;
    const uint32_t a_base = (uint32_t)((wave * 8 + (lane >> 3)) * p.lda) + lchunk;
    const uint32_t b_base = (uint32_t)((wave * 8 + (lane >> 3)) * p.ldb) + lchunk;
    const uint32_t a_step = (uint32_t)(32 * p.lda), b_step = (uint32_t)(32 * p.ldb);
    auto dma = [&](__amdgpu_buffer_rsrc_t r, int lds, uint32_t voff, int soff) __attribute__((always_inline)) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(smem + lds), 16, voff,
                                                 soff, 0, 0);
    };
    auto fetch_a = [&](int t, int j) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t r = t < nk ? rA : rZ;
        const int so = (int)(j * a_step) + t * BK;
        dma(r, A_BASE + (t & 1) * SLOT + (j * 4 + wave) * IB, a_base, so);
    };
    auto fetch_b = [&](int t, int j) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t r = t < nk ? rB : rZ;
        const int so = (int)(j * b_step) + t * BK;
        dma(r, B_BASE + (t & 1) * SLOT + (j * 4 + wave) * IB, b_base, so);
    };
    // (scale offsets are used once per epoch: recomputed from the lane index,
    // which passes through an empty asm so they are not held in registers)
    auto lane_id = [&]() __attribute__((always_inline)) {
        int l = lane;
        asm volatile("" : "+v"(l));
        return l;
    };
    auto fetch_scales = [&](int ep) __attribute__((always_inline)) {
        const int l = lane_id();
        const int so = ep * 16;
        const __amdgpu_buffer_rsrc_t ra = ep < nep ? rSA : rZ;
        const __amdgpu_buffer_rsrc_t rb = ep < nep ? rSB : rZ;
        dma(ra, SA_BASE + (ep & 1) * SS + wave * IB, (uint32_t)((64 * wave + l) * q.ldsfa), so);
        dma(rb, SB_BASE + (ep & 1) * SS + wave * IB, (uint32_t)((64 * wave + l) * q.ldsfb), so);
    };

    // Fragment reads: lane l reads row l % 16 of each block, chunks q and
    // 4 + q (q = l / 16); rows of a block are 16 apart in the swizzle's
    // period, so the chunk offsets are the same for every block.
    const int fr = lane & 15, fq = lane >> 4;
    const int c0 = (fq ^ swz16(fr)) << 4;              // chunk q; chunk 4 + q is c0 ^ 64
    // (the four base addresses pass through an empty asm: otherwise the
    // compiler rewrites base + constant as a bitwise or, which LDS reads
    // cannot take as an immediate offset, and holds one address register per
    // block and slot)
    int la0 = A_BASE + (wm * WTM + fr) * ROWB + c0, la1 = la0 ^ 64;
    int lb0 = B_BASE + (wn * WTN + fr) * ROWB + c0, lb1 = lb0 ^ 64;
    asm volatile("" : "+v"(la0), "+v"(la1), "+v"(lb0), "+v"(lb1));
    auto ld32 = [&](int a0, int a1) __attribute__((always_inline)) {
        const u32x4 lo = *(const u32x4 *)(smem + a0), hi = *(const u32x4 *)(smem + a1);
        return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    f32x4 acc[TM][TN];
    i32x8 fa[TM], fx;                                  // A fragments; fx: row 7 of odd tiles
    i32x8 fb[2][TN];                                   // B fragments by tile parity
    uint32_t sa[2][2], sb[2][2];                       // scale bytes by tile parity, 4 blocks each

    // Reads of tile t, whose position in its epoch U = t % 4 is a
    // compile-time constant at every call site (the loop advances by whole
    // epochs), so register buffers are chosen by constant parity.
    // A fragment of block row I:
    auto read_a = [&](auto uc, auto ic) __attribute__((always_inline)) {
        constexpr int P = decltype(uc)::value & 1, I = decltype(ic)::value;
        constexpr int o = P * SLOT + I * 16 * ROWB;
        const i32x8 v = ld32(la0 + o, la1 + o);
        if constexpr (I < TM - 1)
            fa[I] = v;
        else if constexpr (P)
            fx = v;
        else
            fa[TM - 1] = v;
    };
    auto read_b = [&](auto uc, auto jc) __attribute__((always_inline)) {
        constexpr int P = decltype(uc)::value & 1, J = decltype(jc)::value;
        constexpr int o = P * SLOT + J * 16 * ROWB;
        fb[P][J] = ld32(lb0 + o, lb1 + o);
    };
    // Scale bytes: row r of the quadrant, K block q of tile U at byte
    // r * 16 + 4 U + q of the epoch's slot; four block rows (16 rows apart)
    // per register, byte u for block row 4 h' + u; H: 0, 1 the A registers,
    // 2, 3 the B ones.  A register is built from the four rows' dwords with
    // two v_perm (each keeps byte q of two dwords; the selectors depend only
    // on q).  The dword reads (scale_issue) and the assembly (scale_finish)
    // are 8 MFMAs apart through two stages of raw dwords, so the wave does
    // not wait for LDS reads still in flight.
    const uint32_t sel_lo = (uint32_t)fq | ((uint32_t)(fq + 4) << 8) | 0x0c0c0000u;   // 0x0c: a zero byte
    const uint32_t sel_hi = 0x00000c0cu | ((uint32_t)fq << 16) | ((uint32_t)(fq + 4) << 24);
    uint32_t sraw[2][4];
    // (row bases through an empty asm: every scale read then takes its
    // block-row and epoch offset as an immediate)
    int srow_a = SA_BASE + (wm * WTM + fr) * 16, srow_b = SB_BASE + (wn * WTN + fr) * 16;
    asm volatile("" : "+v"(srow_a), "+v"(srow_b));
    auto scale_issue = [&](auto uc, auto hc, auto gc, int t) __attribute__((always_inline)) {
        constexpr int U = decltype(uc)::value, H = decltype(hc)::value, G = decltype(gc)::value;
        const int base = (H < 2 ? srow_a : srow_b) + ((t >> 2) & 1) * SS + U * 4 + (H & 1) * 4 * 256;
#pragma unroll
        for (int u = 0; u < 4; ++u) sraw[G][u] = *(const uint32_t *)(smem + base + u * 256);
    };
    auto scale_finish = [&](auto uc, auto hc, auto gc) __attribute__((always_inline)) {
        constexpr int P = decltype(uc)::value & 1, H = decltype(hc)::value, G = decltype(gc)::value;
        const uint32_t v = __builtin_amdgcn_perm(sraw[G][1], sraw[G][0], sel_lo) |
                           __builtin_amdgcn_perm(sraw[G][3], sraw[G][2], sel_hi);
        if constexpr (H < 2)
            sa[P][H] = v;
        else
            sb[P][H - 2] = v;
    };
    // MFMA Q (row Q / 8, column Q % 8) of a tile of parity P
    auto mfma = [&](auto pc, auto qc) __attribute__((always_inline)) {
        constexpr int P = decltype(pc)::value, Q = decltype(qc)::value;
        constexpr int I = Q / TN, J = Q % TN;
        if constexpr (I < TM - 1 || !P)
            mfma_mx16_acc<I % 4, J % 4>(acc[I][J], fa[I], fb[P][J], sa[P][I / 4], sb[P][J / 4]);
        else
            mfma_mx16_acc<I % 4, J % 4>(acc[I][J], fx, fb[P][J], sa[P][I / 4], sb[P][J / 4]);
        __builtin_amdgcn_sched_barrier(0);
    };
    // Window t (U = t % 4): MFMAs of tile t - 1 (unless FIRST), reads of
    // tile t -- B block j at MFMA 4 j, A row 7 at MFMA 3 and row i - 1
    // during row i, scales read at MFMAs 34 .. 46 and assembled 8 MFMAs
    // later -- loads of tile t + 1 at every
    // second MFMA of the first 32 (1-2 % faster at 8192^3 than every third
    // of the first 48; all 16 back to back, 7 % slower), the next epoch's
    // scales when U == 2.
    auto window = [&](auto first, auto uc, int t) __attribute__((always_inline)) {
        constexpr bool F = decltype(first)::value;
        constexpr int U = decltype(uc)::value;
        if constexpr (U == 2) fetch_scales((t >> 2) + 1);
        static_for<0, 64>([&](auto qc) __attribute__((always_inline)) {
            constexpr int Q = decltype(qc)::value;
            if constexpr (!F) mfma(std::integral_constant<int, (U + 1) & 1>(), qc);
            if constexpr (Q % 2 == 1 && Q / 2 < 16) {
                constexpr int k = Q / 2;
                if constexpr (k < 8)
                    fetch_a(t + 1, k);
                else
                    fetch_b(t + 1, k - 8);
            }
            if constexpr (Q < 32 && Q % 4 == 0) read_b(uc, std::integral_constant<int, Q / 4>());
            if constexpr (Q == 3) read_a(uc, std::integral_constant<int, TM - 1>());
            if constexpr (Q >= 8 && Q % 8 == 3) read_a(uc, std::integral_constant<int, Q / 8 - 1>());
            if constexpr (Q >= 42 && Q <= 54 && Q % 4 == 2) {
                constexpr int c = (Q - 42) / 4;
                scale_finish(uc, std::integral_constant<int, c>(), std::integral_constant<int, c % 2>());
            }
            if constexpr (Q >= 34 && Q <= 46 && Q % 4 == 2) {
                constexpr int c = (Q - 34) / 4;
                scale_issue(uc, std::integral_constant<int, c>(), std::integral_constant<int, c % 2>(), t);
            }
        });
        wait_vmcnt<0>();
        wait_lgkmcnt0();
        barrier();
    };

    // The first K tile of the current output tile and its scales (nk > 0).
    // wv, as, bs: the wave index and row steps; a persistent kernel passes
    // them through an empty asm so that the 32 LDS destinations and scalar
    // offsets of these loads are computed here, not held through the main
    // loop.
    auto prologue_loads = [&](int wv, uint32_t as, uint32_t bs) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) dma(rA, A_BASE + (j * 4 + wv) * IB, a_base, (int)(j * as));
#pragma unroll
        for (int j = 0; j < 8; ++j) dma(rB, B_BASE + (j * 4 + wv) * IB, b_base, (int)(j * bs));
        const int l = lane_id();
        dma(rSA, SA_BASE + wv * IB, (uint32_t)((64 * wv + l) * q.ldsfa), 0);
        dma(rSB, SB_BASE + wv * IB, (uint32_t)((64 * wv + l) * q.ldsfb), 0);
    };
    // PERSIST: stores per wave of the finished tile's D (epilogue_rows16_vec:
    // WTM / 16 passes of 16 / RPS stores, RPS = 64 / (WTN / 4))
    constexpr int D_STORES = (WTM / 16) * (16 * WTN / 4 / 64);
    // PERSIST: this wave's D staging area, in the slots K tile 0 does not use
    float *stage = (float *)(smem + (wave < 2 ? A_BASE + SLOT : B_BASE + SLOT) + (wave & 1) * 16 * (WTN + 4) * 4);
    static_assert(2 * 16 * (WTN + 4) * 4 <= SLOT, "staging areas");

    if (nk > 0) {
        prologue_loads(wave, a_step, b_step);
        wait_vmcnt<0>();
        barrier();
    }
    while (true) {
        float z = 0.0f;                                // (made here, not a register held through the loop)
        asm volatile("" : "+v"(z));
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{z, z, z, z};
        mfma_result_fence<TM, TN>(acc);                // the zeroing before the first MFMA reads them
        if (nk > 0) {
            window(std::true_type(), std::integral_constant<int, 0>(), 0);
            // windows 1 .. nk (nk a multiple of 4): tiles 0 .. nk - 1 computed
            for (int t = 1; t <= nk; t += 4) {
                window(std::false_type(), std::integral_constant<int, 1>(), t);
                window(std::false_type(), std::integral_constant<int, 2>(), t + 1);
                window(std::false_type(), std::integral_constant<int, 3>(), t + 2);
                window(std::false_type(), std::integral_constant<int, 0>(), t + 3);
            }
        }
        mfma_result_fence<TM, TN>(acc);
        wait_vmcnt<0>();
        wait_lgkmcnt0();
        barrier();
        if constexpr (!PERSIST) {
            mx_epilogue<OUT_BF16, DAUX, SPLIT>(acc, smem, wave, lane, wm, wn, m0, n0, p, split, e);
            break;
        } else {
            const MxArgs r = kernel_arg0_reloaded<MxArgs>();
            const int dm0 = m0, dn0 = n0;              // the finished tile
            const int nt = r.g.tiles_m * r.g.tiles_n;
            vt += gridDim.x;
            const bool more = vt < nt;
            if (more) {
                int tmi, tni;
                tile_order(vt, nt, r.g.tiles_m, r.g.tiles_n, r.g.group_m, tmi, tni);
                m0 = tmi * 256;
                n0 = tni * 256;
                tile_resources(r);
                if (nk > 0) {
                    int wv = wave;
                    uint32_t as = a_step, bs = b_step;
                    asm volatile("" : "+s"(wv), "+s"(as), "+s"(bs));
                    prologue_loads(wv, as, bs);
                }
            }
            epilogue_rows16_vec<OUT_BF16, TM, TN, DAUX>(acc, stage, lane, wm, wn, dm0, dn0, r.g.M, r.g.N, r.g.D,
                                                        r.g.ldd);
            if (!more) break;
            // the next tile's first loads landed; up to 63 of the D stores issued after them may still run
            static_assert(D_STORES >= 63, "vmcnt");
            wait_vmcnt<63>();
            wait_lgkmcnt0();
            barrier();                                 // staging reads done before window 0 refills those slots
        }
    }
}

}  // namespace tg
