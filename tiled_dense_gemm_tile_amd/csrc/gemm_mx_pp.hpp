// Block-scaled fp8 D = A.B + C with the ping-pong schedule and
// v_mfma_scale_f32_16x16x128_f8f6f4, gfx950 (K a multiple of 128).
//
// Same structure as the 16-bit ping-pong kernel: a 256 x 256 tile, 8 waves
// in two groups of four that alternate each phase between a memory phase
// (global->LDS loads for later K tiles, every fragment and scale of the next
// K tile read into registers) and a compute phase (32 MFMAs, nothing else).
// Group g owns rows [128 g, 128 g + 128), wave s of a group columns
// [64 s, 64 s + 64): 8 x 4 blocks of 16 x 16 fp32 accumulators.
//
// Operand placement (measured on gfx950 with one-hot operands and distinct
// per-lane scales): lane l supplies row (A) or column (B) l % 16; its bytes
// 0..15 are K elements [16 q, 16 q + 16) and bytes 16..31 are
// [64 + 16 q, 64 + 16 q + 16) of the 128-wide K step, q = l / 16.  The
// 32-wide K block b of row r takes its scale from lane 16 b + r (byte 0 with
// op_sel 0).  So lane l reads 16-byte chunks q and 4 + q of its row, and the
// scale byte of (its row, block q).
//
// A K tile is 128 fp8 per row (128-byte LDS rows, chunk XOR (row & 7), which
// is conflict free for these reads).  Rings: the two A halves 2 slots each,
// B 2 slots (32 KiB).  Loads by group: group 0 in its memory phase of tile t
// issues B(t+1) and A half 1 of t+1; group 1 issues A half 0 of t+2.  B has
// two phases to land, the A halves three.
//
// Scales come in per "epoch" of four K tiles: 16 bytes per row (the row's
// 16 blocks of 32 over 512 K) with 16-byte lanes, into two alternating slots
// per operand (or A half).  A row's scales of one tile are thus 4 of its 16
// bytes, read per lane as single bytes at the start of each memory phase and
// packed four to a register.  Loading 4 bytes per row per tile instead costs
// one L2 request per row per tile for 4 useful bytes and was the largest
// single cost of the loop.  Epoch E's scales are issued in the memory phase
// of tile 4E - 2 and first read in that of tile 4E.  The loop runs in steps
// of four tiles (zero tiles, loaded out of range, pad the end); the scale
// bytes of tiles past K are replaced by 1.0 so stale bytes cannot turn the
// zero products into NaN.
#pragma once

#include "common.hpp"
#include "gemm_f16_pp.hpp"
#include "gemm_mxfp8.hpp"
#include "pipeline.hpp"

namespace tg {

// One 16x16x128 e4m3 MFMA updating a VGPR accumulator block in place; SA /
// SB: the byte of each scale register used (encoded in op_sel / op_sel_hi).
// Inline asm with the accumulator tied: the compiler's own MFMA form lets
// the register allocator rotate accumulators through freed fragment
// registers, which costs copies and spills at this register budget.
template <int SA, int SB>
__device__ __forceinline__ void mfma_mx16(f32x4 &acc, const i32x8 &a, const i32x8 &b, uint32_t sa, uint32_t sb) {
#define TG_STR2(x) #x
#define TG_STR(x) TG_STR2(x)
    asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[" TG_STR(%c5) "," TG_STR(%c6)
                 ",0] op_sel_hi:[" TG_STR(%c7) "," TG_STR(%c8) ",0]"
                 : "+v"(acc)
                 : "v"(a), "v"(b), "v"(sa), "v"(sb), "n"(SA & 1), "n"(SB & 1), "n"(SA >> 1), "n"(SB >> 1));
#undef TG_STR
#undef TG_STR2
}

// Wait states between VALU writes / MFMA writes of the accumulators and
// their next use by the other kind of instruction; every accumulator passes
// through one of these statements (tied), which issue in order.
template <int TM, int TN>
__device__ __forceinline__ void acc_fence(f32x4 (&acc)[TM][TN]) {
    static_assert(TN == 4, "four blocks per statement");
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        if (i == 0)
            asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 3"
                         : "+v"(acc[i][0]), "+v"(acc[i][1]), "+v"(acc[i][2]), "+v"(acc[i][3]));
        else
            asm volatile("" : "+v"(acc[i][0]), "+v"(acc[i][1]), "+v"(acc[i][2]), "+v"(acc[i][3]));
    }
}

template <bool OUT_BF16>
__global__ void __launch_bounds__(512) gemm_mx_pp_kernel(MxArgs q, F16Epi e) {
    const F16Args &p = q.g;
    constexpr int BK = 128, ROWB = 128;                // fp8: one byte per element
    constexpr int TM = 8, TN = 4, WTM = 128, WTN = 64;
    constexpr int AH_BYTES = 128 * ROWB, B_BYTES = 256 * ROWB;
    constexpr int SS = 4096;                           // one scale slot: 4 waves x 1 KiB
    constexpr int A0_BASE = 0, A1_BASE = 2 * AH_BYTES, B_BASE = 4 * AH_BYTES;
    constexpr int S_BASE = B_BASE + 2 * B_BYTES;       // scales: A0 x2, A1 x2, B x2
    constexpr int SA0_BASE = S_BASE, SA1_BASE = S_BASE + 2 * SS, SB_BASE = S_BASE + 4 * SS;
    constexpr int RING_BYTES = S_BASE + 6 * SS;
    constexpr int EPI_BYTES = epilogue_lds_bytes(8, WTN);
    constexpr int LDS_BYTES = RING_BYTES > EPI_BYTES ? RING_BYTES : EPI_BYTES;
    constexpr int IB = 1024;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");

    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = wave >> 2, s = wave & 3;
    int tmi, tni;
    tile_order(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tmi, tni);
    const int m0 = tmi * 256, n0 = tni * 256;
    const int M = p.M, N = p.N, K = p.K;
    const int nblk = K / 32;
    const int nk = (K + BK - 1) / BK;

    const __amdgpu_buffer_rsrc_t rA =
        make_rsrc((const char *)p.A + (int64_t)m0 * p.lda, span_bytes(M - m0, K, p.lda, 1));
    const __amdgpu_buffer_rsrc_t rB =
        make_rsrc((const char *)p.B + (int64_t)n0 * p.ldb, span_bytes(N - n0, K, p.ldb, 1));
    const __amdgpu_buffer_rsrc_t rSA =
        make_rsrc((const char *)q.SFA + (int64_t)m0 * q.ldsfa, span_bytes(M - m0, nblk, q.ldsfa, 1));
    const __amdgpu_buffer_rsrc_t rSB =
        make_rsrc((const char *)q.SFB + (int64_t)n0 * q.ldsfb, span_bytes(N - n0, nblk, q.ldsfb, 1));

    // Register budget: at two waves per SIMD a wave has 256 VGPRs and the
    // accumulators, fragments and scales of a tile take 227 of them; a spill
    // inside the loop would be fatal (a scratch reload waits on vmcnt, i.e.
    // on every load in flight).  So each per-lane address is held as one base
    // register: the global loads put the row step and the K offset in the
    // load's scalar offset, and the LDS reads put block and slot offsets in
    // the instruction's immediate.
    const int a_row0 = g == 0 ? 128 : 0;                // group 0 loads half 1, group 1 half 0
    const uint32_t a_step = (uint32_t)(32 * p.lda), b_step = (uint32_t)(32 * p.ldb);
    // Operand load instruction j of wave s fills rows (4 j + s) * 8 + lane / 8
    // of its slot: lane L writes physical chunk L % 8 and fetches logical
    // chunk (L % 8) ^ (L / 8); instruction j adds 32 j rows.
    const int lchunk = ((lane & 7) ^ (lane >> 3)) << 4;
    const uint32_t a_base = (uint32_t)((a_row0 + s * 8 + (lane >> 3)) * p.lda) + lchunk;
    const uint32_t b_base = (uint32_t)((s * 8 + (lane >> 3)) * p.ldb) + lchunk;
    // Addresses used once per tile or less are recomputed where used from
    // the lane index, which passes through an empty asm so the compiler
    // cannot hoist them out of the loop into registers held across it.
    auto lane_id = [&]() __attribute__((always_inline)) {
        int l = lane;
        asm volatile("" : "+v"(l));
        return l;
    };
    // K tiles and scale groups past K read from a resource of size zero
    // (every load returns zeros), so no per-lane offset ever leaves the
    // resource's own range.
    const __amdgpu_buffer_rsrc_t rZ = make_rsrc(p.A, 0u);
    const int nep = nblk / 16;                         // scale groups of 512 K

    char *const a_fill = smem + (g == 0 ? A1_BASE : A0_BASE);
    char *const sa_fill = smem + (g == 0 ? SA1_BASE : SA0_BASE);
    auto fetch_a = [&](int t) {                         // this group's A half of K tile t
        const __amdgpu_buffer_rsrc_t r = t < nk ? rA : rZ;
        char *dst = a_fill + (t & 1) * AH_BYTES + s * IB;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int so = (int)(j * a_step) + t * BK;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(dst + j * 4 * IB), 16,
                                                     a_base, so, 0, 0);
        }
    };
    auto fetch_b = [&](int t) {                         // group 0 only
        const __amdgpu_buffer_rsrc_t r = t < nk ? rB : rZ;
        char *dst = smem + B_BASE + (t & 1) * B_BYTES + s * IB;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int so = (int)(j * b_step) + t * BK;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(dst + j * 4 * IB), 16,
                                                     b_base, so, 0, 0);
        }
    };
    // Scales of epoch ep (tiles 4 ep .. 4 ep + 3): group 0 loads B's and A
    // half 1's, group 1 A half 0's.
    // Scale loads (16-byte lanes): for an A half, lanes 0..31 of wave s bring
    // rows 32 s .. 32 s + 31 (lanes 32..63 read nothing); for B, lanes 0..63
    // rows 64 s .. 64 s + 63.  Each wave's instruction fills 1 KiB of the slot.
    auto fetch_scales = [&](int ep) {
        const int so = ep * 16;
        const int l = lane_id();
        const uint32_t sa_base = (uint32_t)((a_row0 + 32 * s + (l & 31)) * q.ldsfa) | (l < 32 ? 0u : kOOB);
        const uint32_t sb_base = (uint32_t)((64 * s + l) * q.ldsfb);
        if (g == 0) {
            const __amdgpu_buffer_rsrc_t r = ep < nep ? rSB : rZ;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(smem + SB_BASE + (ep & 1) * SS + s * IB),
                                                     16, sb_base, so, 0, 0);
        }
        const __amdgpu_buffer_rsrc_t r = ep < nep ? rSA : rZ;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(sa_fill + (ep & 1) * SS + s * IB),
                                                 16, sa_base, so, 0, 0);
    };

    // Fragment reads: lane l reads row l % 16 of each block, chunks q and
    // 4 + q (q = l / 16), and the scale byte of (that row, K block q).
    const int fr = lane & 15, fq = lane >> 4;
    const int c0 = (fq ^ swz16(fr)) << 4;              // chunk q; chunk 4 + q is c0 ^ 64
    const int la0 = (g == 0 ? A0_BASE : A1_BASE) + fr * ROWB + c0, la1 = la0 ^ 64;
    const int lb0 = B_BASE + (s * WTN + fr) * ROWB + c0, lb1 = lb0 ^ 64;

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;
    acc_fence<TM, TN>(acc);                            // zeroing (VALU) before the first MFMA reads them

    i32x8 fa[TM], fb[TN];
    // scale bytes packed four to a register: block i of A is byte i % 4 of
    // sa[i / 4], block j of B byte j of sb (the MFMA's op_sel picks the byte)
    uint32_t sa[TM / 4], sb;
    auto ld16 = [&](int addr) __attribute__((always_inline)) {
        return *(const u32x4 *)(smem + addr);
    };
    auto ld32 = [&](int a0, int a1) __attribute__((always_inline)) {
        const u32x4 lo = ld16(a0), hi = ld16(a1);
        return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // All fragments and scales of tile t: the scale bytes are read first so
    // their latency overlaps the fragment reads, and packed last.  Every
    // address is a held base plus a constant (t % 4 is fixed at each call
    // site) except the scale slot (ep & 1), one addition per tile.
    auto read_frags = [&](int t) {
        const int ep = t >> 2, u = t & 3;
        // scale byte of (row r of the A half, block q of tile u) at
        // (r / 32) KiB + (r % 32) * 16 + 4 u + q; r = 16 i + fr
        const int l = lane_id();
        const int so = (ep & 1) * SS + u * 4 + (l & 15) * 16 + (l >> 4);
        const int sa_t = (g == 0 ? SA0_BASE : SA1_BASE) + so, sb_t = SB_BASE + s * WTN * 16 + so;
        uint32_t ra[TM], rb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
            ra[i] = *(const uint8_t *)(smem + sa_t + (i >> 1) * IB + (i & 1) * 256);
#pragma unroll
        for (int j = 0; j < TN; ++j) rb[j] = *(const uint8_t *)(smem + sb_t + j * 256);
        const int oa = (t & 1) * AH_BYTES, ob = (t & 1) * B_BYTES;
        // half of the fragments, then the packing (the raw bytes' registers
        // are freed before the other half is read: fewer VGPRs at the peak)
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[j] = ld32(lb0 + ob + j * 16 * ROWB, lb1 + ob + j * 16 * ROWB);
#pragma unroll
        for (int i = 0; i < TM / 2; ++i) fa[i] = ld32(la0 + oa + i * 16 * ROWB, la1 + oa + i * 16 * ROWB);
        const bool live = t < nk;                      // tiles past K: scale 1.0 (their operands are zero)
#pragma unroll
        for (int h = 0; h < TM / 4; ++h) {
            const uint32_t v = ra[4 * h] | (ra[4 * h + 1] << 8) | (ra[4 * h + 2] << 16) | (ra[4 * h + 3] << 24);
            sa[h] = live ? v : 0x7f7f7f7fu;
        }
        const uint32_t v = rb[0] | (rb[1] << 8) | (rb[2] << 16) | (rb[3] << 24);
        sb = live ? v : 0x7f7f7f7fu;
#pragma unroll
        for (int i = TM / 2; i < TM; ++i) fa[i] = ld32(la0 + oa + i * 16 * ROWB, la1 + oa + i * 16 * ROWB);
    };
    auto compute = [&]() {
        // (unrolled by hand: the scale-byte selectors must be constants)
#define TG_ROW(i)                                                                                           \
    mfma_mx16<(i) % 4, 0>(acc[i][0], fa[i], fb[0], sa[(i) / 4], sb);                                       \
    mfma_mx16<(i) % 4, 1>(acc[i][1], fa[i], fb[1], sa[(i) / 4], sb);                                       \
    mfma_mx16<(i) % 4, 2>(acc[i][2], fa[i], fb[2], sa[(i) / 4], sb);                                       \
    mfma_mx16<(i) % 4, 3>(acc[i][3], fa[i], fb[3], sa[(i) / 4], sb);
        TG_ROW(0) TG_ROW(1) TG_ROW(2) TG_ROW(3) TG_ROW(4) TG_ROW(5) TG_ROW(6) TG_ROW(7)
#undef TG_ROW
    };

    // Loads in flight that a phase boundary may leave (per wave, per position
    // u of the tile in its epoch; see the derivation in the comments):
    //   group 0 issues in its memory phase of tile t: B(t+1) 8, A1(t+1) 4,
    //   and when t % 4 == 2 the scales of epoch t/4 + 1 (B 1, A1 1);
    //   group 1 issues A0(t+2) 4 and, when t % 4 == 2, the A0 scales 1.
    if (nk > 0) {
        if (g == 0) {
            // prologue: B(0) A1(0) S(epoch 0) | memory phase of tile 0: B(1) A1(1)
            fetch_b(0);
            fetch_a(0);
            fetch_scales(0);
            phase_end<1>();                            // B(0) and its scales landed (A1 scales may run)
            fetch_b(1);
            fetch_a(1);
            read_frags(0);
            phase_end<12>();                           // A1(0) and the A1 scales landed
            for (int t = 0; t < nk; t += 4) {
                // position u: compute tile t + u, then the memory phase of tile t + u + 1
                auto step = [&](auto uc) __attribute__((always_inline)) {
                    constexpr int u = decltype(uc)::value;
                    compute();
                    phase_end<u == 2 ? 6 : 4>();       // B(t + u + 1) landed
                    fetch_b(t + u + 2);
                    fetch_a(t + u + 2);
                    if constexpr (u == 1) fetch_scales(t / 4 + 1);
                    read_frags(t + u + 1);
                    phase_end<u == 2 ? 14 : (u == 1 ? 14 : 12)>();   // A1(t + u + 1) landed
                };
                step(std::integral_constant<int, 0>());
                step(std::integral_constant<int, 1>());
                step(std::integral_constant<int, 2>());
                step(std::integral_constant<int, 3>());
            }
        } else {
            fetch_a(0);
            fetch_a(1);
            fetch_scales(0);
            phase_end<0>();                            // A0(0) and the A0 scales landed
            phase_end<0>();                            // (group 0 reads tile 0)
            for (int t = 0; t < nk; t += 4) {
                auto step = [&](auto uc) __attribute__((always_inline)) {
                    constexpr int u = decltype(uc)::value;
                    fetch_a(t + u + 2);                // memory phase of tile t + u
                    if constexpr (u == 2) fetch_scales(t / 4 + 1);
                    read_frags(t + u);
                    phase_end<u == 2 ? 5 : 4>();       // A0(t + u + 1) (and at u = 3 the A0 scales) landed
                    compute();                         // compute phase of tile t + u
                    phase_end<u == 2 ? 5 : 4>();
                };
                step(std::integral_constant<int, 0>());
                step(std::integral_constant<int, 1>());
                step(std::integral_constant<int, 2>());
                step(std::integral_constant<int, 3>());
            }
        }
    }

    acc_fence<TM, TN>(acc);                            // last MFMAs before the epilogue reads them
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    barrier();
    epilogue_lds16<OUT_BF16, TM, TN, WTM, WTN>(acc, smem, wave, lane, g, s, m0, n0, M, N, p.C, p.ldc, p.D, p.ldd, e);
}

}  // namespace tg
