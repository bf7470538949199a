// Block-scaled fp4 D = A.B + C with four waves and
// v_mfma_scale_f32_16x16x128_f8f6f4 on e2m1 operands (cbsz = blgp = 4),
// gfx950 (K a multiple of 512):
//     a(m,k) = e2m1(A[m][k]) * 2^(SFA[m][k/32] - 127)
//     b(k,n) = e2m1(B[n][k]) * 2^(SFB[n][k/32] - 127)
// A and B hold two elements per byte, element 2i in the low nibble of byte i.
//
// Same frame as the four-wave fp8 kernel: a 256 x 256 output tile, one wave
// per SIMD owning a 128 x 128 quadrant as 8 x 8 blocks of 16 x 16 fp32
// accumulators in AGPRs, A and B arriving by direct global->LDS loads into
// two-slot rings of 128-byte rows (chunk c of row r at chunk c ^ (r & 7)).
// A 128-byte row now holds 256 K elements, i.e. two MFMA K steps, so one K
// tile is 128 MFMAs per wave: the fp4 MFMA takes half the cycles of the fp8
// one, and the window between barriers keeps the same length and the same
// 64 KiB of operand loads.
//
// Operand placement (measured with one-hot operands and distinct per-lane
// scales): lane l supplies row (A) or column (B) l % 16 and, as four
// registers, the 32 elements of K block q = l / 16 of the step -- 16 bytes,
// chunk 4 s + q of the row in step s; the block's scale comes from the same
// lane, op_sel picking the byte.  So a lane reads one 16-byte chunk per block
// and step, and each of its scale registers holds (its row, block 4 s + q)
// for two block rows 16 apart and both steps of a tile.
//
// Scales: 16 bytes per row cover 512 K, i.e. an "epoch" of two K tiles, in
// two slots per operand; the next epoch's are loaded in the second window of
// an epoch.
//
// Window t (between the barriers that open tiles t and t + 1): the 128
// MFMAs of tile t - 1 in row order (row i: step 0 then step 1 of its eight
// blocks), reads of tile t -- B fragments first, A row i - 1 once tile
// t - 1 is done with it, row 7 into a register pair chosen by tile parity --
// and the wave's quarter of the loads of tile t + 1.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "gemm_mx_w4.hpp"
#include "pipeline.hpp"

namespace tg {

// One 16x16x128 e2m1 MFMA on an AGPR accumulator block, in place; SA / SB:
// the byte of each scale register used.
template <int SA, int SB>
__device__ __forceinline__ void mfma_mx4_acc(f32x4 &acc, const u32x4 &a, const u32x4 &b, uint32_t sa, uint32_t sb) {
#define TG_STR2(x) #x
#define TG_STR(x) TG_STR2(x)
    asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[" TG_STR(%c5) "," TG_STR(%c6)
                 ",0] op_sel_hi:[" TG_STR(%c7) "," TG_STR(%c8) ",0] cbsz:4 blgp:4"
                 : "+a"(acc)
                 : "v"(a), "v"(b), "v"(sa), "v"(sb), "n"(SA & 1), "n"(SB & 1), "n"(SA >> 1), "n"(SB >> 1));
#undef TG_STR
#undef TG_STR2
}

// q.g.lda and q.g.ldb are in BYTES here (half the leading dimension in
// elements); q.g.K is in elements.  PERSIST: one workgroup per CU walking
// the tiles, as the persistent fp8 kernel (no C, D rows of whole 16-byte
// segments).
template <bool OUT_BF16, int DAUX = kStoreStream, bool SPLIT = false, bool PERSIST = false>
__global__ void __launch_bounds__(256) gemm_mx4_w4_kernel(MxArgs q, F16Epi e) {
    static_assert(!(PERSIST && SPLIT), "persistent: whole tiles");
    const F16Args &p = q.g;
    constexpr int ROWB = 128, BKB = 128;               // bytes per LDS row = bytes per K tile (256 elements)
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
    const int kb = K / 2, nblk = K / 32;
    const int nk = K / 256, nep = K / 512;
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
        rA = make_rsrc((const char *)g.A + (int64_t)m0 * g.lda + k_lo / 2, span_bytes(g.M - m0, kb, g.lda, 1));
        rB = make_rsrc((const char *)g.B + (int64_t)n0 * g.ldb + k_lo / 2, span_bytes(g.N - n0, kb, g.ldb, 1));
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
        const int so = (int)(j * a_step) + t * BKB;
        dma(r, A_BASE + (t & 1) * SLOT + (j * 4 + wave) * IB, a_base, so);
    };
    auto fetch_b = [&](int t, int j) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t r = t < nk ? rB : rZ;
        const int so = (int)(j * b_step) + t * BKB;
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

    // Fragment reads: lane l reads row l % 16 of each block, chunk s * 4 + q
    // (q = l / 16) in step s; rows of a block are 16 apart in the swizzle's
    // period, so the offsets are the same for every block.
    const int fr = lane & 15, fq = lane >> 4;
    const int c0 = (fq ^ swz16(fr)) << 4;              // step 0: chunk q; step 1: chunk 4 + q at c0 ^ 64
    // (one base per operand and step, through an empty asm so that block and
    // slot offsets fold into the LDS reads' immediate offsets)
    int la[2], lb[2];
    la[0] = A_BASE + (wm * WTM + fr) * ROWB + c0;
    lb[0] = B_BASE + (wn * WTN + fr) * ROWB + c0;
    la[1] = la[0] ^ 64;
    lb[1] = lb[0] ^ 64;
    asm volatile("" : "+v"(la[0]), "+v"(la[1]), "+v"(lb[0]), "+v"(lb[1]));
    auto ld16 = [&](int a) __attribute__((always_inline)) { return *(const u32x4 *)(smem + a); };

    f32x4 acc[TM][TN];
    u32x4 fa[2][TM], fx[2];                            // A fragments by step; fx: row 7 of odd tiles
    u32x4 fb[2][2][TN];                                // B fragments by tile parity and step
    uint32_t sa[2][4], sb[2][4];                       // scale bytes by tile parity and block-row pair

    // Reads of tile t (parity P = U, its place in the epoch, a compile-time
    // constant at every call site).  A fragment of block row I, step S:
    auto read_a = [&](auto uc, auto ic, auto sc) __attribute__((always_inline)) {
        constexpr int P = decltype(uc)::value, I = decltype(ic)::value, S = decltype(sc)::value;
        const u32x4 v = ld16(la[S] + P * SLOT + I * 16 * ROWB);
        if constexpr (I < TM - 1 || !P)
            fa[S][I] = v;
        else
            fx[S] = v;
    };
    auto read_b = [&](auto uc, auto jc, auto sc) __attribute__((always_inline)) {
        constexpr int P = decltype(uc)::value, J = decltype(jc)::value, S = decltype(sc)::value;
        fb[P][S][J] = ld16(lb[S] + P * SLOT + J * 16 * ROWB);
    };
    // Scale registers of a tile: register h of A (of B) holds, for the
    // lane's row r of the quadrant and its K block q of each step, the
    // scales of block rows 2 h and 2 h + 1 -- byte 2 (I & 1) + S for block
    // row I, step S, i.e. K block 8 U + 4 S + q of row r + 16 I, at byte
    // (r + 16 I) * 16 + 8 U + 4 S + q of the epoch's slot.  One 8-byte read
    // per block row gives the two dwords holding steps 0 and 1; v_perm keeps
    // byte q of each (the selectors depend only on q).  The reads of a
    // register (scale_issue) and its assembly (scale_finish) are 16 MFMAs
    // apart, through two stages of raw dwords, so the wave never waits for
    // LDS reads still in flight.
    const uint32_t sel_lo = (uint32_t)fq | ((uint32_t)(fq + 4) << 8) | 0x0c0c0000u;   // 0x0c: a zero byte
    const uint32_t sel_hi = 0x00000c0cu | ((uint32_t)fq << 16) | ((uint32_t)(fq + 4) << 24);
    // (row bases through an empty asm: every scale read then takes its
    // block-row and epoch offset as an immediate, instead of the compiler
    // holding a hoisted address per read)
    int srow_a = SA_BASE + (wm * WTM + fr) * 16, srow_b = SB_BASE + (wn * WTN + fr) * 16;
    asm volatile("" : "+v"(srow_a), "+v"(srow_b));
    u32x2 sraw[2][2];
    // register c of tile t: A pair c (c < 4) or B pair c - 4
    auto scale_issue = [&](auto uc, auto cc, auto gc, int t) __attribute__((always_inline)) {
        constexpr int U = decltype(uc)::value, C = decltype(cc)::value, G = decltype(gc)::value;
        const int base = (C < 4 ? srow_a : srow_b) + ((t >> 1) & 1) * SS + 8 * U + (C % 4) * 512;
        sraw[G][0] = *(const u32x2 *)(smem + base);
        sraw[G][1] = *(const u32x2 *)(smem + base + 256);
    };
    auto scale_finish = [&](auto uc, auto cc, auto gc) __attribute__((always_inline)) {
        constexpr int U = decltype(uc)::value, C = decltype(cc)::value, G = decltype(gc)::value;
        const uint32_t v = __builtin_amdgcn_perm(sraw[G][0][1], sraw[G][0][0], sel_lo) |
                           __builtin_amdgcn_perm(sraw[G][1][1], sraw[G][1][0], sel_hi);
        if constexpr (C < 4)
            sa[U][C] = v;
        else
            sb[U][C - 4] = v;
    };
    // MFMA Q of a tile of parity P: row Q / 16, step (Q / 8) % 2, column Q % 8
    auto mfma = [&](auto pc, auto qc) __attribute__((always_inline)) {
        constexpr int P = decltype(pc)::value, Q = decltype(qc)::value;
        constexpr int I = Q / 16, S = (Q / 8) % 2, J = Q % 8;
        constexpr int BA = 2 * (I & 1) + S, BB = 2 * (J & 1) + S;
        if constexpr (I < TM - 1 || !P)
            mfma_mx4_acc<BA, BB>(acc[I][J], fa[S][I], fb[P][S][J], sa[P][I / 2], sb[P][J / 2]);
        else
            mfma_mx4_acc<BA, BB>(acc[I][J], fx[S], fb[P][S][J], sa[P][I / 2], sb[P][J / 2]);
        __builtin_amdgcn_sched_barrier(0);
    };
    // Window t (U = t % 2): MFMAs of tile t - 1 (unless FIRST); reads of
    // tile t: B (step, block) at MFMAs 0, 4, .., 60, A row 7 at MFMAs 3 and
    // 5, row i - 1 at 16 i + 3 and 16 i + 5, scales issued at 6, 14, .., 62
    // and extracted 16 MFMAs later; loads of
    // tile t + 1 at every sixth MFMA of the first 96; the next epoch's
    // scales when U == 1.
    auto window = [&](auto first, auto uc, int t) __attribute__((always_inline)) {
        constexpr bool F = decltype(first)::value;
        constexpr int U = decltype(uc)::value;
        if constexpr (U == 1) fetch_scales((t >> 1) + 1);
        static_for<0, 128>([&](auto qc) __attribute__((always_inline)) {
            constexpr int Q = decltype(qc)::value;
            if constexpr (!F) mfma(std::integral_constant<int, U ^ 1>(), qc);
            if constexpr (Q % 6 == 1 && Q / 6 < 16) {
                constexpr int k = Q / 6;
                if constexpr (k < 8)
                    fetch_a(t + 1, k);
                else
                    fetch_b(t + 1, k - 8);
            }
            if constexpr (Q < 64 && Q % 4 == 0)
                read_b(uc, std::integral_constant<int, (Q / 4) % 8>(), std::integral_constant<int, Q / 32>());
            if constexpr (Q == 3 || Q == 5)
                read_a(uc, std::integral_constant<int, TM - 1>(), std::integral_constant<int, Q == 5>());
            if constexpr (Q >= 16 && (Q % 16 == 3 || Q % 16 == 5))
                read_a(uc, std::integral_constant<int, Q / 16 - 1>(), std::integral_constant<int, Q % 16 == 5>());
            if constexpr (Q >= 22 && Q <= 78 && Q % 8 == 6) {
                constexpr int c = (Q - 22) / 8;
                scale_finish(uc, std::integral_constant<int, c>(), std::integral_constant<int, c % 2>());
            }
            if constexpr (Q >= 6 && Q <= 62 && Q % 8 == 6) {
                constexpr int c = (Q - 6) / 8;
                scale_issue(uc, std::integral_constant<int, c>(), std::integral_constant<int, c % 2>(), t);
            }
        });
        wait_vmcnt<0>();
        wait_lgkmcnt0();
        barrier();
    };

    // Tile 0 of the current output tile and the first epoch's scales (nk >
    // 0); wv, as, bs as in the persistent fp8 kernel.
    auto prologue_loads = [&](int wv, uint32_t as, uint32_t bs) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) dma(rA, A_BASE + (j * 4 + wv) * IB, a_base, (int)(j * as));
#pragma unroll
        for (int j = 0; j < 8; ++j) dma(rB, B_BASE + (j * 4 + wv) * IB, b_base, (int)(j * bs));
        const int l = lane_id();
        dma(rSA, SA_BASE + wv * IB, (uint32_t)((64 * wv + l) * q.ldsfa), 0);
        dma(rSB, SB_BASE + wv * IB, (uint32_t)((64 * wv + l) * q.ldsfb), 0);
    };
    // PERSIST: this wave's D staging area, in the slots tile 0 does not use
    float *stage = (float *)(smem + (wave < 2 ? A_BASE + SLOT : B_BASE + SLOT) + (wave & 1) * 16 * (WTN + 4) * 4);
    static_assert(2 * 16 * (WTN + 4) * 4 <= SLOT, "staging areas");
    constexpr int D_STORES = (WTM / 16) * (16 * WTN / 4 / 64);

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
            // windows 1 .. nk (nk even): tiles 0 .. nk - 1 computed
            for (int t = 1; t <= nk; t += 2) {
                window(std::false_type(), std::integral_constant<int, 1>(), t);
                window(std::false_type(), std::integral_constant<int, 0>(), t + 1);
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
