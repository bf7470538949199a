// Block-scaled fp6 D = A.B + C with four waves and
// v_mfma_scale_f32_16x16x128_f8f6f4 on e2m3 (FMT 2) or e3m2 (FMT 3)
// operands, gfx950 (K a multiple of 128; a last scale group short of 512 K
// has its bytes past K cleared in LDS):
//     a(m,k) = fp6(A, m, k) * 2^(SFA[m][k/32] - 127)
//     b(k,n) = fp6(B, n, k) * 2^(SFB[n][k/32] - 127)
// A and B hold six bits per element: element k of a row at bits 6k .. 6k+5
// of the row read as a little-endian bit string (four per three bytes).
//
// Same frame as the four-wave fp8 kernel: a 256 x 256 output tile, one wave
// per SIMD owning a 128 x 128 quadrant as 8 x 8 blocks of 16 x 16 fp32
// accumulators in AGPRs, 128-wide K tiles filled by direct global->LDS
// loads, scales in epochs of four K tiles.  The operand rings have three
// slots (the 24 KiB slots of fp6 leave room for a third, 160 KiB in all):
// the loads of tile t + 2 are issued in window t and only waited for at
// the end of window t + 1, so each load has two windows of MFMAs (2048
// cycles) to arrive instead of one.
//
// Operand placement (measured: B all ones, one bit of A at a time): lane l
// supplies row (A) or column (B) l % 16 and, as six registers, the 32
// elements of K block q = l / 16 packed exactly as in memory (element i at
// bits 6i .. 6i+5 of the 192 bits) -- 24 consecutive bytes of the row; the
// block's scale comes from the same lane, op_sel picking the byte.
//
// LDS: a K tile's row is 96 bytes, six 16-byte chunks, rows one after the
// other (the direct loads fill 64 consecutive chunk positions per
// instruction, so a wave's lanes fetch whole rows).  In rows 8 .. 15 of
// every 16 the chunks of each pair (0, 1), (2, 3), (4, 5) trade places:
// rows 96 bytes apart start 6 chunk columns apart, which repeats every 8
// rows, and the swap moves rows 8 .. 15 onto the other parity, so the 16
// rows of a fragment read (8 bytes per lane, one K block) sit in 16
// different 16-byte bank columns.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "gemm_mx_w4.hpp"
#include "pipeline.hpp"

namespace tg {

typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));

// One 16x16x128 fp6 MFMA on an AGPR accumulator block, in place; SA / SB:
// the byte of each scale register used; FMT: 2 e2m3, 3 e3m2.
template <int SA, int SB, int FMT>
__device__ __forceinline__ void mfma_mx6_acc(f32x4 &acc, const u32x6 &a, const u32x6 &b, uint32_t sa, uint32_t sb) {
#define TG_STR2(x) #x
#define TG_STR(x) TG_STR2(x)
    if constexpr (FMT == 2)
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[" TG_STR(%c5) "," TG_STR(%c6)
                     ",0] op_sel_hi:[" TG_STR(%c7) "," TG_STR(%c8) ",0] cbsz:2 blgp:2"
                     : "+a"(acc)
                     : "v"(a), "v"(b), "v"(sa), "v"(sb), "n"(SA & 1), "n"(SB & 1), "n"(SA >> 1), "n"(SB >> 1));
    else
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[" TG_STR(%c5) "," TG_STR(%c6)
                     ",0] op_sel_hi:[" TG_STR(%c7) "," TG_STR(%c8) ",0] cbsz:3 blgp:3"
                     : "+a"(acc)
                     : "v"(a), "v"(b), "v"(sa), "v"(sb), "n"(SA & 1), "n"(SB & 1), "n"(SA >> 1), "n"(SB >> 1));
#undef TG_STR
#undef TG_STR2
}

// q.g.lda and q.g.ldb are in BYTES here (three quarters of the leading
// dimension in elements); q.g.K is in elements.  PERSIST: one workgroup per
// CU walking the tiles, as the persistent fp8 kernel; the finished tile's D
// is staged in ring slot 2 while the next tile's tiles 0 and 1 load into
// slots 0 and 1.
//
// PACKED: A and B come as their LDS images (mx6_pack.hip): K tile
// t of row block b (256 rows) is the 24 KiB at ((b * nk) + t) * 24576, laid
// out exactly as the ring slot holds it, so every load instruction reads
// 1 KiB of consecutive bytes (the row-major operands' 96-byte row pieces
// cost two memory requests each); q.g.lda and q.g.ldb are unused.
template <bool OUT_BF16, int FMT, int DAUX = kStoreStream, bool SPLIT = false, bool PERSIST = false,
          bool PACKED = false>
__global__ void __launch_bounds__(256) gemm_mx6_w4_kernel(MxArgs q, F16Epi e) {
    static_assert(FMT == 2 || FMT == 3, "fp6 formats");
    static_assert(!(PERSIST && SPLIT), "persistent: whole tiles");
    static_assert(!(PACKED && SPLIT), "packed operands: whole K");
    const F16Args &p = q.g;
    constexpr int ROWB = 96;                           // bytes per K tile (128 elements) and LDS row
    constexpr int TM = 8, TN = 8, WTM = 128, WTN = 128;
    constexpr int SLOT = 256 * ROWB;                   // 24 KiB per operand slot
    constexpr int SS = 256 * 16;                       // one scale slot: 256 rows x 16 bytes
    constexpr int NS = 3;                              // slots per operand ring
    constexpr int A_BASE = 0, B_BASE = NS * SLOT, SA_BASE = 2 * NS * SLOT, SB_BASE = SA_BASE + 2 * SS;
    constexpr int RING_BYTES = SB_BASE + 2 * SS;
    constexpr int EPI_BYTES = epilogue_lds_bytes(4, WTN);
    constexpr int LDS_BYTES = RING_BYTES > EPI_BYTES ? RING_BYTES : EPI_BYTES;
    constexpr int IB = 1024;                           // one load instruction: 64 chunks
    constexpr int LPW = 6;                             // load instructions per wave and operand per tile
    static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");
    static_assert(4 * LPW * 64 == 256 * (ROWB / 16), "a tile's chunks are split evenly over the waves");

    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    int m0, n0, split, k_lo, K;
    mx_work_item<SPLIT>(p, m0, n0, split, k_lo, K);
    // K % 128 == 0: whole K tiles; the loop runs whole groups of four, reading
    // zeros past nk
    const int kb = K / 4 * 3, nblk = K / 32, rem = nblk % 16;
    const int nk = K / 128, nep = (K + 511) / 512;
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
        if constexpr (PACKED) {
            rA = make_rsrc((const char *)g.A + (int64_t)(m0 / 256) * nk * SLOT, (uint32_t)nk * SLOT);
            rB = make_rsrc((const char *)g.B + (int64_t)(n0 / 256) * nk * SLOT, (uint32_t)nk * SLOT);
        } else {
            rA = make_rsrc((const char *)g.A + (int64_t)m0 * g.lda + k_lo / 4 * 3,
                           span_bytes(g.M - m0, kb, g.lda, 1));
            rB = make_rsrc((const char *)g.B + (int64_t)n0 * g.ldb + k_lo / 4 * 3,
                           span_bytes(g.N - n0, kb, g.ldb, 1));
        }
        rSA = make_rsrc((const char *)a.SFA + (int64_t)m0 * a.ldsfa + k_lo / 32, scale_span(g.M - m0, nblk, a.ldsfa));
        rSB = make_rsrc((const char *)a.SFB + (int64_t)n0 * a.ldsfb + k_lo / 32, scale_span(g.N - n0, nblk, a.ldsfb));
    };
    tile_resources(q);
    const __amdgpu_buffer_rsrc_t rZ = make_rsrc(p.A, 0u);

    // Operand loads: chunk position c = (4 j + wave) * 64 + lane of a slot
    // is row c / 6, logical chunk (c % 6) ^ (row bit 3); the K offset goes
    // in the scalar offset (PACKED: the chunk is at c * 16 of the tile's
    // image, the image offset in the scalar offset).  Scale loads: lane L of
    // wave w brings row 64 w + L's 16 bytes.
    constexpr int TSTEP = PACKED ? SLOT : ROWB;        // bytes from one K tile to the next
    uint32_t a_off[LPW], b_off[LPW];
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
        const int c = (4 * j + wave) * 64 + lane;
        const int row = c / 6, chunk = (c % 6) ^ ((row >> 3) & 1);
        a_off[j] = PACKED ? (uint32_t)c * 16 : (uint32_t)(row * p.lda) + chunk * 16;
        b_off[j] = PACKED ? (uint32_t)c * 16 : (uint32_t)(row * p.ldb) + chunk * 16;
    }
    auto dma = [&](__amdgpu_buffer_rsrc_t r, int lds, uint32_t voff, int soff) __attribute__((always_inline)) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(smem + lds), 16, voff,
                                                 soff, 0, 0);
    };
    // load k (0 .. 11) of tile t into ring slot `slot`: A instruction k, or
    // B instruction k - 6
    auto fetch = [&](int t, int k, int slot) __attribute__((always_inline)) {
        const bool isa = k < LPW;
        const int j = isa ? k : k - LPW;
        const __amdgpu_buffer_rsrc_t r = t < nk ? (isa ? rA : rB) : rZ;
        const uint32_t voff = isa ? a_off[j] : b_off[j];
        const int lds = (isa ? A_BASE : B_BASE) + slot * SLOT + (j * 4 + wave) * IB;
        dma(r, lds, voff, t * TSTEP);
    };
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

    // Fragment reads: lane l reads bytes 24 q .. 24 q + 23 (q = l / 16) of
    // row l % 16 of each block as 8-byte units 3 q + s, s = 0, 1, 2: unit u
    // is half u % 2 of logical chunk u / 2.
    const int fr = lane & 15, fq = lane >> 4;
    auto unit = [&](int u) { return fr * ROWB + (((u >> 1) ^ (fr >> 3)) << 4) + (u & 1) * 8; };
    // (through an empty asm: block and slot offsets then fold into the LDS
    // reads' immediate offsets)
    int la0 = A_BASE + wm * WTM * ROWB + unit(3 * fq), la1 = A_BASE + wm * WTM * ROWB + unit(3 * fq + 1),
        la2 = A_BASE + wm * WTM * ROWB + unit(3 * fq + 2);
    int lb0 = B_BASE + wn * WTN * ROWB + unit(3 * fq), lb1 = B_BASE + wn * WTN * ROWB + unit(3 * fq + 1),
        lb2 = B_BASE + wn * WTN * ROWB + unit(3 * fq + 2);
    asm volatile("" : "+v"(la0), "+v"(la1), "+v"(la2), "+v"(lb0), "+v"(lb1), "+v"(lb2));
    constexpr int GB = 16 * ROWB;                      // bytes of a block's 16 rows
    auto ld24 = [&](int a0, int a1, int a2) __attribute__((always_inline)) {
        const u32x2 x = *(const u32x2 *)(smem + a0), y = *(const u32x2 *)(smem + a1),
                    z = *(const u32x2 *)(smem + a2);
        return u32x6{x[0], x[1], y[0], y[1], z[0], z[1]};
    };

    f32x4 acc[TM][TN];
    u32x6 fa[TM], fx;                                  // A fragments; fx: row 7 of odd tiles
    u32x6 fb[2][TN];                                   // B fragments by tile parity
    uint32_t sa[2][2], sb[2][2];                       // scale registers by tile parity

    // Reads of tile t from ring slot rs; its place in its epoch U = t % 4 is
    // a compile-time constant at every call site (the loop advances by whole
    // epochs), so register buffers are chosen by constant parity.
    auto read_a = [&](auto uc, auto ic, int rs) __attribute__((always_inline)) {
        constexpr int P = decltype(uc)::value & 1, I = decltype(ic)::value;
        const int o = rs * SLOT + I * GB;
        const u32x6 v = ld24(la0 + o, la1 + o, la2 + o);
        if constexpr (I < TM - 1 || !P)
            fa[I] = v;
        else
            fx = v;
    };
    auto read_b = [&](auto uc, auto jc, int rs) __attribute__((always_inline)) {
        constexpr int P = decltype(uc)::value & 1, J = decltype(jc)::value;
        const int o = rs * SLOT + J * GB;
        fb[P][J] = ld24(lb0 + o, lb1 + o, lb2 + o);
    };
    // Scale registers: as in the fp8 kernel (byte u of register h' = block
    // row 4 h' + u, K block q of tile U at byte 4 U + q of the row's 16),
    // assembled with two v_perm 8 MFMAs after their dword reads.
    const uint32_t sel_lo = (uint32_t)fq | ((uint32_t)(fq + 4) << 8) | 0x0c0c0000u;   // 0x0c: a zero byte
    const uint32_t sel_hi = 0x00000c0cu | ((uint32_t)fq << 16) | ((uint32_t)(fq + 4) << 24);
    uint32_t sraw[2][4];
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
            mfma_mx6_acc<I % 4, J % 4, FMT>(acc[I][J], fa[I], fb[P][J], sa[P][I / 4], sb[P][J / 4]);
        else
            mfma_mx6_acc<I % 4, J % 4, FMT>(acc[I][J], fx, fb[P][J], sa[P][I / 4], sb[P][J / 4]);
        __builtin_amdgcn_sched_barrier(0);
    };
    // Window t (U = t % 4, tile t in slot rs): MFMAs of tile t - 1 (unless
    // FIRST), reads of tile t -- B block j at MFMA 4 j, A row 7 at MFMA 3 and
    // row i - 1 during row i, scales read at MFMAs 34 .. 46 and assembled 8
    // MFMAs later -- loads of tile t + 2 at every fifth MFMA from MFMA 2 on
    // (issued back to back, a wave's 12 loads held up its MFMAs: 5-6 %
    // slower at 8192^3) into the slot tile t - 1 held (its fragments were
    // read in window t - 1), the next epoch's scales when U == 2; then a
    // wait for the loads of tile t + 1 (everything but the 12 just issued).
    auto window = [&](auto first, auto uc, int t, int rs) __attribute__((always_inline)) {
        constexpr bool F = decltype(first)::value;
        constexpr int U = decltype(uc)::value;
        const int ws = rs == 0 ? NS - 1 : rs - 1;      // (rs + 2) % 3
        if constexpr (U == 2) fetch_scales((t >> 2) + 1);
        static_for<0, 64>([&](auto qc) __attribute__((always_inline)) {
            constexpr int Q = decltype(qc)::value;
            if constexpr (!F) mfma(std::integral_constant<int, (U + 1) & 1>(), qc);
            if constexpr (Q >= 2 && (Q - 2) % 5 == 0 && (Q - 2) / 5 < 2 * LPW) fetch(t + 2, (Q - 2) / 5, ws);
            if constexpr (Q < 32 && Q % 4 == 0) read_b(uc, std::integral_constant<int, Q / 4>(), rs);
            if constexpr (Q == 3) read_a(uc, std::integral_constant<int, TM - 1>(), rs);
            if constexpr (Q >= 8 && Q % 8 == 3) read_a(uc, std::integral_constant<int, Q / 8 - 1>(), rs);
            if constexpr (Q >= 42 && Q <= 54 && Q % 4 == 2) {
                constexpr int c = (Q - 42) / 4;
                scale_finish(uc, std::integral_constant<int, c>(), std::integral_constant<int, c % 2>());
            }
            if constexpr (Q >= 34 && Q <= 46 && Q % 4 == 2) {
                constexpr int c = (Q - 34) / 4;
                scale_issue(uc, std::integral_constant<int, c>(), std::integral_constant<int, c % 2>(), t);
            }
        });
        wait_vmcnt<2 * LPW>();
        wait_lgkmcnt0();
        if constexpr (U == 2) {
            if (rem != 0 && (t >> 2) + 1 == nep - 1)
                mx_scale_tail_fixup(smem, SA_BASE + ((nep - 1) & 1) * SS + wave * IB,
                                    SB_BASE + ((nep - 1) & 1) * SS + wave * IB, lane_id(), rem);
        }
        barrier();
    };

    // tile 0 (slot 0), the first epoch's scales, tile 1 (slot 1), for the
    // current output tile (nk > 0); wv: the wave index (a persistent kernel
    // passes it through an empty asm, so these loads' LDS destinations are
    // computed here)
    // (operands computed into locals first: see the build notes on
    // conditional expressions as arguments of the direct-to-LDS load)
    auto prologue_loads = [&](int wv) __attribute__((always_inline)) {
        const int l = lane_id();
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int k = 0; k < 2 * LPW; ++k) {
                const bool isa = k < LPW;
                const int j = isa ? k : k - LPW;
                const __amdgpu_buffer_rsrc_t r = t < nk ? (isa ? rA : rB) : rZ;
                const uint32_t voff = isa ? a_off[j] : b_off[j];
                const int lds = (isa ? A_BASE : B_BASE) + t * SLOT + (j * 4 + wv) * IB;
                dma(r, lds, voff, t * TSTEP);
            }
            if (t == 0) {
                const uint32_t va = (uint32_t)((64 * wv + l) * q.ldsfa), vb = (uint32_t)((64 * wv + l) * q.ldsfb);
                dma(rSA, SA_BASE + wv * IB, va, 0);
                dma(rSB, SB_BASE + wv * IB, vb, 0);
            }
        }
    };
    // PERSIST: this wave's D staging area, in ring slot 2 (the next tile's
    // first loads use slots 0 and 1)
    float *stage = (float *)(smem + (wave < 2 ? A_BASE : B_BASE) + 2 * SLOT + (wave & 1) * 16 * (WTN + 4) * 4);
    static_assert(2 * 16 * (WTN + 4) * 4 <= SLOT, "staging areas");
    constexpr int D_STORES = (WTM / 16) * (16 * WTN / 4 / 64);

    if (nk > 0) {
        prologue_loads(wave);
        wait_vmcnt<2 * LPW>();                         // all but tile 1's loads
        if (rem != 0 && nep == 1) mx_scale_tail_fixup(smem, SA_BASE + wave * IB, SB_BASE + wave * IB, lane_id(), rem);
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
            window(std::true_type(), std::integral_constant<int, 0>(), 0, 0);
            // windows 1 .. (nk rounded up to a multiple of 4): tiles 0 .. nk - 1
            // computed, then zero tiles
            int rs = 1;
            auto next = [](int r) { return r == NS - 1 ? 0 : r + 1; };
            for (int t = 1; t <= nk; t += 4) {
                window(std::false_type(), std::integral_constant<int, 1>(), t, rs);
                rs = next(rs);
                window(std::false_type(), std::integral_constant<int, 2>(), t + 1, rs);
                rs = next(rs);
                window(std::false_type(), std::integral_constant<int, 3>(), t + 2, rs);
                rs = next(rs);
                window(std::false_type(), std::integral_constant<int, 0>(), t + 3, rs);
                rs = next(rs);
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
                    asm volatile("" : "+s"(wv));
                    prologue_loads(wv);
                }
            }
            epilogue_rows16_vec<OUT_BF16, TM, TN, DAUX>(acc, stage, lane, wm, wn, dm0, dn0, r.g.M, r.g.N, r.g.D,
                                                        r.g.ldd);
            if (!more) break;
            // the next tile's loads (26 per lane) then 64 D stores were issued:
            // at most 63 in flight means every load has landed
            static_assert(D_STORES >= 63, "vmcnt");
            wait_vmcnt<63>();
            wait_lgkmcnt0();
            if (rem != 0 && nep == 1)
                mx_scale_tail_fixup(smem, SA_BASE + wave * IB, SB_BASE + wave * IB, lane_id(), rem);
            barrier();                                 // staging reads done before the ring refills slot 2
        }
    }
}

}  // namespace tg
