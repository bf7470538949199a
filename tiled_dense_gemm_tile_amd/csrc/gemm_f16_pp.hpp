// Ping-pong schedule for D = A.B + C with 16-bit inputs whose rows are
// 16-byte aligned (K a multiple of 8), gfx950.
//
// The workgroup computes a 256 x 256 output tile with 8 waves, two per SIMD,
// split into two groups of four (one wave of each group per SIMD).  Group g
// owns output rows [128 g, 128 g + 128) of the tile; wave s of a group owns
// columns [64 s, 64 s + 64): 4 x 2 blocks of 32 x 32 accumulators (MS = 32,
// v_mfma_f32_32x32x16) or 8 x 4 blocks of 16 x 16 (MS = 16,
// v_mfma_f32_16x16x32).  Both do the same work per K tile; the 16x16 form
// draws less power per flop on random data, so the clock holds higher.
//
// Time is cut into phases separated by workgroup barriers.  In every phase
// one group is in its "memory" phase -- it issues direct global->LDS loads
// for later K tiles and reads ALL fragments of its next K tile from LDS into
// registers -- while the other group is in its "compute" phase and issues
// nothing but the 32 MFMAs of one K tile.  The groups swap at each barrier,
// so each SIMD's matrix pipe is fed by one of its two waves at all times and
// no MFMA waits on a fragment read: group 0 computes K tile t in phase 2t,
// group 1 in phase 2t + 1.
//
// LDS holds three rings: the two 128-row halves of the A tile separately
// (two slots each, 16 KiB a slot) and the B tile (three slots, 32 KiB) --
// 160 KiB in all.  Half h of A is read only by group h, in one phase, so its
// slot frees a phase earlier than B's, which both groups read.  Loads are
// issued by the group that does not read them next:
//   group 0, memory phase of tile t:  A half 1 of tile t + 1, B of tile t + 2
//   group 1, memory phase of tile t:  A half 0 of tile t + 2
// giving every load three (A) or four (B) phases to land.  Each wave waits
// on its own loads (s_waitcnt vmcnt) before the barrier that opens the phase
// in which they are read; loads return in issue order, so the waits are fixed
// counts.  Fetches past K read nothing (offsets out of range give zeros) and
// keep those counts constant through the last tiles.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "gemm_f16.hpp"
#include "pipeline.hpp"

namespace tg {

// Keep the compiler's scheduler from moving any instruction (MFMAs
// included) across a phase boundary.
__device__ __forceinline__ void phase_fence() { __builtin_amdgcn_sched_barrier(0); }

template <int N>
__device__ __forceinline__ void phase_end() {
    phase_fence();
    wait_vmcnt<N>();
    wait_lgkmcnt0();
    barrier();
    phase_fence();
}

template <int MS, bool FP16, bool OUT_BF16>
__global__ void __launch_bounds__(512) gemm_f16_pp_kernel(F16Args p, F16Epi e) {
    static_assert(MS == 32 || MS == 16, "MFMA block size");
    constexpr int BK = 64, KS = MS == 32 ? 16 : 32, KK = BK / KS;   // K per MFMA, MFMA steps per tile
    constexpr int WTM = 128, WTN = 64, TM = WTM / MS, TN = WTN / MS;
    constexpr int ROWB = BK * 2, CPR = ROWB / 16;
    constexpr int AH_BYTES = 128 * ROWB;               // one half of the A tile
    constexpr int B_BYTES = 256 * ROWB;
    constexpr int A0_BASE = 0, A1_BASE = 2 * AH_BYTES, B_BASE = 4 * AH_BYTES;
    constexpr int RING_BYTES = B_BASE + 3 * B_BYTES;
    constexpr int EPI_BYTES = epilogue_lds_bytes(8, WTN);
    constexpr int LDS_BYTES = RING_BYTES > EPI_BYTES ? RING_BYTES : EPI_BYTES;
    constexpr int IB = 1024;                           // LDS bytes one load instruction fills
    // loads per wave: group 0 issues 4 (A half 1) + 8 (B) per tile, group 1 4 (A half 0)
    constexpr int G0_A = 4, G0_B = 8, G1_A = 4;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");

    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches
    const int g = wave >> 2, s = wave & 3;
    int tmi, tni;
    tile_order(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tmi, tni);
    const int m0 = tmi * 256, n0 = tni * 256;
    const int M = p.M, N = p.N, K = p.K;

    const __amdgpu_buffer_rsrc_t rA =
        make_rsrc((const char *)p.A + (int64_t)m0 * p.lda * 2, span_bytes(M - m0, K, p.lda, 2));
    const __amdgpu_buffer_rsrc_t rB =
        make_rsrc((const char *)p.B + (int64_t)n0 * p.ldb * 2, span_bytes(N - n0, K, p.ldb, 2));

    // Load instruction j of wave s fills LDS rows (4 j + s) * 8 + lrow of its
    // ring slot: lane L writes physical chunk L % 8 of row L / 8 and fetches
    // logical chunk (L % 8) ^ swz(row), which is the same for every j.
    const int lrow = lane >> 3;
    // 32x32 fragment reads use swz<8>, 16x16 ones swz16 (bank-conflict free
    // for each read pattern); rows (4 j + s) * 8 + lrow give the same chunk for every j.
    const int chunk = (lane & 7) ^ (MS == 32 ? swz<CPR>(s * 8 + lrow) : swz16(lrow));
    const int kel = chunk * 8;                          // first K element of this lane's chunk
    const int a_row0 = g == 0 ? 128 : 0;                // group 0 loads half 1, group 1 half 0
    uint32_t a_off[4], b_off[8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        a_off[j] = (uint32_t)((a_row0 + (4 * j + s) * 8 + lrow) * p.lda * 2) + chunk * 16;
#pragma unroll
    for (int j = 0; j < 8; ++j) b_off[j] = (uint32_t)(((4 * j + s) * 8 + lrow) * p.ldb * 2) + chunk * 16;

    char *const a_fill = smem + (g == 0 ? A1_BASE : A0_BASE);
    auto fetch_a = [&](int t) {                         // this group's A half-tile loads of K tile t
        const int k0 = t * BK;
        const uint32_t oob = (uint32_t)(k0 + kel >= K) << 31;   // offsets stay below 2^31
        char *dst = a_fill + (t & 1) * AH_BYTES + s * IB;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t off = (a_off[j] + (uint32_t)k0 * 2) | oob;
            dma_load<16>(rA, dst + j * 4 * IB, off);
        }
    };
    auto fetch_b = [&](int t) {                         // group 0 only
        const int k0 = t * BK;
        const uint32_t oob = (uint32_t)(k0 + kel >= K) << 31;
        char *dst = smem + B_BASE + (t % 3) * B_BYTES + s * IB;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t off = (b_off[j] + (uint32_t)k0 * 2) | oob;
            dma_load<16>(rB, dst + j * 4 * IB, off);
        }
    };

    // Fragment reads: lane l reads row l % MS of each block and 16-byte chunk
    // KK-step * (KS / 8) + l / MS of that row (its 8 K elements).
    const int fr = lane % MS, fq = lane / MS;
    const int fswz = MS == 32 ? swz<CPR>(fr) : swz16(fr);   // the same for every block (MS rows apart)
    const char *const a_read = smem + (g == 0 ? A0_BASE : A1_BASE) + fr * ROWB;
    const char *const b_read = smem + B_BASE + (s * WTN + fr) * ROWB;

    typedef typename std::conditional<MS == 32, f32x16, f32x4>::type AccT;
    constexpr int AR = MS == 32 ? 16 : 4;              // accumulator registers per block
    AccT acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < AR; ++r) acc[i][j][r] = 0.0f;

    u32x4 fa[KK][TM], fb[KK][TN];
    auto read_frags = [&](int t) {                      // every fragment of K tile t
        const char *sA = a_read + (t & 1) * AH_BYTES;
        const char *sB = b_read + (t % 3) * B_BYTES;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int coff = ((kk * (KS / 8) + fq) ^ fswz) << 4;
#pragma unroll
            for (int i = 0; i < TM; ++i) fa[kk][i] = *(const u32x4 *)(sA + i * MS * ROWB + coff);
#pragma unroll
            for (int j = 0; j < TN; ++j) fb[kk][j] = *(const u32x4 *)(sB + j * MS * ROWB + coff);
        }
    };
    auto compute = [&]() {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    if constexpr (MS == 32)
                        acc[i][j] = mfma_32x32x16<FP16>(fa[kk][i], fb[kk][j], acc[i][j]);
                    else
                        acc[i][j] = mfma_16x16x32<FP16>(fa[kk][i], fb[kk][j], acc[i][j]);
                }
    };

    const int nk = (K + BK - 1) / BK;
    if (nk > 0) {
        if (g == 0) {
            // issue order B(0) A1(0) B(1) | A1(1) B(2) | A1(2) B(3) | ...
            fetch_b(0);
            fetch_a(0);
            fetch_b(1);
            phase_end<G0_A + G0_B>();                  // B(0) landed
            fetch_a(1);                                // memory phase of tile 0
            fetch_b(2);
            read_frags(0);
            phase_end<G0_B + G0_A + G0_B>();           // A1(0) landed
            for (int t = 0; t < nk; ++t) {
                compute();                             // compute phase of tile t
                phase_end<G0_A + G0_B>();              // B(t + 1) landed
                fetch_a(t + 2);                        // memory phase of tile t + 1
                fetch_b(t + 3);
                if (t + 1 < nk) read_frags(t + 1);
                phase_end<G0_B + G0_A + G0_B>();       // A1(t + 1) landed
            }
        } else {
            fetch_a(0);
            fetch_a(1);
            phase_end<G1_A>();                         // A0(0) landed
            phase_end<G1_A>();                         // (group 0 reads tile 0)
            for (int t = 0; t < nk; ++t) {
                fetch_a(t + 2);                        // memory phase of tile t
                read_frags(t);
                phase_end<G1_A>();                     // A0(t + 1) landed
                compute();                             // compute phase of tile t
                phase_end<G1_A>();
            }
        }
    }

    // ---- epilogue: D = acc + C, staged through LDS ------------------------
    wait_vmcnt<0>();                                   // no load still writing a slot
    wait_lgkmcnt0();
    barrier();
    if constexpr (MS == 32)
        epilogue_lds<OUT_BF16, TM, TN, WTM, WTN>(acc, smem, wave, lane, g, s, m0, n0, M, N, p.C, p.ldc, p.D, p.ldd, e);
    else
        epilogue_lds16<OUT_BF16, TM, TN, WTM, WTN>(acc, smem, wave, lane, g, s, m0, n0, M, N, p.C, p.ldc, p.D, p.ldd,
                                                   e);
}

}  // namespace tg
