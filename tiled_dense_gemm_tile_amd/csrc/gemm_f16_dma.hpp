// Tiled D = A.B + C for 16-bit inputs with 16-byte-aligned rows, gfx950.
//
//   * Global->LDS tile loads are direct (buffer_load_dwordx4 ... lds): one
//     wave instruction moves 64 x 16 bytes straight into 1 KiB of LDS, so no
//     VGPRs hold tiles in flight and no ds_write is issued.  The XOR swizzle
//     is applied on the global side: lane L of an instruction lands on
//     physical chunk L mod CPR of its LDS row and so fetches logical chunk
//     (L mod CPR) ^ swz(row).  Out-of-range rows and K chunks read as zero.
//   * Separate prefetch rings for the A and B tiles in LDS: NA slots for A
//     (prefetch distance SA = NA - 1) and NB = 2 slots for B (distance 1).
//     Tile t lives in A slot t mod NA and B slot t mod 2.  Right after the
//     barrier that opens tile t the fetches of B(t + 1) and then A(t + SA) are
//     issued, each into the slot tile t - 1 used, whose reads every wave
//     completed before that barrier.  With SA = 2 only half of a tile (B) must
//     land within one tile's compute; A gets two.  One barrier per K tile.
//   * Fragments are software-pipelined: while the MFMAs of K step kk run, the
//     fragments of step kk + 1 are read from LDS; the last step's MFMAs are
//     issued after the next tile's barrier so the matrix pipe restarts at once.
//   * Epilogue through LDS: each wave stages 32 rows of its accumulators at a
//     time and writes D (and reads C) as whole 16-byte row segments.
#pragma once

#include "common.hpp"
#include "gemm_f16.hpp"
#include "pipeline.hpp"

namespace tg {

template <int BM_, int BN_, int BK_, int WM_, int WN_, int NA_, int NB_>
struct DmaCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, NA = NA_, NB = NB_;
    static constexpr int NT = WM * WN * 64;
};

template <class Cfg, bool FP16, bool OUT_BF16>
__global__ void __launch_bounds__(Cfg::NT) gemm_f16_dma_kernel(F16Args p, F16Epi e) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NA = Cfg::NA, NB = Cfg::NB;
    constexpr int WM = Cfg::WM, WN = Cfg::WN, NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int KK = BK / 16;                        // MFMA K steps per tile
    constexpr int ROWB = BK * 2, CPR = ROWB / 16;
    constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
    constexpr int RPI = 1024 / ROWB;                   // rows one load instruction fills
    constexpr int A_INST = A_BYTES / 1024 / NW;        // load instructions per wave per tile
    constexpr int B_INST = B_BYTES / 1024 / NW;
    constexpr int LPW = A_INST + B_INST;
    constexpr int SA = NA - 1, SB = NB - 1;            // prefetch distances
    constexpr int WAIT_N = (SA - SB) * A_INST;         // loads still in flight at a tile barrier
    constexpr int B_BASE = NA * A_BYTES;               // B ring follows the A ring
    constexpr int RING_BYTES = NA * A_BYTES + NB * B_BYTES;
    constexpr int EPI_BYTES = epilogue_lds_bytes(NW, WTN);
    constexpr int LDS_BYTES = RING_BYTES > EPI_BYTES ? RING_BYTES : EPI_BYTES;
    static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "load tiling");
    static_assert(SB == 1 && (SA == 1 || SA == 2), "ring depths");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");
    static_assert(KK % 2 == 0, "fragment double buffer parity");

    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    int tmi, tni;
    tile_order(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tmi, tni);
    const int m0 = tmi * BM, n0 = tni * BN;
    const int M = p.M, N = p.N, K = p.K;

    const __amdgpu_buffer_rsrc_t rA =
        make_rsrc((const char *)p.A + (int64_t)m0 * p.lda * 2, span_bytes(M - m0, K, p.lda, 2));
    const __amdgpu_buffer_rsrc_t rB =
        make_rsrc((const char *)p.B + (int64_t)n0 * p.ldb * 2, span_bytes(N - n0, K, p.ldb, 2));

    // Per-lane global offsets (without the K offset) and the first K element
    // of each lane's chunk, for every load instruction of this wave.
    uint32_t a_goff[A_INST], b_goff[B_INST];
    int a_kel[A_INST], b_kel[B_INST];
    {
        const int lrow = lane / CPR, lchunk = lane % CPR;
#pragma unroll
        for (int j = 0; j < A_INST; ++j) {
            const int row = (j * NW + wave) * RPI + lrow;
            const int c = lchunk ^ swz<CPR>(row);
            a_goff[j] = (uint32_t)(row * p.lda * 2) + c * 16;
            a_kel[j] = c * 8;
        }
#pragma unroll
        for (int j = 0; j < B_INST; ++j) {
            const int row = (j * NW + wave) * RPI + lrow;
            const int c = lchunk ^ swz<CPR>(row);
            b_goff[j] = (uint32_t)(row * p.ldb * 2) + c * 16;
            b_kel[j] = c * 8;
        }
    }

    auto fetchA = [&](int t) {
        const int k0 = t * BK;
        char *sA = smem + (t % NA) * A_BYTES;
#pragma unroll
        for (int j = 0; j < A_INST; ++j) {
            const uint32_t off = (k0 + a_kel[j] < K) ? a_goff[j] + (uint32_t)k0 * 2 : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rA, (__attribute__((address_space(3))) void *)(sA + (j * NW + wave) * 1024), 16, off, 0, 0, 0);
        }
    };
    auto fetchB = [&](int t) {
        const int k0 = t * BK;
        char *sB = smem + B_BASE + (t % NB) * B_BYTES;
#pragma unroll
        for (int j = 0; j < B_INST; ++j) {
            const uint32_t off = (k0 + b_kel[j] < K) ? b_goff[j] + (uint32_t)k0 * 2 : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rB, (__attribute__((address_space(3))) void *)(sB + (j * NW + wave) * 1024), 16, off, 0, 0, 0);
        }
    };

    const int wm = wave / WN, wn = wave % WN;
    const int fr = lane & 31, fh = lane >> 5;
    const int a_frag = (wm * WTM + fr) * ROWB;
    const int b_frag = (wn * WTN + fr) * ROWB;
    const int fswz = swz<CPR>(fr);

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    u32x4 fa[2][TM], fb[2][TN];
    auto load_frags = [&](int buf, int t, int kk) {
        const char *sA = smem + (t % NA) * A_BYTES;
        const char *sB = smem + B_BASE + (t % NB) * B_BYTES;
        const int coff = (((kk * 2 + fh) ^ fswz) << 4);
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[buf][i] = *(const u32x4 *)(sA + a_frag + i * 32 * ROWB + coff);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[buf][j] = *(const u32x4 *)(sB + b_frag + j * 32 * ROWB + coff);
    };
    auto mfmas = [&](int buf) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = mfma_32x32x16<FP16>(fa[buf][i], fb[buf][j], acc[i][j]);
    };
    // Ask the scheduler to spread the fragment reads of the next step over
    // the MFMAs of the current one.
    auto interleave_ds = [&]() {
        constexpr int NDS = TM + TN, NMF = TM * TN;
        constexpr int PER = NMF / NDS > 0 ? NMF / NDS : 1;
#pragma unroll
        for (int g = 0; g < NDS; ++g) {
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, PER, 0);
        }
        if constexpr (NMF > PER * NDS) __builtin_amdgcn_sched_group_barrier(kSchedMfma, NMF - PER * NDS, 0);
    };

    // Transition region after a tile barrier: restart the matrix pipe with
    // the previous tile's last MFMAs while the next fetch and the next
    // tile's first fragment reads are issued between them.
    auto interleave_transition = [&]() {
        constexpr int NDS = TM + TN, NMF = TM * TN;
        constexpr int G = NMF > LPW ? NMF : LPW;
        constexpr int DS_EVERY = G / NDS > 0 ? G / NDS : 1;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (g < NMF) __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            if (g < LPW) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
            if (g % DS_EVERY == DS_EVERY - 1 && g / DS_EVERY < NDS)
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        if constexpr (NDS > G / DS_EVERY) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, NDS - G / DS_EVERY, 0);
    };
    auto tile_steps = [&](int t) {
#pragma unroll
        for (int kk = 0; kk + 1 < KK; ++kk) {
            load_frags((kk + 1) & 1, t, kk + 1);
            mfmas(kk & 1);
            interleave_ds();
        }
    };

    // The rings always fetch once per tile; fetches of tiles past the end
    // read nothing (every chunk is out of range), write zeros into a slot no
    // later tile uses, and keep the loads in flight at every tile barrier at
    // exactly WAIT_N: the B fetch of the next tile is the newest one that
    // must have landed, and only the A fetch issued after it may still run.
    const int nk = (K + BK - 1) / BK;
    if (nk > 0) {
        fetchB(0);
        fetchA(0);
        if constexpr (SA == 2) fetchA(1);
        wait_vmcnt<WAIT_N>();
        wait_lgkmcnt0();
        barrier();
        fetchB(SB);
        fetchA(SA);
        load_frags(0, 0, 0);
        for (int t = 0; t + 1 < nk; ++t) {
            tile_steps(t);
            wait_vmcnt<WAIT_N>();
            wait_lgkmcnt0();
            barrier();
            fetchB(t + 1 + SB);
            fetchA(t + 1 + SA);
            load_frags(0, t + 1, 0);
            mfmas((KK - 1) & 1);
            interleave_transition();
        }
        tile_steps(nk - 1);
        mfmas((KK - 1) & 1);
    }

    // ---- epilogue: D = acc + C, staged through LDS ------------------------
    wait_vmcnt<0>();                                   // no fetch still writing a slot
    wait_lgkmcnt0();
    barrier();                                         // every wave is done with the tile slots
    epilogue_lds<OUT_BF16, TM, TN, WTM, WTN>(acc, smem, wave, lane, wm, wn, m0, n0, M, N, p.C, p.ldc, p.D, p.ldd, e);
}

}  // namespace tg
