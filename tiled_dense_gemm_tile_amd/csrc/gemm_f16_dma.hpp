// Tiled D = A.B + C for 16-bit inputs with 16-byte-aligned rows, gfx950.
//
//   * Global->LDS tile loads are direct (buffer_load_dwordx4 ... lds): one
//     wave instruction moves 64 x 16 bytes straight into 1 KiB of LDS, so no
//     VGPRs hold tiles in flight and no ds_write is issued.  The XOR swizzle
//     is applied on the global side: lane L of an instruction lands on
//     physical chunk L mod CPR of its LDS row and so fetches logical chunk
//     (L mod CPR) ^ swz(row).  Out-of-range rows and K chunks read as zero.
//   * Separate prefetch rings for the A and B tiles in LDS: NA slots for A
//     (prefetch distance SA = NA - 1) and NB slots for B (distance SB =
//     NB - 1).  Tile t lives in A slot t mod NA and B slot t mod NB.  Right
//     after the barrier that opens tile t the fetches of B(t + SB) and then
//     A(t + SA) are issued, each into the slot tile t - 1 used, whose reads
//     every wave completed before that barrier.  With SB = 1, SA = 2 only half
//     of a tile (B) must land within one tile's compute; A gets two.  With
//     SA = SB = S >= 2 (small tiles, where LDS holds deeper rings) both get S
//     tiles, and the loads of S - 1 tiles stay in flight across every
//     barrier.  One barrier per K tile.
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

// acc[i][j][r0 .. r0 + QR) += cq for part q = Q of a TM x TN block grid
// (16 / QR parts per block), selected at run time among the static indices.
template <int TN, int QR, int Q, int NQ, class Acc>
__device__ __forceinline__ void add_part(Acc &acc, const float *cq, int q) {
    if constexpr (Q < NQ) {
        if (q == Q) {
            constexpr int blk = Q / (16 / QR), r0 = (Q % (16 / QR)) * QR;
#pragma unroll
            for (int u = 0; u < QR; ++u) acc[blk / TN][blk % TN][r0 + u] += cq[u];
            return;
        }
        add_part<TN, QR, Q + 1, NQ>(acc, cq, q);
    }
}

template <int BM_, int BN_, int BK_, int WM_, int WN_, int NA_, int NB_>
struct DmaCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, NA = NA_, NB = NB_;
    static constexpr int NT = WM * WN * 64;
};

// LB: bytes each lane moves per global->LDS instruction: 16 (rows 16-byte
// aligned) or 4 (rows only 4-byte aligned; K even).
template <class Cfg, bool FP16, bool OUT_BF16, int LB>
__global__ void __launch_bounds__(Cfg::NT) gemm_f16_dma_kernel(F16Args p, F16Epi e) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NA = Cfg::NA, NB = Cfg::NB;
    constexpr int WM = Cfg::WM, WN = Cfg::WN, NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int KK = BK / 16;                        // MFMA K steps per tile
    constexpr int ROWB = BK * 2, CPR = ROWB / 16;
    constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
    constexpr int IB = 64 * LB;                        // LDS bytes one load instruction fills
    constexpr int RPI = IB / ROWB;                     // rows one load instruction fills
    constexpr int A_INST = A_BYTES / IB / NW;          // load instructions per wave per tile
    constexpr int B_INST = B_BYTES / IB / NW;
    constexpr int LPW = A_INST + B_INST;
    constexpr int SA = NA - 1, SB = NB - 1;            // prefetch distances
    // loads still in flight at a tile barrier: those issued after the newest
    // fetch the next tile needs (see the issue order below)
    constexpr int WAIT_N = SB == 1 ? (SA - SB) * A_INST : (SB - 1) * LPW;
    constexpr int B_BASE = NA * A_BYTES;               // B ring follows the A ring
    constexpr int RING_BYTES = NA * A_BYTES + NB * B_BYTES;
    constexpr int EPI_BYTES = epilogue_lds_bytes(NW, WTN);
    constexpr int LDS_BYTES = RING_BYTES > EPI_BYTES ? RING_BYTES : EPI_BYTES;
    static_assert(LB == 16 || LB == 4, "lane bytes");
    static_assert(A_BYTES % (IB * NW) == 0 && B_BYTES % (IB * NW) == 0 && RPI >= 1, "load tiling");
    static_assert(SB == 1 ? (SA == 1 || SA == 2) : SA == SB, "ring depths");
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

    // Lane L of a load instruction fills LDS bytes [L*LB, L*LB + LB) of the
    // instruction's IB bytes: row L*LB / ROWB, physical chunk p, byte q of
    // the chunk; it fetches the same bytes of logical chunk p ^ swz(row).
    // Global offsets exclude the K offset; kel is the first K element.
    const int lrow = (lane * LB) / ROWB, lp = ((lane * LB) % ROWB) / 16, lq = (lane * LB) % 16;
    auto chunk_of = [&](int j) {
        const int row = (j * NW + wave) * RPI + lrow;
        return lp ^ swz<CPR>(row);
    };
    constexpr int NOFF = LB == 16 ? (A_INST > B_INST ? A_INST : B_INST) : 1;
    uint32_t a_goff[NOFF], b_goff[NOFF];
    int kel[NOFF];
    if constexpr (LB == 16) {
#pragma unroll
        for (int j = 0; j < NOFF; ++j) {
            const int row = (j * NW + wave) * RPI + lrow;
            const int c = chunk_of(j);
            a_goff[j] = (uint32_t)(row * p.lda * 2) + c * 16;
            b_goff[j] = (uint32_t)(row * p.ldb * 2) + c * 16;
            kel[j] = c * 8;
        }
    } else {
        a_goff[0] = (uint32_t)((wave * RPI + lrow) * p.lda * 2) + lq;
        b_goff[0] = (uint32_t)((wave * RPI + lrow) * p.ldb * 2) + lq;
    }
    // offset of instruction j (K element k0 onward) or kOOB past K
    auto goff = [&](const uint32_t *base, int64_t ld, int j, int k0) -> uint32_t {
        if constexpr (LB == 16) {
            return (k0 + kel[j] < K) ? base[j] + (uint32_t)k0 * 2 : kOOB;
        } else {
            const int c = chunk_of(j);
            const int k = k0 + c * 8 + lq / 2;
            const uint32_t o = base[0] + (uint32_t)(j * NW * RPI * ld * 2) + c * 16 + (uint32_t)k0 * 2;
            return k < K ? o : kOOB;
        }
    };

    auto fetchA = [&](int t) {
        const int k0 = t * BK;
        char *sA = smem + (t % NA) * A_BYTES;
#pragma unroll
        for (int j = 0; j < A_INST; ++j) {
            const uint32_t off = goff(a_goff, p.lda, j, k0);
            dma_load<LB>(rA, sA + (j * NW + wave) * IB, off);
        }
    };
    auto fetchB = [&](int t) {
        const int k0 = t * BK;
        char *sB = smem + B_BASE + (t % NB) * B_BYTES;
#pragma unroll
        for (int j = 0; j < B_INST; ++j) {
            const uint32_t off = goff(b_goff, p.ldb, j, k0);
            dma_load<LB>(rB, sB + (j * NW + wave) * IB, off);
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

    // C is streamed into the accumulators during the K loop so the epilogue
    // only writes D: C "part" q (QR accumulator registers of one 32x32 block
    // per lane) is loaded at the transition into tile q + 1, ahead of that
    // transition's B fetch, so the next barrier's wait covers it, and added
    // right after that wait.  With fewer than NQ + 2 tiles, or with deep
    // rings (the wait no longer covers the previous transition's loads), the
    // epilogue adds C.
    constexpr int QR = (TM * TN * 16 / 32) > 4 ? (TM * TN * 16 / 32) : 4;
    constexpr int NQ = TM * TN * 16 / QR;
    constexpr int OS = OUT_BF16 ? 2 : 4;
    const int nk = (K + BK - 1) / BK;
    const bool hasC = p.C != nullptr;
    const bool c_loop = SB == 1 && hasC && nk >= NQ + 2;
    const __amdgpu_buffer_rsrc_t rC =
        make_rsrc(hasC ? (const char *)p.C + (int64_t)m0 * p.ldc * OS : (const char *)p.D,
                  hasC ? span_bytes(M - m0, N, p.ldc, OS) : 0u);
    float cq[QR];
    auto load_c_part = [&](int q) {                    // inactive parts read nothing (zeros)
        const bool act = c_loop && q < NQ;
        const int qq = act ? q : 0;
        const int blk = qq / (16 / QR), r0 = (qq % (16 / QR)) * QR;
        const int i = blk / TN, j = blk % TN;
        const int col = n0 + wn * WTN + j * 32 + fr;
#pragma unroll
        for (int u = 0; u < QR; ++u) {
            const int r = r0 + u;
            const int row = wm * WTM + i * 32 + 8 * (r >> 2) + 4 * fh + (r & 3);
            const uint32_t off = (act && col < N) ? (uint32_t)(row * p.ldc + col) * OS : kOOB;
            if constexpr (OUT_BF16)
                cq[u] = __builtin_bit_cast(float, (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rC, off, 0, 0) << 16);
            else
                cq[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rC, off, 0, 0));
        }
    };
    auto add_c_part = [&](int q) {
        if (c_loop && q >= 0 && q < NQ) add_part<TN, QR, 0, NQ>(acc, cq, q);
    };

    // The rings always fetch once per tile; fetches of tiles past the end
    // read nothing (every chunk is out of range), write zeros into a slot no
    // later tile uses, and keep the loads in flight at every tile barrier at
    // exactly WAIT_N.  SB = 1: the B fetch of the next tile (with the C part
    // before it) is the newest load that must have landed, and only the A
    // fetch issued after it may still run.  SA = SB = S: fetches go out in
    // (B, A) pairs, tile after tile (S pairs before the first barrier, one
    // after each), so the next tile's pair is followed by S - 1 newer pairs.
    if (nk > 0) {
        fetchB(0);
        fetchA(0);
        if constexpr (SB == 1) {
            if constexpr (SA == 2) fetchA(1);
        } else {
#pragma unroll
            for (int u = 1; u < SB; ++u) {
                fetchB(u);
                fetchA(u);
            }
        }
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
            add_c_part(t - 1);
            barrier();
            if constexpr (SB == 1) load_c_part(t);
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
    epilogue_lds<OUT_BF16, TM, TN, WTM, WTN>(acc, smem, wave, lane, wm, wn, m0, n0, M, N, c_loop ? nullptr : p.C,
                                             p.ldc, p.D, p.ldd, e);
}

}  // namespace tg
