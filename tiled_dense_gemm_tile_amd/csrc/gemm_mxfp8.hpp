// Block-scaled fp8 tiled D = A.B + C on gfx950:
//     a(m,k) = e4m3(A[m][k]) * 2^(SFA[m][k/32] - 127)
//     b(k,n) = e4m3(B[n][k]) * 2^(SFB[n][k/32] - 127)
// with v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 operands, one e8m0 scale per
// lane per operand), fp32 accumulators in registers.
//
// Same structure as the 16-bit direct-to-LDS kernel: a K tile is 128 fp8
// elements (one 128-byte row chunked and XOR-swizzled in 16-byte units),
// A and B tiles arrive by buffer_load ... lds into rings of NS slots (the
// tile NS - 1 ahead is fetched), one barrier per K tile, fragments
// software-pipelined, LDS-staged epilogue.
//
// Operand placement (measured on gfx950 with one-hot operands): in a
// 32 x 32 x 64 MFMA, bytes 0-15 of a lane form half of the first 32-wide K
// block and bytes 16-31 half of the second; lane half h (lanes 32h .. 32h+31)
// holds K sub-range [16h, 16h + 16) of each block.  The scale register of
// lane i (row i) applies to the first block and that of lane 32 + i to the
// second; op_sel picks the byte.  Step kk of a 128-wide K tile takes blocks
// 2kk and 2kk + 1, so lane half h reads 16-byte chunks 4kk + h and
// 4kk + 2 + h of its row, and supplies the scale of block 2kk + h.
//
// Scales ride with the B fetch: each tile's scale bytes for its 256 (or
// 128) rows of A and of B, 4 bytes per row (the four 32-wide K blocks of
// the tile), are brought into LDS with dword loads.  This needs K % 128 == 0
// and 4-byte aligned scale rows; the host routes other cases elsewhere.
#pragma once

#include "common.hpp"
#include "gemm_f16.hpp"
#include "pipeline.hpp"

namespace tg {

struct MxArgs {
    F16Args g;           // A, B (e4m3 bytes), C, D, leading dims, sizes, tile grid
    const void *SFA;
    const void *SFB;
    int64_t ldsfa, ldsfb;
    int kb_shift = 0;    // scale block width = 32 << kb_shift (general kernel only; the tiled kernels take 0)
};

template <int BM_, int BN_, int WM_, int WN_, int NS_ = 2>
struct MxCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NS = NS_;
    static constexpr int NT = WM * WN * 64;
};

template <int SEL>
__device__ __forceinline__ f32x16 mfma_mx(const i32x8 &a, const i32x8 &b, const f32x16 &c, uint32_t sa,
                                          uint32_t sb) {
    // operand formats 0/0 = e4m3 / e4m3; op_sel picks byte SEL of each scale register
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, SEL, (int)sa, SEL, (int)sb);
}

template <class Cfg, bool OUT_BF16>
__global__ void __launch_bounds__(Cfg::NT) gemm_mxfp8_kernel(MxArgs q, F16Epi e) {
    const F16Args &p = q.g;
    constexpr int BM = Cfg::BM, BN = Cfg::BN, WM = Cfg::WM, WN = Cfg::WN, NW = WM * WN, NS = Cfg::NS;
    constexpr int BK = 128;                            // fp8 elements per K tile = bytes per row
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int KK = BK / 64;                        // MFMA K steps per tile
    constexpr int ROWB = BK, CPR = ROWB / 16;
    constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
    constexpr int SA_BYTES = BM * 4, SB_BYTES = BN * 4; // scale rows: 4 blocks per K tile
    constexpr int RPI = 1024 / ROWB;
    constexpr int A_INST = A_BYTES / 1024 / NW;
    constexpr int B_INST = B_BYTES / 1024 / NW;
    constexpr int NSI = (BM + BN) / 64;                // scale load instructions per tile (whole group)
    constexpr int A_BASE = 0, B_BASE = NS * A_BYTES, S_BASE = B_BASE + NS * B_BYTES;
    constexpr int S_SLOT = SA_BYTES + SB_BYTES;
    constexpr int RING_BYTES = S_BASE + NS * S_SLOT;
    constexpr int EPI_BYTES = epilogue_lds_bytes(NW, WTN);
    constexpr int LDS_BYTES = RING_BYTES > EPI_BYTES ? RING_BYTES : EPI_BYTES;
    static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "load tiling");
    static_assert(BM % 64 == 0 && BN % 64 == 0, "scale load tiling");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");
    static_assert(KK == 2, "fragment double buffer parity");
    static_assert(NS >= 2, "ring depth");

    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tmi, tni;
    tile_order(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tmi, tni);
    const int m0 = tmi * BM, n0 = tni * BN;
    const int M = p.M, N = p.N, K = p.K;
    const int nblk = K / 32;

    const __amdgpu_buffer_rsrc_t rA =
        make_rsrc((const char *)p.A + (int64_t)m0 * p.lda, span_bytes(M - m0, K, p.lda, 1));
    const __amdgpu_buffer_rsrc_t rB =
        make_rsrc((const char *)p.B + (int64_t)n0 * p.ldb, span_bytes(N - n0, K, p.ldb, 1));
    const __amdgpu_buffer_rsrc_t rSA =
        make_rsrc((const char *)q.SFA + (int64_t)m0 * q.ldsfa, span_bytes(M - m0, nblk, q.ldsfa, 1));
    const __amdgpu_buffer_rsrc_t rSB =
        make_rsrc((const char *)q.SFB + (int64_t)n0 * q.ldsfb, span_bytes(N - n0, nblk, q.ldsfb, 1));

    uint32_t a_goff[A_INST], b_goff[B_INST];
    {
        const int lrow = lane / CPR, lchunk = lane % CPR;
#pragma unroll
        for (int j = 0; j < A_INST; ++j) {
            const int row = (j * NW + wave) * RPI + lrow;
            a_goff[j] = (uint32_t)(row * p.lda) + ((lchunk ^ swz<CPR>(row)) << 4);
        }
#pragma unroll
        for (int j = 0; j < B_INST; ++j) {
            const int row = (j * NW + wave) * RPI + lrow;
            b_goff[j] = (uint32_t)(row * p.ldb) + ((lchunk ^ swz<CPR>(row)) << 4);
        }
    }
    // K % 128 == 0: every chunk of a tile before K is in range, every chunk of
    // a tile at or past K is not.
    auto fetchA = [&](int t) {
        const int k0 = t * BK;
        char *s = smem + A_BASE + (t % NS) * A_BYTES;
#pragma unroll
        for (int j = 0; j < A_INST; ++j) {
            const uint32_t off = k0 < K ? a_goff[j] + (uint32_t)k0 : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rA, (__attribute__((address_space(3))) void *)(s + (j * NW + wave) * 1024), 16, off, 0, 0, 0);
        }
    };
    auto fetchB = [&](int t) {
        const int k0 = t * BK;
        char *s = smem + B_BASE + (t % NS) * B_BYTES;
#pragma unroll
        for (int j = 0; j < B_INST; ++j) {
            const uint32_t off = k0 < K ? b_goff[j] + (uint32_t)k0 : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rB, (__attribute__((address_space(3))) void *)(s + (j * NW + wave) * 1024), 16, off, 0, 0, 0);
        }
        // scale rows of this tile: 4 bytes (blocks 4t .. 4t+3) per row of A and of B
        char *ss = smem + S_BASE + (t % NS) * S_SLOT;
        const bool kin = k0 < K;
#pragma unroll
        for (int j = wave; j < NSI; j += NW) {
            // (offsets are computed into locals: an inline conditional as a
            // builtin argument makes the host pass drop the kernel)
            if (j < BM / 64) {
                const int row = j * 64 + lane;
                const uint32_t off = kin ? (uint32_t)(row * q.ldsfa) + (uint32_t)(t * 4) : kOOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rSA, (__attribute__((address_space(3))) void *)(ss + j * 256), 4, off, 0, 0, 0);
            } else {
                const int row = (j - BM / 64) * 64 + lane;
                const uint32_t off = kin ? (uint32_t)(row * q.ldsfb) + (uint32_t)(t * 4) : kOOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rSB, (__attribute__((address_space(3))) void *)(ss + SA_BYTES + (j - BM / 64) * 256), 4, off,
                    0, 0, 0);
            }
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

    i32x8 fa[2][TM], fb[2][TN];
    uint32_t sa[2][TM], sb[2][TN];                     // scale bytes of step (buffer) kk
    auto ld32 = [&](const char *base, int off0, int off1) {
        const u32x4 lo = *(const u32x4 *)(base + off0);
        const u32x4 hi = *(const u32x4 *)(base + off1);
        i32x8 v;
        v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
        v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
        return v;
    };
    // Operands of step kk of tile t into buffer kk: chunks 4kk + fh and
    // 4kk + 2 + fh of each row, and the row's scale dword (the tile's four
    // blocks) shifted so byte 2kk is block 2kk + fh (op_sel 2kk picks it).
    auto load_step = [&](int kk, int t) {
        const char *sA = smem + A_BASE + (t % NS) * A_BYTES;
        const char *sB = smem + B_BASE + (t % NS) * B_BYTES;
        const char *ss = smem + S_BASE + (t % NS) * S_SLOT;
        const int c0 = ((4 * kk + fh) ^ fswz) << 4, c1 = ((4 * kk + 2 + fh) ^ fswz) << 4;
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[kk][i] = ld32(sA + a_frag + i * 32 * ROWB, c0, c1);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[kk][j] = ld32(sB + b_frag + j * 32 * ROWB, c0, c1);
#pragma unroll
        for (int i = 0; i < TM; ++i)
            sa[kk][i] = *(const uint32_t *)(ss + 4 * (wm * WTM + i * 32 + fr)) >> (8 * fh);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            sb[kk][j] = *(const uint32_t *)(ss + SA_BYTES + 4 * (wn * WTN + j * 32 + fr)) >> (8 * fh);
    };
    auto mfmas = [&](int kk) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if (kk == 0)
                    acc[i][j] = mfma_mx<0>(fa[0][i], fb[0][j], acc[i][j], sa[0][i], sb[0][j]);
                else
                    acc[i][j] = mfma_mx<2>(fa[1][i], fb[1][j], acc[i][j], sa[1][i], sb[1][j]);
            }
    };
    // Spread the next step's LDS reads over the current step's MFMAs.
    auto interleave = [&]() {
        constexpr int NDS = 2 * (TM + TN) + TM + TN, NMF = TM * TN;
        if constexpr (NMF >= NDS) {
#pragma unroll
            for (int g = 0; g < NDS; ++g) {
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, NMF / NDS, 0);
            }
        } else {
#pragma unroll
            for (int g = 0; g < NMF; ++g) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, NDS / NMF, 0);
            }
        }
    };

    // Rings: A and B NS slots each (prefetch distance S = NS - 1), scales
    // with B.  Fetches go out one tile at a time (B with its scales, then A):
    // S tiles before the first barrier, one after each.  A tile barrier waits
    // until only the S - 1 newest tiles' fetches may still be in flight, so
    // the tile it opens has landed; the slot refilled after it held the tile
    // whose last reads finished before it.  A fetch past the last tile reads
    // nothing and fills a slot no later tile uses.  A wave's loads per tile
    // depend on how many of the scale loads fall to it.
    constexpr int NSI_LO = NSI / NW, NSI_HI = (NSI + NW - 1) / NW;
    constexpr int WAIT_LO = (NS - 2) * (A_INST + B_INST + NSI_LO);
    constexpr int WAIT_HI = (NS - 2) * (A_INST + B_INST + NSI_HI);
    auto wait_ring = [&]() {
        if (wave < NSI % NW)
            wait_vmcnt<WAIT_HI>();
        else
            wait_vmcnt<WAIT_LO>();
    };
    const int nk = K / BK;
    if (nk > 0) {
        fetchB(0);
        fetchA(0);
#pragma unroll
        for (int u = 1; u < NS - 1; ++u) {
            fetchB(u);
            fetchA(u);
        }
        wait_ring();
        wait_lgkmcnt0();
        barrier();
        fetchB(NS - 1);
        fetchA(NS - 1);
        load_step(0, 0);
        for (int t = 0; t + 1 < nk; ++t) {
            load_step(1, t);
            mfmas(0);
            interleave();
            wait_ring();
            wait_lgkmcnt0();
            barrier();
            fetchB(t + NS);
            fetchA(t + NS);
            load_step(0, t + 1);
            mfmas(1);
            interleave();
        }
        load_step(1, nk - 1);
        mfmas(0);
        mfmas(1);
    }

    wait_vmcnt<0>();
    wait_lgkmcnt0();
    barrier();
    epilogue_lds<OUT_BF16, TM, TN, WTM, WTN>(acc, smem, wave, lane, wm, wn, m0, n0, M, N, p.C, p.ldc, p.D, p.ldd, e);
}

}  // namespace tg
