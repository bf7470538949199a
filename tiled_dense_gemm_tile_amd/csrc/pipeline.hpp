// Pieces shared by the direct-to-LDS GEMM kernels: explicit waits, the
// workgroup barrier, scheduling masks and the LDS-staged epilogue.
#pragma once

#include "common.hpp"

namespace tg {

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt low bits [3:0], high bits [15:14]; expcnt and lgkmcnt left at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier that also stops the compiler from moving memory
// accesses across it (the waits before it are issued explicitly).
__device__ __forceinline__ void barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One direct global->LDS load: each lane moves LB bytes from `off` in the
// resource to LDS at lds + lane * LB.
template <int LB>
__device__ __forceinline__ void dma_load(__amdgpu_buffer_rsrc_t r, char *lds, uint32_t off) {
    if constexpr (LB == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, off, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 4, off, 0, 0, 0);
}

// Scheduling masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100, kSchedVmemRead = 0x020;

struct F16Epi {
    bool vec_c, vec_d;   // C / D rows allow full-width vector access
};

// LDS bytes the staged epilogue needs: 32 rows of every wave's tile columns.
constexpr int epilogue_lds_bytes(int nwaves, int wtn) { return nwaves * 32 * (wtn + 8) * 4; }

// D = acc + C for one wave's WTM x WTN block of a tile, in WTM / 32 passes
// (DAUX: cache-policy bits of the D stores)
// of 32 rows.  stage(pass, ep) writes the accumulators of rows
// [32 pass, 32 pass + 32) of the wave block into this wave's private LDS
// area ep (row-major, pitch WTN + PAD floats, PAD chosen by the stager so
// its writes hit disjoint banks); the pass then reads them back as 16-byte
// row segments:
// C is read and D written with whole-vector accesses where the row and
// alignment allow, element-wise at the right edge.
// The caller guarantees every wave is done with the LDS it reuses.
template <bool OUT_BF16, int WTM, int WTN, int PAD, int DAUX = 0, class Stage>
__device__ __forceinline__ void epilogue_lds_passes(Stage &&stage, char *smem, int wave, int lane, int wm, int wn,
                                                    int m0, int n0, int M, int N, const void *C, int64_t ldc,
                                                    void *D, int64_t ldd, F16Epi e) {
    static_assert(PAD <= 8, "stage area");
    constexpr int OS = OUT_BF16 ? 2 : 4;
    constexpr int EP = WTN + PAD;
    float *ep = (float *)smem + wave * 32 * EP;
    const __amdgpu_buffer_rsrc_t rD =
        make_rsrc((char *)D + (int64_t)m0 * ldd * OS, span_bytes(M - m0, N, ldd, OS));
    const bool hasC = C != nullptr;
    const __amdgpu_buffer_rsrc_t rC =
        make_rsrc(hasC ? (const char *)C + (int64_t)m0 * ldc * OS : (const char *)D,
                  hasC ? span_bytes(M - m0, N, ldc, OS) : 0u);
    constexpr int LPR = WTN / 4;                       // lanes per staged row (4 floats each)
    constexpr int RPS = 64 / LPR;                      // rows per read instruction
    const int erow = lane / LPR, ecol = (lane % LPR) * 4;
    const int gcol = n0 + wn * WTN + ecol;             // first output column of this lane
#pragma unroll
    for (int i = 0; i < WTM / 32; ++i) {
        stage(i, ep);
        wait_lgkmcnt0();
#pragma unroll
        for (int q = 0; q < 32 / RPS; ++q) {
            const int lr = q * RPS + erow;             // row inside the 32-row pass
            const f32x4 v = *(const f32x4 *)(ep + lr * EP + ecol);
            const int row = wm * WTM + i * 32 + lr;    // tile-relative row
            const bool rin = m0 + row < M;
            const bool full = rin && gcol + 4 <= N;
            float o[4] = {v[0], v[1], v[2], v[3]};
            if (hasC) {
                if (full && e.vec_c) {
                    const uint32_t coff = (uint32_t)(row * ldc + gcol) * OS;
                    if constexpr (OUT_BF16) {
                        const u32x2 cb = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rC, coff, 0, 0));
                        o[0] += __builtin_bit_cast(float, cb[0] << 16);
                        o[1] += __builtin_bit_cast(float, cb[0] & 0xffff0000u);
                        o[2] += __builtin_bit_cast(float, cb[1] << 16);
                        o[3] += __builtin_bit_cast(float, cb[1] & 0xffff0000u);
                    } else {
                        const f32x4 c4 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rC, coff, 0, 0));
                        o[0] += c4[0];
                        o[1] += c4[1];
                        o[2] += c4[2];
                        o[3] += c4[3];
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const uint32_t coff = (rin && gcol + u < N) ? (uint32_t)(row * ldc + gcol + u) * OS : kOOB;
                        if constexpr (OUT_BF16)
                            o[u] += __builtin_bit_cast(float, (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rC, coff, 0, 0) << 16);
                        else
                            o[u] += __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rC, coff, 0, 0));
                    }
                }
            }
            if (full && e.vec_d) {
                const uint32_t doff = (uint32_t)(row * ldd + gcol) * OS;
                if constexpr (OUT_BF16) {
                    u32x2 pk;
                    pk[0] = pack_bf16x2(o[0], o[1]);
                    pk[1] = pack_bf16x2(o[2], o[3]);
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, pk), rD, doff, 0, DAUX);
                } else {
                    u32x4 pk;
                    pk[0] = __builtin_bit_cast(uint32_t, o[0]);
                    pk[1] = __builtin_bit_cast(uint32_t, o[1]);
                    pk[2] = __builtin_bit_cast(uint32_t, o[2]);
                    pk[3] = __builtin_bit_cast(uint32_t, o[3]);
                    __builtin_amdgcn_raw_buffer_store_b128(pk, rD, doff, 0, DAUX);
                }
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t doff = (rin && gcol + u < N) ? (uint32_t)(row * ldd + gcol + u) * OS : kOOB;
                    if constexpr (OUT_BF16)
                        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(o[u]), rD, doff, 0, DAUX);
                    else
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o[u]), rD, doff, 0, DAUX);
                }
            }
        }
        wait_lgkmcnt0();   // reads of this pass done before the next pass overwrites the stage
    }
}

// Epilogue for 32x32 MFMA accumulators acc[i][j] (lane l, register r holds
// row 8*(r/4) + 4*(l/32) + r%4 and column l%32 of block (i, j)).
template <bool OUT_BF16, int TM, int TN, int WTM, int WTN>
__device__ __forceinline__ void epilogue_lds(const f32x16 (&acc)[TM][TN], char *smem, int wave, int lane, int wm,
                                             int wn, int m0, int n0, int M, int N, const void *C, int64_t ldc,
                                             void *D, int64_t ldd, F16Epi e) {
    static_assert(TM * 32 == WTM && TN * 32 == WTN, "32x32 blocks");
    constexpr int EP = WTN + 8;                        // half-waves 4 rows apart: 32 banks apart
    const int fr = lane & 31, fh = lane >> 5;
    auto stage = [&](int i, float *ep) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                ep[(8 * (r >> 2) + 4 * fh + (r & 3)) * EP + j * 32 + fr] = acc[i][j][r];
    };
    epilogue_lds_passes<OUT_BF16, WTM, WTN, 8>(stage, smem, wave, lane, wm, wn, m0, n0, M, N, C, ldc, D, ldd, e);
}

// Epilogue for 16x16 MFMA accumulators acc[i][j] (lane l, register r holds
// row 4*(l/16) + r and column l%16 of block (i, j)); a pass stages two block rows.
template <bool OUT_BF16, int TM, int TN, int WTM, int WTN, int DAUX = 0>
__device__ __forceinline__ void epilogue_lds16(const f32x4 (&acc)[TM][TN], char *smem, int wave, int lane, int wm,
                                               int wn, int m0, int n0, int M, int N, const void *C, int64_t ldc,
                                               void *D, int64_t ldd, F16Epi e) {
    static_assert(TM * 16 == WTM && TN * 16 == WTN && TM % 2 == 0, "16x16 blocks");
    constexpr int EP = WTN + 4;                        // lane quarters 4 rows apart: 16 banks apart
    const int fc = lane & 15, fq = lane >> 4;
    auto stage = [&](int p, float *ep) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) ep[(16 * h + 4 * fq + r) * EP + j * 16 + fc] = acc[2 * p + h][j][r];
    };
    epilogue_lds_passes<OUT_BF16, WTM, WTN, 4, DAUX>(stage, smem, wave, lane, wm, wn, m0, n0, M, N, C, ldc, D, ldd, e);
}

// D = acc (no C) for one wave's (16 TM) x (16 TN) block of 16x16 MFMA
// accumulators acc[i][j] -- lane l, register r: row 4 (l / 16) + r, column
// l % 16 of block (i, j); with TRANS row l % 16, column 4 (l / 16) + r --
// for the persistent kernels: passes of one block row (16 rows) staged
// through `stage`, this wave's own 16 x (16 TN + 4) floats, and every lane
// stores whole 16-byte (bf16: 8-byte) row segments -- the caller guarantees
// N % 4 == 0, 16-byte-aligned D rows, and segments past M or N get an
// offset beyond the resource, which drops them.  So a pass issues exactly
// 16 / RPS stores per lane whatever the tile's edges (the caller counts them
// to wait for loads issued before the stores).
template <bool OUT_BF16, int TM, int TN, int DAUX, bool TRANS = false>
__device__ __forceinline__ void epilogue_rows16_vec(const f32x4 (&acc)[TM][TN], float *stage, int lane, int wm,
                                                    int wn, int m0, int n0, int M, int N, void *D, int64_t ldd) {
    constexpr int OS = OUT_BF16 ? 2 : 4;
    constexpr int WTM = TM * 16, WTN = TN * 16;
    constexpr int EP = WTN + 4;                        // lane quarters 4 rows apart: 16 banks apart
    constexpr int LPR = WTN / 4;                       // lanes per staged row (4 floats each)
    constexpr int RPS = 64 / LPR;                      // rows per store instruction
    const __amdgpu_buffer_rsrc_t rD =
        make_rsrc((char *)D + (int64_t)m0 * ldd * OS, span_bytes(M - m0, N, ldd, OS));
    // (the lane index passes through an empty asm: in a persistent kernel's
    // tile loop, offsets derived from it would otherwise be hoisted out of
    // the loop and held in registers through the whole main loop)
    asm volatile("" : "+v"(lane));
    const int fc = lane & 15, fq = lane >> 4;
    const int erow = lane / LPR, ecol = (lane % LPR) * 4;
    const int gcol = n0 + wn * WTN + ecol;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        // (one block row's accumulators in flight at a time: the scheduler
        // would otherwise read them all out of the AGPRs at once)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            // (read out of the AGPRs here, at their store: left to the
            // compiler, all of acc is copied to VGPRs at the epilogue's start)
            f32x4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[r]) : "a"(acc[i][j][r]));
            if constexpr (TRANS) {
                *(f32x4 *)(stage + fc * EP + j * 16 + 4 * fq) = v;      // rows EP apart: 4 banks apart
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) stage[(4 * fq + r) * EP + j * 16 + fc] = v[r];
            }
        }
        wait_lgkmcnt0();
#pragma unroll
        for (int q = 0; q < 16 / RPS; ++q) {
            const int lr = q * RPS + erow;
            const f32x4 v = *(const f32x4 *)(stage + lr * EP + ecol);
            const int row = wm * WTM + i * 16 + lr;
            const uint32_t doff = (m0 + row < M && gcol < N) ? (uint32_t)(row * ldd + gcol) * OS : kOOB;
            if constexpr (OUT_BF16) {
                u32x2 pk;
                pk[0] = pack_bf16x2(v[0], v[1]);
                pk[1] = pack_bf16x2(v[2], v[3]);
                __builtin_amdgcn_raw_buffer_store_b64(pk, rD, doff, 0, DAUX);
            } else {
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rD, doff, 0, DAUX);
            }
        }
        wait_lgkmcnt0();   // reads of this pass done before the next pass overwrites the stage
    }
}

// Epilogue for transposed 16x16 MFMA blocks acc[i][j] (lane l, register r
// holds row l % 16 and column 4 (l / 16) + r of block (i, j)); a pass stages
// two block rows, one 16-byte LDS write per block.
template <bool OUT_BF16, int TM, int TN, int WTM, int WTN, int DAUX = 0>
__device__ __forceinline__ void epilogue_lds16t(const f32x4 (&acc)[TM][TN], char *smem, int wave, int lane, int wm,
                                                int wn, int m0, int n0, int M, int N, const void *C, int64_t ldc,
                                                void *D, int64_t ldd, F16Epi e) {
    static_assert(TM * 16 == WTM && TN * 16 == WTN && TM % 2 == 0, "16x16 blocks");
    constexpr int EP = WTN + 4;
    const int fr = lane & 15, fq = lane >> 4;
    auto stage = [&](int p, float *ep) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < TN; ++j) *(f32x4 *)(ep + (16 * h + fr) * EP + j * 16 + 4 * fq) = acc[2 * p + h][j];
    };
    epilogue_lds_passes<OUT_BF16, WTM, WTN, 4, DAUX>(stage, smem, wave, lane, wm, wn, m0, n0, M, N, C, ldc, D, ldd, e);
}

}  // namespace tg
