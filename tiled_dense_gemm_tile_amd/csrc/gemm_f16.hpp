// Tiled D = A.B + C for 16-bit inputs (bf16 / fp16) on gfx950.
//
// Structure of one workgroup (one BM x BN output tile):
//   1. tile_order() maps the workgroup id to a tile (row-major tiles, XCD-aware
//      order);
//   2. a K loop over BK-wide K tiles.  Global->LDS tile loads run one K tile
//      ahead of the MFMAs (a prefetch ring of two LDS slots, with the next
//      tile held in VGPRs while the current one is consumed);
//   3. MFMA v_mfma_f32_32x32x16_{bf16,f16} on fragments read from the
//      swizzled LDS layout, fp32 accumulators held in registers;
//   4. an epilogue that adds C, converts and stores D with predicated
//      buffer stores.
// Remainders of M, N and K are predicated through buffer-resource range
// checks (rows past the end) and explicit out-of-range offsets (K and N
// past the end inside an in-range row).
#pragma once

#include "common.hpp"

namespace tg {

struct F16Args {
    const void *A;
    const void *B;
    const void *C;
    void *D;
    int64_t lda, ldb, ldc, ldd;
    int M, N, K;
    int tiles_m, tiles_n, group_m;
    // split-K (kernels instantiated with SPLIT only): K is cut into ranges
    // of `kt_split` K tiles; split s writes its fp32 partial tile to the
    // M x ldw matrix at ws + s * M * ldw (C and D are left to the reduction)
    int kt_split = 0;
    float *ws = nullptr;
    int64_t ldw = 0;
};

template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int NT = WM * WN * 64;
};

template <bool FP16>
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (FP16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// One 16x16x32 MFMA: lane l holds row (A) / column (B) l % 16 and K
// elements 8*(l/16) .. 8*(l/16)+7; accumulator register r of lane l is
// row 4*(l/16) + r, column l % 16 of the 16x16 block.
template <bool FP16>
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (FP16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// A global vector of VEC 16-bit elements.
template <int VEC> struct GVec;
template <> struct GVec<8> {
    typedef u32x4 T;
    static __device__ __forceinline__ T load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
};
template <> struct GVec<4> {
    typedef u32x2 T;
    static __device__ __forceinline__ T load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    }
};
template <> struct GVec<2> {
    typedef uint32_t T;
    static __device__ __forceinline__ T load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    }
};
template <> struct GVec<1> {
    typedef uint16_t T;
    static __device__ __forceinline__ T load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
    }
};

template <class Cfg, int VEC, bool FP16, bool OUT_BF16>
__global__ void __launch_bounds__(Cfg::NT) gemm_f16_kernel(F16Args p) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
    constexpr int WM = Cfg::WM, WN = Cfg::WN, NT = Cfg::NT;
    constexpr int WTM = BM / WM, WTN = BN / WN;        // wave tile
    constexpr int TM = WTM / 32, TN = WTN / 32;        // 32x32 MFMA blocks per wave
    constexpr int ROWB = BK * 2;                       // LDS row bytes
    constexpr int CPR = ROWB / 16;                     // 16-byte chunks per row
    constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
    constexpr int SLOT = A_BYTES + B_BYTES;
    constexpr int VPR = BK / VEC;                      // global vectors per tile row
    constexpr int ROWS_PER_PASS = NT / VPR;            // rows one pass of all threads covers
    constexpr int A_PASSES = BM / ROWS_PER_PASS, B_PASSES = BN / ROWS_PER_PASS;
    constexpr int OS = OUT_BF16 ? 2 : 4;               // output element size
    static_assert(NT % VPR == 0 && BM % ROWS_PER_PASS == 0 && BN % ROWS_PER_PASS == 0, "load tiling");
    static_assert(TM >= 1 && TN >= 1 && BK % 16 == 0, "wave tiling");
    typedef typename GVec<VEC>::T VT;

    __shared__ __attribute__((aligned(16))) char smem[2 * SLOT];

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

    // ---- global -> register -> LDS tile movement ----------------------
    const int ld_kv = tid % VPR;                       // vector index along K (fixed per thread)
    const int ld_row = tid / VPR;                      // first row this thread loads
    const uint32_t a_row_off = (uint32_t)(ld_row * p.lda * 2);
    const uint32_t b_row_off = (uint32_t)(ld_row * p.ldb * 2);
    const uint32_t a_pass_off = (uint32_t)(ROWS_PER_PASS * p.lda * 2);
    const uint32_t b_pass_off = (uint32_t)(ROWS_PER_PASS * p.ldb * 2);
    // LDS byte offset of this thread's vector inside a row (swizzled chunk)
    const int kbyte = ld_kv * VEC * 2;
    uint32_t lds_off[A_PASSES > B_PASSES ? A_PASSES : B_PASSES];
#pragma unroll
    for (int i = 0; i < (A_PASSES > B_PASSES ? A_PASSES : B_PASSES); ++i) {
        const int r = ld_row + i * ROWS_PER_PASS;
        lds_off[i] = r * ROWB + (((kbyte >> 4) ^ swz<CPR>(r)) << 4) + (kbyte & 15);
    }

    VT ra[A_PASSES], rb[B_PASSES];
    auto load_tile = [&](int t) {
        const int k = t * BK + ld_kv * VEC;
        const bool kin = k < K;
        const uint32_t koff = (uint32_t)k * 2;
#pragma unroll
        for (int i = 0; i < A_PASSES; ++i)
            ra[i] = GVec<VEC>::load(rA, kin ? a_row_off + i * a_pass_off + koff : kOOB);
#pragma unroll
        for (int i = 0; i < B_PASSES; ++i)
            rb[i] = GVec<VEC>::load(rB, kin ? b_row_off + i * b_pass_off + koff : kOOB);
    };
    auto store_tile = [&](int slot) {
        char *sA = smem + slot * SLOT;
        char *sB = sA + A_BYTES;
#pragma unroll
        for (int i = 0; i < A_PASSES; ++i) *(VT *)(sA + lds_off[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < B_PASSES; ++i) *(VT *)(sB + lds_off[i]) = rb[i];
    };

    // ---- MFMA fragments ------------------------------------------------
    const int wm = wave / WN, wn = wave % WN;
    const int fr = lane & 31, fh = lane >> 5;          // fragment row, K half
    const int a_frag = (wm * WTM + fr) * ROWB;
    const int b_frag = (wn * WTN + fr) * ROWB;
    const int fswz = swz<CPR>(fr);                     // same for every 32-row block

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    auto compute = [&](int slot) {
        const char *sA = smem + slot * SLOT;
        const char *sB = sA + A_BYTES;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int coff = (((kk * 2 + fh) ^ fswz) << 4);
            u32x4 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) af[i] = *(const u32x4 *)(sA + a_frag + i * 32 * ROWB + coff);
#pragma unroll
            for (int j = 0; j < TN; ++j) bfr[j] = *(const u32x4 *)(sB + b_frag + j * 32 * ROWB + coff);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma_32x32x16<FP16>(af[i], bfr[j], acc[i][j]);
        }
    };

    // ---- K loop: fetch tile t+1 while tile t is multiplied --------------
    const int nk = (K + BK - 1) / BK;
    if (nk > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();
    for (int t = 0; t < nk; ++t) {
        const bool more = t + 1 < nk;
        if (more) load_tile(t + 1);
        compute(t & 1);
        if (more) store_tile((t + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: D = acc + C ------------------------------------------
    const __amdgpu_buffer_rsrc_t rD =
        make_rsrc((char *)p.D + (int64_t)m0 * p.ldd * OS, span_bytes(M - m0, N, p.ldd, OS));
    const bool hasC = p.C != nullptr;
    const __amdgpu_buffer_rsrc_t rC =
        make_rsrc(hasC ? (const char *)p.C + (int64_t)m0 * p.ldc * OS : (const char *)p.D,
                  hasC ? span_bytes(M - m0, N, p.ldc, OS) : 0u);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int col = n0 + wn * WTN + j * 32 + fr;
        const bool cin = col < N;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * WTM + i * 32 + 8 * (r >> 2) + 4 * fh + (r & 3);  // tile-relative
                const uint32_t doff = cin ? (uint32_t)(row * p.ldd + col) * OS : kOOB;
                float v = acc[i][j][r];
                if (hasC) {
                    const uint32_t coff = cin ? (uint32_t)(row * p.ldc + col) * OS : kOOB;
                    if constexpr (OUT_BF16) {
                        uint32_t cb = __builtin_amdgcn_raw_buffer_load_b16(rC, coff, 0, 0);
                        v += __builtin_bit_cast(float, cb << 16);
                    } else {
                        v += __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rC, coff, 0, 0));
                    }
                }
                if constexpr (OUT_BF16)
                    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(v), rD, doff, 0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rD, doff, 0, 0);
            }
        }
    }
}

}  // namespace tg
