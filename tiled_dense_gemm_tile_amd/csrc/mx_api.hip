// C ABI of the tiled GEMM library, block-scaled fp8 inputs: argument
// validation, kernel selection and launch on the caller's stream.  The
// declarations and their contract are in include/tilegemm.h.
#include <stdlib.h>

#include "api.hpp"
#include "transpose.hpp"
#include "mx_any_api.hpp"
#include "mx_launch.hpp"

using namespace tg_api;

namespace {

// Test override: TILEGEMM_MX_CONFIG=<id> forces one configuration where
// the call's alignment allows it (read at every call).
int forced_mx_cfg() {
    const char *e = getenv("TILEGEMM_MX_CONFIG");
    if (!e || !*e) return -1;
    const int id = atoi(e);
    return (id >= 0 && id < tg::kNumMxCfgs) ? id : -1;
}

gemm_status dispatch_mx(const Common &a, const void *SFA, int64_t ldsfa, const void *SFB, int64_t ldsfb,
                        hipStream_t s) {
    // The kernel streams 16-byte A/B chunks and 4-byte scale words per K tile of 128.
    const bool fast = a.K % 128 == 0 && (uintptr_t)a.A % 16 == 0 && (uintptr_t)a.B % 16 == 0 && a.lda % 16 == 0 &&
                      a.ldb % 16 == 0 && (uintptr_t)SFA % 4 == 0 && (uintptr_t)SFB % 4 == 0 && ldsfa % 4 == 0 &&
                      ldsfb % 4 == 0;
    // other K % 32 and alignments: the general kernel
    if (!fast && a.K > 0) return run_mx_any(a, 0, a.lda, a.ldb, SFA, ldsfa, SFB, ldsfb, s);
    // The four-wave kernel loads a row's scales 16 bytes (512 K) at a time,
    // so it needs 16-byte-aligned scale rows and whole groups of 16 blocks.
    const bool scales16 = a.K % 512 == 0 && (uintptr_t)SFA % 16 == 0 && (uintptr_t)SFB % 16 == 0 &&
                          ldsfa % 16 == 0 && ldsfb % 16 == 0;
    int cfg = forced_mx_cfg();
    if ((cfg == tg::kMxFourWave || cfg == tg::kMxFourWavePersist) && !scales16) cfg = -1;
    if (cfg < 0) {
        // the four-wave kernel once its 256 x 256 grid is over half a wave
        // (measured at K = 4096: 160 tiles 46.9 against 71.3 us with
        // 128 x 128 tiles; at 128 tiles 128 x 128 is 2 % ahead)
        const int64_t t256 = tiles_of(a, 256, 256), t128 = tiles_of(a, 128, 128);
        if (scales16 && t256 > 128)
            cfg = tg::kMxFourWavePersist;             // (persistent when the grid is over one wave, below)
        else if (t256 >= 240)
            cfg = tg::kMxWide;
        else if (t128 > 256)
            cfg = tg::kMx128;                           // two workgroups per CU share the waves
        else if (t128 > 128)
            cfg = tg::kMxDeep128;                       // at most one 128 x 128 tile per CU: three-slot rings
        else
            cfg = tg::kMxDeep64;                        // (2048 x 2048 x 8192: 43.8 against 59.3 us;
                                                        //  1024 x 1024 x 8192 in 64 x 64 tiles: 23.2 against 37.4)
    }
    tg::MxArgs q;
    q.g.A = a.A;
    q.g.B = a.B;
    q.g.C = a.C;
    q.g.D = a.D;
    q.g.lda = a.lda;
    q.g.ldb = a.ldb;
    q.g.ldc = a.ldc;
    q.g.ldd = a.ldd;
    q.g.M = (int)a.M;
    q.g.N = (int)a.N;
    q.g.K = (int)a.K;
    q.g.group_m = 4;
    q.g.tiles_m = (int)((a.M + tg::kMxCfgs[cfg].bm - 1) / tg::kMxCfgs[cfg].bm);
    q.g.tiles_n = (int)((a.N + tg::kMxCfgs[cfg].bn - 1) / tg::kMxCfgs[cfg].bn);
    // K == 0 reads no scales: any valid address stands in for NULL ones
    q.SFA = SFA ? SFA : a.D;
    q.SFB = SFB ? SFB : a.D;
    q.ldsfa = ldsfa;
    q.ldsfb = ldsfb;
    const int64_t tiles = (int64_t)q.g.tiles_m * q.g.tiles_n;
    if (tiles >= kMaxDim) return GEMM_ERR_UNSUPPORTED;
    const bool bf16 = a.out_type == GEMM_OUT_BF16;
    const int os = bf16 ? 2 : 4;
    const uintptr_t vb = (uintptr_t)os * 4;
    tg::F16Epi e;
    e.vec_d = ((uintptr_t)a.D % vb) == 0 && a.ldd % 4 == 0;
    e.vec_c = a.C && ((uintptr_t)a.C % vb) == 0 && a.ldc % 4 == 0;
    if (cfg == tg::kMxFourWavePersist) {
        // persistent over grids of more than one workgroup per CU, without C
        // and with D rows of whole 16-byte segments (its epilogue's stores)
        const int cus = cu_count(s);
        if (!a.C && e.vec_d && a.N % 4 == 0 && cus > 0 && tiles > cus)
            return launched(bf16 ? tg::launch_mx_persist<true>((unsigned)cus, s, q, e)
                                 : tg::launch_mx_persist<false>((unsigned)cus, s, q, e));
        cfg = tg::kMxFourWave;
    }
    return launched(bf16 ? tg::launch_mx<true>(cfg, (unsigned)tiles, s, q, e)
                         : tg::launch_mx<false>(cfg, (unsigned)tiles, s, q, e));
}

// Checks of a gemm_mxfp8 call beyond the shared ones.
// lda_min / ldb_min: as validate (MN-contiguous operands: M, N).
gemm_status validate_mx8(const Common &a, const void *SFA, int64_t ldsfa, const void *SFB, int64_t ldsfb,
                         bool *none, int64_t lda_min = -1, int64_t ldb_min = -1) {
    gemm_status st = validate(a, none, lda_min, ldb_min);
    if (st != GEMM_OK || *none) return st;
    if (a.K > 0) {
        if (ldsfa < a.K / 32 || ldsfb < a.K / 32) return GEMM_ERR_BAD_LD;
        if (!SFA || !SFB) return GEMM_ERR_NULL_POINTER;
    }
    if (a.K % 32 != 0) return GEMM_ERR_UNSUPPORTED;
    if (ldsfa >= kMaxLdBytes || ldsfb >= kMaxLdBytes) return GEMM_ERR_UNSUPPORTED;
    return GEMM_OK;
}

// Split-K: the four-wave kernel per (K range of whole scale epochs, tile),
// then the reduction.  Calls the four-wave kernel cannot take run unsplit.
gemm_status run_mx8_splitk(const Common &a, const void *SFA, int64_t ldsfa, const void *SFB, int64_t ldsfb,
                           int splits, void *ws, size_t ws_bytes, hipStream_t s) {
    bool none = false;
    gemm_status st = validate_mx8(a, SFA, ldsfa, SFB, ldsfb, &none);
    if (st != GEMM_OK || none) return st;
    if (splits < 0 || splits > kMaxSplits) return GEMM_ERR_UNSUPPORTED;
    const int S = effective_splits(a.K, splits == 0 ? auto_splits(a.M, a.N, a.K) : splits, 512);
    const bool four_wave = a.K % 512 == 0 && (uintptr_t)a.A % 16 == 0 && (uintptr_t)a.B % 16 == 0 &&
                           a.lda % 16 == 0 && a.ldb % 16 == 0 && (uintptr_t)SFA % 16 == 0 &&
                           (uintptr_t)SFB % 16 == 0 && ldsfa % 16 == 0 && ldsfb % 16 == 0;
    if (S == 1 || !four_wave) return dispatch_mx(a, SFA, ldsfa, SFB, ldsfb, s);
    st = check_workspace(a, S, ws, ws_bytes);
    if (st != GEMM_OK) return st;
    tg::MxArgs q;
    q.g.A = a.A;
    q.g.B = a.B;
    q.g.C = nullptr;
    q.g.D = nullptr;
    q.g.lda = a.lda;
    q.g.ldb = a.ldb;
    q.g.ldc = 0;
    q.g.ldd = 0;
    q.g.M = (int)a.M;
    q.g.N = (int)a.N;
    q.g.K = (int)a.K;
    q.g.group_m = 4;
    q.g.tiles_m = (int)((a.M + 255) / 256);
    q.g.tiles_n = (int)((a.N + 255) / 256);
    const int64_t epochs = a.K / 512;
    q.g.kt_split = (int)((epochs + S - 1) / S);
    q.g.ws = (float *)ws;
    q.g.ldw = splitk_ldw(a.N);
    q.SFA = SFA;
    q.SFB = SFB;
    q.ldsfa = ldsfa;
    q.ldsfb = ldsfb;
    const int64_t grid = (int64_t)q.g.tiles_m * q.g.tiles_n * S;
    if (grid >= kMaxDim) return GEMM_ERR_UNSUPPORTED;
    tg::F16Epi e;
    e.vec_c = false;
    e.vec_d = true;                                    // 256-byte aligned base, ldw % 4 == 0
    hipError_t err = tg::launch_mx_split((unsigned)grid, s, q, e);
    if (err != hipSuccess) return launched(err);
    return reduce_splits(a, ws, S, s);
}

}  // namespace

extern "C" {

gemm_status gemm_mxfp8(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *SFA, int64_t ldsfa,
                       const void *B, int64_t ldb, const void *SFB, int64_t ldsfb, const void *C, int64_t ldc,
                       void *D, int64_t ldd, int out_type, hipStream_t stream) {
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 1};
    bool none = false;
    gemm_status st = validate_mx8(a, SFA, ldsfa, SFB, ldsfb, &none);
    if (st != GEMM_OK || none) return st;
    return dispatch_mx(a, SFA, ldsfa, SFB, ldsfb, stream);
}

gemm_status gemm_mxfp8_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int a_order,
                          const void *SFA, int64_t ldsfa, const void *B, int64_t ldb, int b_order, const void *SFB,
                          int64_t ldsfb, const void *C, int64_t ldc, void *D, int64_t ldd, int out_type,
                          hipStream_t stream) {
    if ((a_order != GEMM_K_CONTIGUOUS && a_order != GEMM_MN_CONTIGUOUS) ||
        (b_order != GEMM_K_CONTIGUOUS && b_order != GEMM_MN_CONTIGUOUS))
        return GEMM_ERR_UNSUPPORTED;
    const bool amn = a_order == GEMM_MN_CONTIGUOUS, bmn = b_order == GEMM_MN_CONTIGUOUS;
    if (!amn && !bmn)
        return gemm_mxfp8(M, N, K, A, lda, SFA, ldsfa, B, ldb, SFB, ldsfb, C, ldc, D, ldd, out_type, stream);
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 1};
    bool none = false;
    gemm_status st = validate_mx8(a, SFA, ldsfa, SFB, ldsfb, &none, amn ? M : -1, bmn ? N : -1);
    if (st != GEMM_OK || none) return st;
    if (K == 0) return dispatch_mx(a, SFA, ldsfa, SFB, ldsfb, stream);
    return run_mx_any(a, 0, lda, ldb, SFA, ldsfa, SFB, ldsfb, stream, amn, bmn);
}

gemm_status gemm_mxfp8_ex_ws(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int a_order,
                             const void *SFA, int64_t ldsfa, const void *B, int64_t ldb, int b_order,
                             const void *SFB, int64_t ldsfb, const void *C, int64_t ldc, void *D, int64_t ldd,
                             int out_type, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if ((a_order != GEMM_K_CONTIGUOUS && a_order != GEMM_MN_CONTIGUOUS) ||
        (b_order != GEMM_K_CONTIGUOUS && b_order != GEMM_MN_CONTIGUOUS))
        return GEMM_ERR_UNSUPPORTED;
    const bool amn = a_order == GEMM_MN_CONTIGUOUS, bmn = b_order == GEMM_MN_CONTIGUOUS;
    if (!workspace || (!amn && !bmn) || K == 0)
        return gemm_mxfp8_ex(M, N, K, A, lda, a_order, SFA, ldsfa, B, ldb, b_order, SFB, ldsfb, C, ldc, D, ldd,
                             out_type, stream);
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 1};
    bool none = false;
    gemm_status st = validate_mx8(a, SFA, ldsfa, SFB, ldsfb, &none, amn ? M : -1, bmn ? N : -1);
    if (st != GEMM_OK || none) return st;
    Common k = a;
    st = k_contiguous_operands(8, a, amn, bmn, workspace, workspace_bytes, stream, &k.A, &k.lda, &k.B, &k.ldb);
    if (st != GEMM_OK) return st;
    return gemm_mxfp8(M, N, K, k.A, k.lda, SFA, ldsfa, k.B, k.ldb, SFB, ldsfb, C, ldc, D, ldd, out_type, stream);
}

gemm_status gemm_mxfp8_splitk(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *SFA,
                              int64_t ldsfa, const void *B, int64_t ldb, const void *SFB, int64_t ldsfb,
                              const void *C, int64_t ldc, void *D, int64_t ldd, int out_type, int splits,
                              void *workspace, size_t workspace_bytes, hipStream_t stream) {
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 1};
    return run_mx8_splitk(a, SFA, ldsfa, SFB, ldsfb, splits, workspace, workspace_bytes, stream);
}

}  // extern "C"
