// C ABI of the tiled GEMM library, block-scaled fp6 inputs: argument
// validation, kernel selection and launch on the caller's stream.  The
// declarations and their contract are in include/tilegemm.h.
#include <stdlib.h>

#include "api.hpp"
#include "transpose.hpp"
#include "mx6_launch.hpp"
#include "mx_any_api.hpp"

using namespace tg_api;

namespace {

// 16-byte A/B rows (lda multiple of 64 elements), 16-byte scale words (512
// K) per row, whole 128-wide K tiles (scale bytes past K cleared)
bool fast_mx6(const Common &a, const void *SFA, int64_t ldsfa, const void *SFB, int64_t ldsfb) {
    return a.K % 128 == 0 && (uintptr_t)a.A % 16 == 0 && (uintptr_t)a.B % 16 == 0 && a.lda % 64 == 0 &&
           a.ldb % 64 == 0 && (uintptr_t)SFA % 16 == 0 && (uintptr_t)SFB % 16 == 0 && ldsfa % 16 == 0 &&
           ldsfb % 16 == 0;
}

// Kernel arguments; a.lda and a.ldb are in elements (multiples of 4), the
// kernel takes them in bytes (three quarters of that).
tg::MxArgs mx6_args(const Common &a, const void *SFA, int64_t ldsfa, const void *SFB, int64_t ldsfb) {
    tg::MxArgs q;
    q.g.A = a.A;
    q.g.B = a.B;
    q.g.C = a.C;
    q.g.D = a.D;
    q.g.lda = a.lda / 4 * 3;
    q.g.ldb = a.ldb / 4 * 3;
    q.g.ldc = a.ldc;
    q.g.ldd = a.ldd;
    q.g.M = (int)a.M;
    q.g.N = (int)a.N;
    q.g.K = (int)a.K;
    q.g.group_m = 4;
    q.g.tiles_m = (int)((a.M + 255) / 256);
    q.g.tiles_n = (int)((a.N + 255) / 256);
    // K == 0 reads no operand or scale: any valid address stands in for NULL ones
    if (!q.g.A) q.g.A = a.D;
    if (!q.g.B) q.g.B = a.D;
    q.SFA = SFA ? SFA : a.D;
    q.SFB = SFB ? SFB : a.D;
    q.ldsfa = ldsfa;
    q.ldsfb = ldsfb;
    return q;
}

// Test override: TILEGEMM_MX6_PERSIST=0 launches one workgroup per tile
// where the persistent kernel would run.
bool persist_allowed() {
    const char *e = getenv("TILEGEMM_MX6_PERSIST");
    return !(e && e[0] == '0');
}

gemm_status dispatch_mx6(const Common &a, bool e3m2, const void *SFA, int64_t ldsfa, const void *SFB, int64_t ldsfb,
                         hipStream_t s) {
    // other K % 32 and alignments: the general kernel
    if (!fast_mx6(a, SFA, ldsfa, SFB, ldsfb) && a.K > 0)
        return run_mx_any(a, e3m2 ? 3 : 2, a.lda / 4 * 3, a.ldb / 4 * 3, SFA, ldsfa, SFB, ldsfb, s);
    const tg::MxArgs q = mx6_args(a, SFA, ldsfa, SFB, ldsfb);
    const int64_t tiles = (int64_t)q.g.tiles_m * q.g.tiles_n;
    if (tiles >= kMaxDim) return GEMM_ERR_UNSUPPORTED;
    const bool bf16 = a.out_type == GEMM_OUT_BF16;
    const int os = bf16 ? 2 : 4;
    const uintptr_t vb = (uintptr_t)os * 4;
    tg::F16Epi e;
    e.vec_d = ((uintptr_t)a.D % vb) == 0 && a.ldd % 4 == 0;
    e.vec_c = a.C && ((uintptr_t)a.C % vb) == 0 && a.ldc % 4 == 0;
    // more tiles than CUs, no C, D rows of whole 16-byte segments: the
    // persistent kernel (TILEGEMM_MX6_PERSIST=0 turns it off)
    const int cus = cu_count(s);
    if (!a.C && e.vec_d && a.N % 4 == 0 && cus > 0 && tiles > cus && persist_allowed())
        return launched(bf16 ? tg::launch_mx6_persist<true>(e3m2, (unsigned)cus, s, q, e)
                             : tg::launch_mx6_persist<false>(e3m2, (unsigned)cus, s, q, e));
    return launched(bf16 ? tg::launch_mx6<true>(e3m2, (unsigned)tiles, s, q, e)
                         : tg::launch_mx6<false>(e3m2, (unsigned)tiles, s, q, e));
}

// Checks of a gemm_mxfp6 call beyond the shared ones (A and B extents in
// bytes: three quarters of the element counts; for K and lda multiples of 4,
// lda < K exactly when the byte counts compare so, and other K or lda are
// unsupported).
// amn / bmn: A / B stored MN-contiguous (leading dimension at least M / N).
gemm_status validate_mx6(const Common &a, int format, const void *SFA, int64_t ldsfa, const void *SFB,
                         int64_t ldsfb, bool *none, bool amn = false, bool bmn = false) {
    *none = false;
    if (format != GEMM_FP6_E2M3 && format != GEMM_FP6_E3M2) return GEMM_ERR_UNSUPPORTED;
    Common bytes = a;
    bytes.K = a.K / 4 * 3;
    bytes.lda = a.lda / 4 * 3;
    bytes.ldb = a.ldb / 4 * 3;
    // (for lda a multiple of 4: lda * 3 / 4 >= ceil(M / 4) * 3 exactly when lda >= M)
    gemm_status st = validate(bytes, none, amn ? (a.M + 3) / 4 * 3 : -1, bmn ? (a.N + 3) / 4 * 3 : -1);
    if (st != GEMM_OK || *none) return st;
    if (a.K >= kMaxDim || a.K % 32 != 0 || a.lda % 4 != 0 || a.ldb % 4 != 0) return GEMM_ERR_UNSUPPORTED;
    if (a.K > 0) {
        if (ldsfa < a.K / 32 || ldsfb < a.K / 32) return GEMM_ERR_BAD_LD;
        if (!SFA || !SFB) return GEMM_ERR_NULL_POINTER;
    }
    if (ldsfa >= kMaxLdBytes || ldsfb >= kMaxLdBytes) return GEMM_ERR_UNSUPPORTED;
    return GEMM_OK;
}

// Split-K: the kernel per (K range of whole scale epochs, tile), then the
// reduction.
gemm_status run_mx6_splitk(const Common &a, int format, const void *SFA, int64_t ldsfa, const void *SFB,
                           int64_t ldsfb, int splits, void *ws, size_t ws_bytes, hipStream_t s) {
    bool none = false;
    gemm_status st = validate_mx6(a, format, SFA, ldsfa, SFB, ldsfb, &none);
    if (st != GEMM_OK || none) return st;
    if (splits < 0 || splits > kMaxSplits) return GEMM_ERR_UNSUPPORTED;
    const bool e3m2 = format == GEMM_FP6_E3M2;
    const int S = effective_splits(a.K, splits == 0 ? auto_splits(a.M, a.N, a.K) : splits, 512);
    if (S == 1 || !fast_mx6(a, SFA, ldsfa, SFB, ldsfb)) return dispatch_mx6(a, e3m2, SFA, ldsfa, SFB, ldsfb, s);
    st = check_workspace(a, S, ws, ws_bytes);
    if (st != GEMM_OK) return st;
    tg::MxArgs q = mx6_args(a, SFA, ldsfa, SFB, ldsfb);
    q.g.C = nullptr;
    q.g.D = nullptr;
    q.g.ldc = 0;
    q.g.ldd = 0;
    const int64_t epochs = (a.K + 511) / 512;           // the last may be partial
    q.g.kt_split = (int)((epochs + S - 1) / S);
    q.g.ws = (float *)ws;
    q.g.ldw = splitk_ldw(a.N);
    const int64_t grid = (int64_t)q.g.tiles_m * q.g.tiles_n * S;
    if (grid >= kMaxDim) return GEMM_ERR_UNSUPPORTED;
    tg::F16Epi e;
    e.vec_c = false;
    e.vec_d = true;                                    // 256-byte aligned base, ldw % 4 == 0
    hipError_t err = tg::launch_mx6_split(e3m2, (unsigned)grid, s, q, e);
    if (err != hipSuccess) return launched(err);
    return reduce_splits(a, ws, S, s);
}

// Operands given as tile images (gemm_mxfp6_pack): the tiled kernel's
// PACKED form, one workgroup per tile or persistent as dispatch_mx6.
gemm_status run_mx6_packed(const Common &a, int format, const void *SFA, int64_t ldsfa, const void *SFB,
                           int64_t ldsfb, hipStream_t s) {
    if (format != GEMM_FP6_E2M3 && format != GEMM_FP6_E3M2) return GEMM_ERR_UNSUPPORTED;
    // (the shared checks on a byte view; the images' extents are implied by
    // M, N and K)
    Common bytes = a;
    bytes.K = a.K / 4 * 3;
    bytes.lda = bytes.K;
    bytes.ldb = bytes.K;
    bool none = false;
    gemm_status st = validate(bytes, &none);
    if (st != GEMM_OK || none) return st;
    if (a.K % 128 != 0 || a.K >= ((int64_t)1 << 23)) return GEMM_ERR_UNSUPPORTED;
    if (a.K > 0) {
        if (misaligned(a.A, 16) || misaligned(a.B, 16)) return GEMM_ERR_MISALIGNED;
        if (ldsfa < a.K / 32 || ldsfb < a.K / 32) return GEMM_ERR_BAD_LD;
        if (!SFA || !SFB) return GEMM_ERR_NULL_POINTER;
        if (misaligned(SFA, 16) || misaligned(SFB, 16) || ldsfa % 16 != 0 || ldsfb % 16 != 0 ||
            ldsfa >= kMaxLdBytes || ldsfb >= kMaxLdBytes)
            return GEMM_ERR_UNSUPPORTED;
    }
    Common k = a;
    k.lda = 0;
    k.ldb = 0;
    const tg::MxArgs q = mx6_args(k, SFA, ldsfa, SFB, ldsfb);
    const int64_t tiles = (int64_t)q.g.tiles_m * q.g.tiles_n;
    if (tiles >= kMaxDim) return GEMM_ERR_UNSUPPORTED;
    const bool bf16 = a.out_type == GEMM_OUT_BF16, e3m2 = format == GEMM_FP6_E3M2;
    const uintptr_t vb = (uintptr_t)(bf16 ? 2 : 4) * 4;
    tg::F16Epi e;
    e.vec_d = ((uintptr_t)a.D % vb) == 0 && a.ldd % 4 == 0;
    e.vec_c = a.C && ((uintptr_t)a.C % vb) == 0 && a.ldc % 4 == 0;
    const int cus = cu_count(s);
    const bool persist = !a.C && e.vec_d && a.N % 4 == 0 && cus > 0 && tiles > cus && persist_allowed();
    const unsigned grid = persist ? (unsigned)cus : (unsigned)tiles;
    return launched(bf16 ? tg::launch_mx6_packed<true>(e3m2, persist, grid, s, q, e)
                         : tg::launch_mx6_packed<false>(e3m2, persist, grid, s, q, e));
}

}  // namespace

extern "C" {

gemm_status gemm_mxfp6(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *SFA, int64_t ldsfa,
                       const void *B, int64_t ldb, const void *SFB, int64_t ldsfb, const void *C, int64_t ldc,
                       void *D, int64_t ldd, int format, int out_type, hipStream_t stream) {
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 1};
    bool none = false;
    gemm_status st = validate_mx6(a, format, SFA, ldsfa, SFB, ldsfb, &none);
    if (st != GEMM_OK || none) return st;
    return dispatch_mx6(a, format == GEMM_FP6_E3M2, SFA, ldsfa, SFB, ldsfb, stream);
}

gemm_status gemm_mxfp6_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int a_order,
                          const void *SFA, int64_t ldsfa, const void *B, int64_t ldb, int b_order, const void *SFB,
                          int64_t ldsfb, const void *C, int64_t ldc, void *D, int64_t ldd, int format,
                          int out_type, hipStream_t stream) {
    if ((a_order != GEMM_K_CONTIGUOUS && a_order != GEMM_MN_CONTIGUOUS) ||
        (b_order != GEMM_K_CONTIGUOUS && b_order != GEMM_MN_CONTIGUOUS))
        return GEMM_ERR_UNSUPPORTED;
    const bool amn = a_order == GEMM_MN_CONTIGUOUS, bmn = b_order == GEMM_MN_CONTIGUOUS;
    if (!amn && !bmn)
        return gemm_mxfp6(M, N, K, A, lda, SFA, ldsfa, B, ldb, SFB, ldsfb, C, ldc, D, ldd, format, out_type,
                          stream);
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 1};
    bool none = false;
    gemm_status st = validate_mx6(a, format, SFA, ldsfa, SFB, ldsfb, &none, amn, bmn);
    if (st != GEMM_OK || none) return st;
    const bool e3m2 = format == GEMM_FP6_E3M2;
    if (K == 0) return dispatch_mx6(a, e3m2, SFA, ldsfa, SFB, ldsfb, stream);
    return run_mx_any(a, e3m2 ? 3 : 2, lda / 4 * 3, ldb / 4 * 3, SFA, ldsfa, SFB, ldsfb, stream, amn, bmn);
}

gemm_status gemm_mxfp6_ex_ws(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int a_order,
                             const void *SFA, int64_t ldsfa, const void *B, int64_t ldb, int b_order,
                             const void *SFB, int64_t ldsfb, const void *C, int64_t ldc, void *D, int64_t ldd,
                             int format, int out_type, void *workspace, size_t workspace_bytes,
                             hipStream_t stream) {
    if ((a_order != GEMM_K_CONTIGUOUS && a_order != GEMM_MN_CONTIGUOUS) ||
        (b_order != GEMM_K_CONTIGUOUS && b_order != GEMM_MN_CONTIGUOUS))
        return GEMM_ERR_UNSUPPORTED;
    const bool amn = a_order == GEMM_MN_CONTIGUOUS, bmn = b_order == GEMM_MN_CONTIGUOUS;
    if (workspace && !amn && !bmn && K > 0) {
        // both K-contiguous: their tile images in the workspace, then the
        // packed kernel (the same D bit for bit), where the call allows it
        Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 1};
        bool none = false;
        gemm_status st = validate_mx6(a, format, SFA, ldsfa, SFB, ldsfb, &none);
        if (st != GEMM_OK || none) return st;
        const size_t need = mx6_images_bytes(M, N, K);
        if (need > 0 && workspace_bytes >= need && (uintptr_t)workspace % 256 == 0 && (uintptr_t)SFA % 16 == 0 &&
            (uintptr_t)SFB % 16 == 0 && ldsfa % 16 == 0 && ldsfb % 16 == 0) {
            char *AP = (char *)workspace, *BP = AP + (gemm_mxfp6_packed_bytes(M, K) + 255) / 256 * 256;
            st = gemm_mxfp6_pack(M, K, A, lda, AP, gemm_mxfp6_packed_bytes(M, K), stream);
            if (st != GEMM_OK) return st;
            st = gemm_mxfp6_pack(N, K, B, ldb, BP, gemm_mxfp6_packed_bytes(N, K), stream);
            if (st != GEMM_OK) return st;
            return gemm_mxfp6_packed(M, N, K, AP, SFA, ldsfa, BP, SFB, ldsfb, C, ldc, D, ldd, format, out_type,
                                     stream);
        }
    }
    if (!workspace || (!amn && !bmn) || K == 0)
        return gemm_mxfp6_ex(M, N, K, A, lda, a_order, SFA, ldsfa, B, ldb, b_order, SFB, ldsfb, C, ldc, D, ldd,
                             format, out_type, stream);
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 1};
    bool none = false;
    gemm_status st = validate_mx6(a, format, SFA, ldsfa, SFB, ldsfb, &none, amn, bmn);
    if (st != GEMM_OK || none) return st;
    Common k = a;
    st = k_contiguous_operands(6, a, amn, bmn, workspace, workspace_bytes, stream, &k.A, &k.lda, &k.B, &k.ldb);
    if (st != GEMM_OK) return st;
    return gemm_mxfp6(M, N, K, k.A, k.lda, SFA, ldsfa, k.B, k.ldb, SFB, ldsfb, C, ldc, D, ldd, format, out_type,
                      stream);
}

gemm_status gemm_mxfp6_packed(int64_t M, int64_t N, int64_t K, const void *AP, const void *SFA, int64_t ldsfa,
                              const void *BP, const void *SFB, int64_t ldsfb, const void *C, int64_t ldc, void *D,
                              int64_t ldd, int format, int out_type, hipStream_t stream) {
    Common a{M, N, K, AP, K, BP, K, C, ldc, D, ldd, out_type, 1};
    return run_mx6_packed(a, format, SFA, ldsfa, SFB, ldsfb, stream);
}

gemm_status gemm_mxfp6_splitk(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *SFA,
                              int64_t ldsfa, const void *B, int64_t ldb, const void *SFB, int64_t ldsfb,
                              const void *C, int64_t ldc, void *D, int64_t ldd, int format, int out_type,
                              int splits, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 1};
    return run_mx6_splitk(a, format, SFA, ldsfa, SFB, ldsfb, splits, workspace, workspace_bytes, stream);
}

}  // extern "C"
