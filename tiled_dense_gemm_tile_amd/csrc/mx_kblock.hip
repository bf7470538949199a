// C ABI of the tiled GEMM library: block-scaled forms with scale blocks
// wider than 32 K elements (gemm_mx_kblock).  The declaration and its
// contract are in include/tilegemm.h.
#include "api.hpp"
#include "mx_any_api.hpp"

using namespace tg_api;

extern "C" gemm_status gemm_mx_kblock(int format, int64_t M, int64_t N, int64_t K, int64_t kblock, const void *A,
                                      int64_t lda, const void *SFA, int64_t ldsfa, const void *B, int64_t ldb,
                                      const void *SFB, int64_t ldsfb, const void *C, int64_t ldc, void *D,
                                      int64_t ldd, int out_type, hipStream_t stream) {
    if (format < GEMM_MX_E4M3 || format > GEMM_MX_E3M2 || kblock <= 0 || kblock % 32 != 0 || kblock >= kMaxDim)
        return GEMM_ERR_UNSUPPORTED;
    // the kernel takes widths 32 << s, and any width >= K (one scale per row)
    int kb_shift = 0;
    while ((32LL << kb_shift) < kblock) ++kb_shift;
    const bool per_row = K > 0 && kblock >= K;
    if ((32LL << kb_shift) != kblock && !per_row) return GEMM_ERR_UNSUPPORTED;
    if (per_row) kb_shift = 31;
    if (kblock == 32) {
        switch (format) {
        case GEMM_MX_E4M3:
            return gemm_mxfp8(M, N, K, A, lda, SFA, ldsfa, B, ldb, SFB, ldsfb, C, ldc, D, ldd, out_type, stream);
        case GEMM_MX_E2M1:
            return gemm_mxfp4(M, N, K, A, lda, SFA, ldsfa, B, ldb, SFB, ldsfb, C, ldc, D, ldd, out_type, stream);
        default:
            return gemm_mxfp6(M, N, K, A, lda, SFA, ldsfa, B, ldb, SFB, ldsfb, C, ldc, D, ldd,
                              format == GEMM_MX_E2M3 ? GEMM_FP6_E2M3 : GEMM_FP6_E3M2, out_type, stream);
        }
    }
    // operand extents in bytes: elements per byte 1 (fp8), 2 (fp4), 4 per 3 (fp6)
    const int64_t num = format == GEMM_MX_E4M3 ? 1 : format == GEMM_MX_E2M1 ? 2 : 4;
    const int64_t den = format == GEMM_MX_E2M1 ? 1 : format == GEMM_MX_E4M3 ? 1 : 3;
    if (lda % num != 0 || ldb % num != 0 || (K >= 0 && K % 32 != 0)) return GEMM_ERR_UNSUPPORTED;
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 1};
    Common bytes = a;
    bytes.K = K / num * den;
    bytes.lda = lda / num * den;
    bytes.ldb = ldb / num * den;
    bool none = false;
    gemm_status st = validate(bytes, &none);
    if (st != GEMM_OK || none) return st;
    if (K >= kMaxDim) return GEMM_ERR_UNSUPPORTED;
    const int64_t nsc = (K + kblock - 1) / kblock;      // scales per row
    if (K > 0) {
        if (ldsfa < nsc || ldsfb < nsc) return GEMM_ERR_BAD_LD;
        if (!SFA || !SFB) return GEMM_ERR_NULL_POINTER;
    }
    if (ldsfa >= kMaxLdBytes || ldsfb >= kMaxLdBytes) return GEMM_ERR_UNSUPPORTED;
    // the general kernel's format codes: 0 e4m3, 4 e2m1, 2 e2m3, 3 e3m2
    const int fmt = format == GEMM_MX_E4M3 ? 0 : format == GEMM_MX_E2M1 ? 4 : format == GEMM_MX_E2M3 ? 2 : 3;
    return run_mx_any(a, fmt, bytes.lda, bytes.ldb, SFA, ldsfa, SFB, ldsfb, stream, false, false, kb_shift);
}
