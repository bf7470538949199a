// C ABI of the tiled GEMM library: block-scaled forms with scale blocks
// wider than 32 K elements (gemm_mx_kblock).  The declaration and its
// contract are in include/tilegemm.h.
#include "api.hpp"
#include "mx_any_api.hpp"

using namespace tg_api;

namespace {

// Scale replication for gemm_mx_kblock_ws: row r of dst (ldd bytes, a
// multiple of 16) gets, at byte b < nb32, the scale of the kb-wide block
// holding 32-element block b -- src byte b >> shift (shift 31: one scale per
// row, byte 0) -- and 127 (a scale of 1) in the padding up to ldd.  One
// thread per 16-byte piece of a destination row.
__global__ void __launch_bounds__(256) expand_scales_kernel(const uint8_t *src, int64_t lds, uint8_t *dst,
                                                            int64_t ldd, int64_t pieces, int per_row, int nb32,
                                                            int shift) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= pieces) return;
    const int64_t r = i / per_row;
    const int c = (int)(i - r * per_row);
    const uint8_t *row = src + r * lds;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t v = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = 16 * c + 4 * k + j;
            const uint32_t code = b < nb32 ? (uint32_t)row[(uint32_t)b >> shift] : 127u;
            v |= code << (8 * j);
        }
        w[k] = v;
    }
    *(uint4 *)(dst + r * ldd + 16 * c) = make_uint4(w[0], w[1], w[2], w[3]);
}

// bytes of one replicated scale row: ceil(K / 32) rounded up to 16
int64_t kblock_ld32(int64_t K) { return ((K + 31) / 32 + 15) / 16 * 16; }

// The checks of a gemm_mx_kblock call (all of them: the replicated-scale
// path launches nothing before they pass).  Sets the scale index shift
// (31: one scale per row), the call's Common form with operand extents in
// bytes, and *none when M or N is zero.
gemm_status kblock_validate(int format, int64_t M, int64_t N, int64_t K, int64_t kblock, const void *A, int64_t lda,
                            const void *SFA, int64_t ldsfa, const void *B, int64_t ldb, const void *SFB,
                            int64_t ldsfb, const void *C, int64_t ldc, void *D, int64_t ldd, int out_type,
                            int *kb_shift, Common *a, Common *bytes, bool *none) {
    *none = false;
    if (format < GEMM_MX_E4M3 || format > GEMM_MX_E3M2 || kblock <= 0 || kblock % 32 != 0 || kblock >= kMaxDim)
        return GEMM_ERR_UNSUPPORTED;
    // the kernel takes widths 32 << s, and any width >= K (one scale per row)
    int s = 0;
    while ((32LL << s) < kblock) ++s;
    const bool per_row = K > 0 && kblock >= K;
    if ((32LL << s) != kblock && !per_row) return GEMM_ERR_UNSUPPORTED;
    *kb_shift = per_row ? 31 : s;
    // operand extents in bytes: elements per byte 1 (fp8), 2 (fp4), 4 per 3 (fp6)
    const int64_t num = format == GEMM_MX_E4M3 ? 1 : format == GEMM_MX_E2M1 ? 2 : 4;
    const int64_t den = format == GEMM_MX_E2M1 ? 1 : format == GEMM_MX_E4M3 ? 1 : 3;
    if (lda % num != 0 || ldb % num != 0 || (K >= 0 && K % 32 != 0)) return GEMM_ERR_UNSUPPORTED;
    *a = Common{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 1};
    *bytes = *a;
    bytes->K = K / num * den;
    bytes->lda = lda / num * den;
    bytes->ldb = ldb / num * den;
    gemm_status st = validate(*bytes, none);
    if (st != GEMM_OK || *none) return st;
    if (K >= kMaxDim) return GEMM_ERR_UNSUPPORTED;
    const int64_t nsc = (K + kblock - 1) / kblock;      // scales per row
    if (K > 0) {
        if (ldsfa < nsc || ldsfb < nsc) return GEMM_ERR_BAD_LD;
        if (!SFA || !SFB) return GEMM_ERR_NULL_POINTER;
    }
    if (ldsfa >= kMaxLdBytes || ldsfb >= kMaxLdBytes) return GEMM_ERR_UNSUPPORTED;
    return GEMM_OK;
}

// the standard call of a format on 32-wide scales
gemm_status standard_call(int format, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *SFA,
                          int64_t ldsfa, const void *B, int64_t ldb, const void *SFB, int64_t ldsfb, const void *C,
                          int64_t ldc, void *D, int64_t ldd, int out_type, hipStream_t stream) {
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

}  // namespace

extern "C" gemm_status gemm_mx_kblock(int format, int64_t M, int64_t N, int64_t K, int64_t kblock, const void *A,
                                      int64_t lda, const void *SFA, int64_t ldsfa, const void *B, int64_t ldb,
                                      const void *SFB, int64_t ldsfb, const void *C, int64_t ldc, void *D,
                                      int64_t ldd, int out_type, hipStream_t stream) {
    if (kblock == 32 && format >= GEMM_MX_E4M3 && format <= GEMM_MX_E3M2)
        return standard_call(format, M, N, K, A, lda, SFA, ldsfa, B, ldb, SFB, ldsfb, C, ldc, D, ldd, out_type,
                             stream);
    int kb_shift = 0;
    Common a, bytes;
    bool none = false;
    const gemm_status st = kblock_validate(format, M, N, K, kblock, A, lda, SFA, ldsfa, B, ldb, SFB, ldsfb, C, ldc,
                                           D, ldd, out_type, &kb_shift, &a, &bytes, &none);
    if (st != GEMM_OK || none) return st;
    // the general kernel's format codes: 0 e4m3, 4 e2m1, 2 e2m3, 3 e3m2
    const int fmt = format == GEMM_MX_E4M3 ? 0 : format == GEMM_MX_E2M1 ? 4 : format == GEMM_MX_E2M3 ? 2 : 3;
    return run_mx_any(a, fmt, bytes.lda, bytes.ldb, SFA, ldsfa, SFB, ldsfb, stream, false, false, kb_shift);
}

extern "C" size_t gemm_mx_kblock_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return 0;
    return (size_t)(M + N) * (size_t)kblock_ld32(K);
}

extern "C" gemm_status gemm_mx_kblock_ws(int format, int64_t M, int64_t N, int64_t K, int64_t kblock,
                                         const void *A, int64_t lda, const void *SFA, int64_t ldsfa,
                                         const void *B, int64_t ldb, const void *SFB, int64_t ldsfb,
                                         const void *C, int64_t ldc, void *D, int64_t ldd, int out_type,
                                         void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!workspace || kblock == 32)
        return gemm_mx_kblock(format, M, N, K, kblock, A, lda, SFA, ldsfa, B, ldb, SFB, ldsfb, C, ldc, D, ldd,
                              out_type, stream);
    int shift = 0;
    Common a, bytes;
    bool none = false;
    gemm_status st = kblock_validate(format, M, N, K, kblock, A, lda, SFA, ldsfa, B, ldb, SFB, ldsfb, C, ldc, D,
                                     ldd, out_type, &shift, &a, &bytes, &none);
    if (st != GEMM_OK || none) return st;
    if (K == 0)                                        // D = C (or 0): no scale is read
        return gemm_mx_kblock(format, M, N, K, kblock, A, lda, SFA, ldsfa, B, ldb, SFB, ldsfb, C, ldc, D, ldd,
                              out_type, stream);
    if (workspace_bytes < gemm_mx_kblock_workspace_bytes(M, N, K)) return GEMM_ERR_WORKSPACE;
    if ((uintptr_t)workspace % 256 != 0) return GEMM_ERR_MISALIGNED;
    // The standard call then sees the same operands, C and D (checked
    // above) and replicated scale rows of ld32 >= K / 32 bytes, 256-byte
    // aligned, so it accepts the call.
    const int64_t ld32 = kblock_ld32(K);
    uint8_t *sfa32 = (uint8_t *)workspace, *sfb32 = sfa32 + M * ld32;
    const int nb32 = (int)(K / 32), per_row = (int)(ld32 / 16);
    auto expand = [&](const void *src, int64_t lds, uint8_t *dst, int64_t rows) {
        const int64_t pieces = rows * per_row;
        hipLaunchKernelGGL(expand_scales_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, stream,
                           (const uint8_t *)src, lds, dst, ld32, pieces, per_row, nb32, shift);
        return hipGetLastError();
    };
    st = launched(expand(SFA, ldsfa, sfa32, M));
    if (st == GEMM_OK) st = launched(expand(SFB, ldsfb, sfb32, N));
    if (st != GEMM_OK) return st;
    return standard_call(format, M, N, K, A, lda, sfa32, ld32, B, ldb, sfb32, ld32, C, ldc, D, ldd, out_type,
                         stream);
}
