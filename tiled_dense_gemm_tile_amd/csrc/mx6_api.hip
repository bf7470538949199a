// C ABI of the tiled GEMM library, block-scaled fp6 inputs: argument
// validation, kernel selection and launch on the caller's stream.  The
// declarations and their contract are in include/tilegemm.h.
#include <stdlib.h>

#include "api.hpp"
#include "mx6_launch.hpp"

using namespace tg_api;

namespace {

// a.lda and a.ldb are in elements (multiples of 4); the kernel takes them in
// bytes (three quarters of that).
gemm_status dispatch_mx6(const Common &a, bool e3m2, const void *SFA, int64_t ldsfa, const void *SFB, int64_t ldsfb,
                         hipStream_t s) {
    // 16-byte A/B rows (lda multiple of 64 elements), 16-byte scale words
    // (512 K) per row
    const bool fast = a.K % 512 == 0 && (uintptr_t)a.A % 16 == 0 && (uintptr_t)a.B % 16 == 0 && a.lda % 64 == 0 &&
                      a.ldb % 64 == 0 && (uintptr_t)SFA % 16 == 0 && (uintptr_t)SFB % 16 == 0 &&
                      ldsfa % 16 == 0 && ldsfb % 16 == 0;
    if (!fast && a.K > 0) return GEMM_ERR_UNSUPPORTED;
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
    const int64_t tiles = (int64_t)q.g.tiles_m * q.g.tiles_n;
    if (tiles >= kMaxDim) return GEMM_ERR_UNSUPPORTED;
    const bool bf16 = a.out_type == GEMM_OUT_BF16;
    const int os = bf16 ? 2 : 4;
    const uintptr_t vb = (uintptr_t)os * 4;
    tg::F16Epi e;
    e.vec_d = ((uintptr_t)a.D % vb) == 0 && a.ldd % 4 == 0;
    e.vec_c = a.C && ((uintptr_t)a.C % vb) == 0 && a.ldc % 4 == 0;
    return launched(bf16 ? tg::launch_mx6<true>(e3m2, (unsigned)tiles, s, q, e)
                         : tg::launch_mx6<false>(e3m2, (unsigned)tiles, s, q, e));
}

}  // namespace

extern "C" {

gemm_status gemm_mxfp6(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *SFA, int64_t ldsfa,
                       const void *B, int64_t ldb, const void *SFB, int64_t ldsfb, const void *C, int64_t ldc,
                       void *D, int64_t ldd, int format, int out_type, hipStream_t stream) {
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 1};
    if (format != GEMM_FP6_E2M3 && format != GEMM_FP6_E3M2) return GEMM_ERR_UNSUPPORTED;
    bool none = false;
    // A and B extents validated in bytes (three quarters of the element
    // counts; for K and lda multiples of 4, lda < K exactly when the byte
    // counts compare so, and other K or lda are unsupported)
    Common bytes = a;
    bytes.K = K / 4 * 3;
    bytes.lda = lda / 4 * 3;
    bytes.ldb = ldb / 4 * 3;
    gemm_status st = validate(bytes, &none);
    if (st != GEMM_OK || none) return st;
    if (K >= kMaxDim || K % 32 != 0 || lda % 4 != 0 || ldb % 4 != 0) return GEMM_ERR_UNSUPPORTED;
    if (K > 0) {
        if (ldsfa < K / 32 || ldsfb < K / 32) return GEMM_ERR_BAD_LD;
        if (!SFA || !SFB) return GEMM_ERR_NULL_POINTER;
    }
    if (ldsfa >= kMaxLdBytes || ldsfb >= kMaxLdBytes) return GEMM_ERR_UNSUPPORTED;
    return dispatch_mx6(a, format == GEMM_FP6_E3M2, SFA, ldsfa, SFB, ldsfb, stream);
}

}  // extern "C"
