// C ABI of the tiled GEMM library, block-scaled fp4 inputs: argument
// validation, kernel selection and launch on the caller's stream.  The
// declarations and their contract are in include/tilegemm.h.
#include <stdlib.h>

#include "api.hpp"
#include "mx4_launch.hpp"

using namespace tg_api;

namespace {

// a.lda and a.ldb are in elements (even); the kernel takes them in bytes.
gemm_status dispatch_mx4(const Common &a, const void *SFA, int64_t ldsfa, const void *SFB, int64_t ldsfb,
                         hipStream_t s) {
    // 16-byte A/B chunks (32 elements), 16-byte scale words (512 K) per row
    const bool fast = a.K % 512 == 0 && (uintptr_t)a.A % 16 == 0 && (uintptr_t)a.B % 16 == 0 && a.lda % 32 == 0 &&
                      a.ldb % 32 == 0 && (uintptr_t)SFA % 16 == 0 && (uintptr_t)SFB % 16 == 0 &&
                      ldsfa % 16 == 0 && ldsfb % 16 == 0;
    if (!fast && a.K > 0) return GEMM_ERR_UNSUPPORTED;
    tg::MxArgs q;
    q.g.A = a.A;
    q.g.B = a.B;
    q.g.C = a.C;
    q.g.D = a.D;
    q.g.lda = a.lda / 2;
    q.g.ldb = a.ldb / 2;
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
    return launched(bf16 ? tg::launch_mx4<true>((unsigned)tiles, s, q, e)
                         : tg::launch_mx4<false>((unsigned)tiles, s, q, e));
}

}  // namespace

extern "C" {

gemm_status gemm_mxfp4(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *SFA, int64_t ldsfa,
                       const void *B, int64_t ldb, const void *SFB, int64_t ldsfb, const void *C, int64_t ldc,
                       void *D, int64_t ldd, int out_type, hipStream_t stream) {
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 1};
    bool none = false;
    // A and B extents validated in bytes (half the element counts; for even
    // K, lda / 2 < K / 2 exactly when lda < K, and odd K is unsupported)
    Common bytes = a;
    bytes.K = K / 2;
    bytes.lda = lda / 2;
    bytes.ldb = ldb / 2;
    gemm_status st = validate(bytes, &none);
    if (st != GEMM_OK || none) return st;
    if (K >= kMaxDim || K % 32 != 0 || lda % 2 != 0 || ldb % 2 != 0) return GEMM_ERR_UNSUPPORTED;
    if (K > 0) {
        if (ldsfa < K / 32 || ldsfb < K / 32) return GEMM_ERR_BAD_LD;
        if (!SFA || !SFB) return GEMM_ERR_NULL_POINTER;
    }
    if (ldsfa >= kMaxLdBytes || ldsfb >= kMaxLdBytes) return GEMM_ERR_UNSUPPORTED;
    return dispatch_mx4(a, SFA, ldsfa, SFB, ldsfb, stream);
}

}  // extern "C"
