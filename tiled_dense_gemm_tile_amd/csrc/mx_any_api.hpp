// Host side of the general block-scaled kernel, shared by the fp8, fp4 and
// fp6 entry points: the calls their tiled kernels do not take.
#pragma once

#include "api.hpp"
#include "gemm_mx_any.hpp"

namespace tg_api {

// fmt: 0 e4m3, 2 e2m3, 3 e3m2, 4 e2m1; lda_b / ldb_b: leading dimensions in
// bytes; amn / bmn: A / B stored MN-contiguous.  The call has been validated
// (K % 32 == 0, whole-byte rows).
// kb_shift: the scale block width is 32 << kb_shift (0: the standard form).
inline gemm_status run_mx_any(const Common &a, int fmt, int64_t lda_b, int64_t ldb_b, const void *SFA,
                              int64_t ldsfa, const void *SFB, int64_t ldsfb, hipStream_t s, bool amn = false,
                              bool bmn = false, int kb_shift = 0) {
    tg::MxArgs q;
    q.g.A = a.A ? a.A : a.D;                            // K == 0 reads nothing
    q.g.B = a.B ? a.B : a.D;
    q.g.C = a.C;
    q.g.D = a.D;
    q.g.lda = lda_b;
    q.g.ldb = ldb_b;
    q.g.ldc = a.ldc;
    q.g.ldd = a.ldd;
    q.g.M = (int)a.M;
    q.g.N = (int)a.N;
    q.g.K = (int)a.K;
    q.g.group_m = 1;
    q.g.tiles_m = (int)((a.M + 63) / 64);
    q.g.tiles_n = (int)((a.N + 63) / 64);
    q.SFA = SFA ? SFA : a.D;
    q.SFB = SFB ? SFB : a.D;
    q.ldsfa = ldsfa;
    q.ldsfb = ldsfb;
    q.kb_shift = kb_shift;
    const int64_t grid = (int64_t)q.g.tiles_m * q.g.tiles_n;
    if (grid >= kMaxDim) return GEMM_ERR_UNSUPPORTED;
    // the widest load every K-contiguous row start allows
    const uint64_t abits = (uint64_t)(uintptr_t)q.g.A | (uint64_t)lda_b;
    const uint64_t bbits = (uint64_t)(uintptr_t)q.g.B | (uint64_t)ldb_b;
    const uint64_t bits = (amn ? 0 : abits) | (bmn ? 0 : bbits);
    const int vec = bits % 16 == 0 ? 16 : bits % 8 == 0 ? 8 : bits % 4 == 0 ? 4 : 1;
    // fp8 MN-contiguous operands with 16-byte rows: staged panels
    const bool stage = fmt == 0 && (amn || bmn) && (!amn || abits % 16 == 0) && (!bmn || bbits % 16 == 0);
    return launched(tg::launch_mx_any(fmt, a.out_type == GEMM_OUT_BF16, vec, amn, bmn, stage, (unsigned)grid, s, q));
}

}  // namespace tg_api
