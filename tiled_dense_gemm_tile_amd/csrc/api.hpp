// Shared host-side pieces of the C ABI (include/tilegemm.h): sizes and
// limits, argument validation, launch-status recording.  Included by the
// entry-point translation units of each input family.
#pragma once

#include "../../include/tilegemm.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg_api {

// hipError_t of the calling thread's last failed launch (gemm_last_hip_error)
inline thread_local int g_last_hip_error = 0;



constexpr int64_t kMaxDim = (int64_t)1 << 31;
// Each tile's rows are addressed with 32-bit offsets from a per-tile base:
// 256 rows of the widest leading dimension must stay below 2^31 bytes.
constexpr int64_t kMaxLdBytes = ((int64_t)1 << 31) / 256;

struct Common {
    int64_t M, N, K;
    const void *A;
    int64_t lda;
    const void *B;
    int64_t ldb;
    const void *C;
    int64_t ldc;
    void *D;
    int64_t ldd;
    int out_type;
    int in_size;   // bytes per A/B element
};

inline bool misaligned(const void *p, int size) { return p && (((uintptr_t)p) % (uintptr_t)size) != 0; }

// Validation shared by every entry point; returns GEMM_OK when a launch may
// proceed (and sets *nothing_to_do when M or N is zero).
inline gemm_status validate(const Common &a, bool *nothing_to_do) {
    *nothing_to_do = false;
    if (a.M < 0 || a.N < 0 || a.K < 0) return GEMM_ERR_INVALID_SIZE;
    if (a.M >= kMaxDim || a.N >= kMaxDim || a.K >= kMaxDim) return GEMM_ERR_UNSUPPORTED;
    if (a.out_type != GEMM_OUT_F32 && a.out_type != GEMM_OUT_BF16) return GEMM_ERR_UNSUPPORTED;
    if (a.M == 0 || a.N == 0) {
        *nothing_to_do = true;
        return GEMM_OK;
    }
    if (a.lda < a.K || a.ldb < a.K || a.ldd < a.N || (a.C && a.ldc < a.N)) return GEMM_ERR_BAD_LD;
    if (!a.D) return GEMM_ERR_NULL_POINTER;
    if (a.K > 0 && (!a.A || !a.B)) return GEMM_ERR_NULL_POINTER;
    const int os = a.out_type == GEMM_OUT_BF16 ? 2 : 4;
    if (misaligned(a.A, a.in_size) || misaligned(a.B, a.in_size) || misaligned(a.C, os) ||
        misaligned(a.D, os))
        return GEMM_ERR_MISALIGNED;
    if (a.lda * a.in_size >= kMaxLdBytes || a.ldb * a.in_size >= kMaxLdBytes ||
        a.ldd * os >= kMaxLdBytes || (a.C && a.ldc * os >= kMaxLdBytes))
        return GEMM_ERR_UNSUPPORTED;
    if (a.C && a.C != a.D) {
        const uintptr_t c0 = (uintptr_t)a.C, c1 = c0 + (uintptr_t)(((a.M - 1) * a.ldc + a.N) * os);
        const uintptr_t d0 = (uintptr_t)a.D, d1 = d0 + (uintptr_t)(((a.M - 1) * a.ldd + a.N) * os);
        if (c0 < d1 && d0 < c1) return GEMM_ERR_UNSUPPORTED;
    }
    if (a.C && a.C == a.D && a.ldc != a.ldd) return GEMM_ERR_UNSUPPORTED;
    return GEMM_OK;
}

inline gemm_status launched(hipError_t e) {
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return GEMM_ERR_HIP;
    }
    return GEMM_OK;
}

inline int64_t tiles_of(const Common &a, int bm, int bn) { return ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn); }

}  // namespace tg_api
