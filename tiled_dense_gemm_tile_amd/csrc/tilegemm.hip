// C ABI of the tiled GEMM library: argument validation, kernel selection
// and launch on the caller's stream.  The declarations and their contract
// are in include/tilegemm.h.
#include "../../include/tilegemm.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_f16.hpp"

namespace {

thread_local int g_last_hip_error = 0;

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

bool misaligned(const void *p, int size) { return p && (((uintptr_t)p) % (uintptr_t)size) != 0; }

// Validation shared by every entry point; returns GEMM_OK when a launch may
// proceed (and sets *nothing_to_do when M or N is zero).
gemm_status validate(const Common &a, bool *nothing_to_do) {
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

gemm_status launched(hipError_t e) {
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return GEMM_ERR_HIP;
    }
    return GEMM_OK;
}

// ---- 16-bit inputs ------------------------------------------------------

using CfgBig = tg::TileCfg<256, 256, 64, 2, 2>;
using CfgMid = tg::TileCfg<128, 128, 64, 2, 2>;
using CfgSmall = tg::TileCfg<64, 64, 64, 2, 2>;

template <class Cfg, int VEC, bool FP16, bool OUT_BF16>
gemm_status launch_f16(const Common &a, hipStream_t s) {
    tg::F16Args p;
    p.A = a.A;
    p.B = a.B;
    p.C = a.C;
    p.D = a.D;
    p.lda = a.lda;
    p.ldb = a.ldb;
    p.ldc = a.ldc;
    p.ldd = a.ldd;
    p.M = (int)a.M;
    p.N = (int)a.N;
    p.K = (int)a.K;
    p.tiles_m = (int)((a.M + Cfg::BM - 1) / Cfg::BM);
    p.tiles_n = (int)((a.N + Cfg::BN - 1) / Cfg::BN);
    p.group_m = 4;
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    if (tiles >= kMaxDim) return GEMM_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((tg::gemm_f16_kernel<Cfg, VEC, FP16, OUT_BF16>), dim3((unsigned)tiles), dim3(Cfg::NT),
                       0, s, p);
    return launched(hipGetLastError());
}

// Widest vector (in elements) that every row start and K boundary allows.
int pick_vec(const Common &a) {
    for (int v = 8; v > 1; v >>= 1) {
        const uintptr_t bytes = (uintptr_t)v * 2;
        if (((uintptr_t)a.A % bytes) == 0 && ((uintptr_t)a.B % bytes) == 0 && a.lda % v == 0 &&
            a.ldb % v == 0 && a.K % v == 0)
            return v;
    }
    return 1;
}

template <bool FP16, bool OUT_BF16>
gemm_status dispatch_f16(const Common &a, hipStream_t s) {
    const int vec = pick_vec(a);
    const int64_t big_tiles = ((a.M + 255) / 256) * ((a.N + 255) / 256);
    const int64_t mid_tiles = ((a.M + 127) / 128) * ((a.N + 127) / 128);
    if (vec == 8) {
        if (big_tiles >= 256) return launch_f16<CfgBig, 8, FP16, OUT_BF16>(a, s);
        if (mid_tiles >= 256) return launch_f16<CfgMid, 8, FP16, OUT_BF16>(a, s);
        return launch_f16<CfgSmall, 8, FP16, OUT_BF16>(a, s);
    }
    switch (vec) {
    case 4: return launch_f16<CfgMid, 4, FP16, OUT_BF16>(a, s);
    case 2: return launch_f16<CfgMid, 2, FP16, OUT_BF16>(a, s);
    default: return launch_f16<CfgMid, 1, FP16, OUT_BF16>(a, s);
    }
}

gemm_status run_f16(bool fp16, const Common &a, hipStream_t s) {
    bool none = false;
    gemm_status st = validate(a, &none);
    if (st != GEMM_OK || none) return st;
    if (fp16)
        return a.out_type == GEMM_OUT_BF16 ? dispatch_f16<true, true>(a, s) : dispatch_f16<true, false>(a, s);
    return a.out_type == GEMM_OUT_BF16 ? dispatch_f16<false, true>(a, s) : dispatch_f16<false, false>(a, s);
}

}  // namespace

extern "C" {

gemm_status gemm_bf16(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                      const void *C, int64_t ldc, void *D, int64_t ldd, int out_type, hipStream_t stream) {
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 2};
    return run_f16(false, a, stream);
}

gemm_status gemm_fp16(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                      const void *C, int64_t ldc, void *D, int64_t ldd, int out_type, hipStream_t stream) {
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 2};
    return run_f16(true, a, stream);
}

gemm_status gemm_mxfp8(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *SFA, int64_t ldsfa,
                       const void *B, int64_t ldb, const void *SFB, int64_t ldsfb, const void *C, int64_t ldc,
                       void *D, int64_t ldd, int out_type, hipStream_t stream) {
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 1};
    bool none = false;
    gemm_status st = validate(a, &none);
    if (st != GEMM_OK || none) return st;
    if (K > 0) {
        if (ldsfa < K / 32 || ldsfb < K / 32) return GEMM_ERR_BAD_LD;
        if (!SFA || !SFB) return GEMM_ERR_NULL_POINTER;
    }
    if (K % 32 != 0) return GEMM_ERR_UNSUPPORTED;
    if (ldsfa >= kMaxLdBytes || ldsfb >= kMaxLdBytes) return GEMM_ERR_UNSUPPORTED;
    (void)stream;
    return GEMM_ERR_UNSUPPORTED;
}

const char *gemm_status_string(int s) {
    switch (s) {
    case GEMM_OK: return "GEMM_OK";
    case GEMM_ERR_INVALID_SIZE: return "GEMM_ERR_INVALID_SIZE: M, N or K is negative";
    case GEMM_ERR_NULL_POINTER: return "GEMM_ERR_NULL_POINTER: a required pointer is NULL";
    case GEMM_ERR_BAD_LD: return "GEMM_ERR_BAD_LD: a leading dimension is smaller than its row";
    case GEMM_ERR_MISALIGNED: return "GEMM_ERR_MISALIGNED: a pointer is not aligned to its element size";
    case GEMM_ERR_UNSUPPORTED: return "GEMM_ERR_UNSUPPORTED: outside the library's limits";
    case GEMM_ERR_HIP: return "GEMM_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown gemm_status";
    }
}

int gemm_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
