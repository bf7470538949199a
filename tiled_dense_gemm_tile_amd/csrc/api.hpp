// Shared host-side pieces of the C ABI (include/tilegemm.h): sizes and
// limits, argument validation, launch-status recording.  Included by the
// entry-point translation units of each input family.
#pragma once

#include "../../include/tilegemm.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "splitk.hpp"

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
// proceed (and sets *nothing_to_do when M or N is zero).  lda_min / ldb_min:
// the shortest leading dimension of each operand (negative: K, for
// K-contiguous storage).
inline gemm_status validate(const Common &a, bool *nothing_to_do, int64_t lda_min = -1, int64_t ldb_min = -1) {
    *nothing_to_do = false;
    if (a.M < 0 || a.N < 0 || a.K < 0) return GEMM_ERR_INVALID_SIZE;
    if (a.M >= kMaxDim || a.N >= kMaxDim || a.K >= kMaxDim) return GEMM_ERR_UNSUPPORTED;
    if (a.out_type != GEMM_OUT_F32 && a.out_type != GEMM_OUT_BF16) return GEMM_ERR_UNSUPPORTED;
    if (a.M == 0 || a.N == 0) {
        *nothing_to_do = true;
        return GEMM_OK;
    }
    if (a.lda < (lda_min < 0 ? a.K : lda_min) || a.ldb < (ldb_min < 0 ? a.K : ldb_min) || a.ldd < a.N ||
        (a.C && a.ldc < a.N))
        return GEMM_ERR_BAD_LD;
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

// Compute units of the stream's GPU (NULL stream: the current device),
// looked up once per device; 0 when the runtime cannot tell.
inline int cu_count(hipStream_t s) {
    static std::atomic<int> counts[64];
    int dev = 0;
    if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = counts[dev].load(std::memory_order_relaxed);
    if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
        counts[dev].store(n, std::memory_order_relaxed);
    return n > 0 ? n : 0;
}

// ---- split-K (every input family) ------------------------------------------

constexpr int kMaxSplits = 64;

// Split count actually used for a requested one when K is cut at multiples
// of `unit` elements (the kernel's K tile or scale epoch): at most one split
// per unit, every split non-empty (ranges of ceil(units / s) units).
inline int effective_splits(int64_t K, int splits, int64_t unit = 64) {
    const int64_t kt = (K + unit - 1) / unit;
    if (kt <= 1 || splits <= 1) return 1;
    const int64_t s = splits > kt ? kt : splits;
    const int64_t kps = (kt + s - 1) / s;
    return (int)((kt + kps - 1) / kps);
}

// The library's choice: split only grids of fewer than 128 tiles of 256 x 256,
// up to one wave of 256 workgroups, keeping at least 4096 K per split so that
// writing and re-reading a split's fp32 partial tile stays small next to its
// multiply work.
// Only grids of fewer than 128 output tiles of 256 x 256 are split, into as
// many K ranges as fill one wave (256 / tiles).  Under 16 tiles each range
// keeps at least 64 K tiles of 64.  From 16 tiles each keeps at least 20, and
// the grid is split only if the ranges then give 200 or more workgroups:
// below that the unsplit call's small-tile kernels, which cover the chip by
// themselves, are as fast or faster (bf16, measured: 1024 x 1024 x 8192
// unsplit 34.2 us, 2 ranges 77.3; 2048 x 2048 x 4096 unsplit 40-44, 3 ranges
// 46.0; 2304 x 2304 x 4096 unsplit 58.7, 3 ranges 52.7; 2048 x 2048 x 8192
// unsplit 76.2, 4 ranges 66.8).
inline int auto_splits(int64_t M, int64_t N, int64_t K) {
    const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
    if (tiles <= 0 || tiles >= 128) return 1;
    int64_t s = 256 / tiles;
    const int64_t kt = (K + 63) / 64;
    const int64_t by_k = tiles < 16 ? kt / 64 : kt / 20;
    if (by_k < s) s = by_k;
    if (s > kMaxSplits) s = kMaxSplits;
    if (tiles >= 16 && tiles * s < 200) return 1;
    return s < 2 ? 1 : (int)s;
}

inline int64_t splitk_ldw(int64_t N) { return (N + 3) / 4 * 4; }

// Workspace bytes for S splits: S fp32 partial matrices of M x splitk_ldw(N).
// A coarser unit never yields more splits than 64-element K tiles for the
// same request (ceil(8E / ceil(8E / s)) >= ceil(E / ceil(E / s))), so the
// 64-tile count bounds every family's need.
inline size_t splitk_bytes(int64_t M, int64_t N, int splits) {
    return splits <= 1 ? 0 : (size_t)splits * (size_t)M * (size_t)splitk_ldw(N) * 4;
}

inline gemm_status check_workspace(const Common &a, int S, const void *ws, size_t ws_bytes) {
    if (!ws || ws_bytes < splitk_bytes(a.M, a.N, S)) return GEMM_ERR_WORKSPACE;
    if ((uintptr_t)ws % 256 != 0) return GEMM_ERR_MISALIGNED;
    if (splitk_ldw(a.N) * 4 >= kMaxLdBytes) return GEMM_ERR_UNSUPPORTED;
    return GEMM_OK;
}

// Second pass of a split call, on the same stream: D = the S partial slices
// summed in order, plus C, rounded to the output type.
inline gemm_status reduce_splits(const Common &a, const void *ws, int S, hipStream_t s) {
    const bool bf16 = a.out_type == GEMM_OUT_BF16;
    const uintptr_t vb = bf16 ? 8 : 16;
    const int64_t ldw = splitk_ldw(a.N);
    tg::SplitReduceArgs r;
    r.ws = (const float *)ws;
    r.ldw = ldw;
    r.slice = a.M * ldw;
    r.splits = S;
    r.C = a.C;
    r.ldc = a.ldc;
    r.D = a.D;
    r.ldd = a.ldd;
    r.M = (int)a.M;
    r.N = (int)a.N;
    r.vec_c = a.C && ((uintptr_t)a.C % vb) == 0 && a.ldc % 4 == 0;
    r.vec_d = ((uintptr_t)a.D % vb) == 0 && a.ldd % 4 == 0;
    return launched(tg::launch_splitk_reduce(bf16, s, r));
}

}  // namespace tg_api
