// K-contiguous copies of operands stored MN-contiguous, for the *_ex_ws
// entry points: an MN-contiguous operand (K rows of R elements) is copied
// into the caller's workspace as R rows of K elements, so the call runs on
// the K-contiguous tiled kernels.  Elements of `bits` bits (16, 8, 6 or 4)
// are packed along a row as in the plain calls: element i at bits
// bits*i .. bits*i + bits - 1 of the row read as a little-endian bit string.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "api.hpp"

namespace tg_api {

// Bytes per row of a copy: whole copy tiles of 128 bytes (fp6: 192
// elements, 144 bytes), which also gives every tiled kernel its row
// alignment (16 bytes; fp6 48).
inline int64_t kc_row_bytes(int bits, int64_t K) {
    const int64_t te = bits == 6 ? 192 : 1024 / bits;
    return (K + te - 1) / te * te * bits / 8;
}

// Workspace bytes of one copy of `rows` rows, rounded up to 256.
inline size_t kc_copy_bytes(int bits, int64_t rows, int64_t K) {
    return ((size_t)rows * (size_t)kc_row_bytes(bits, K) + 255) / 256 * 256;
}

// Enqueues dst (rows x K, K-contiguous, ldd_bytes per row) = the operand at
// src stored MN-contiguous (K rows of `rows` elements, lds elements apart).
hipError_t launch_k_contiguous_copy(int bits, const void *src, int64_t lds, int64_t K, int64_t rows, void *dst,
                                    int64_t ldd_bytes, hipStream_t s);

// The workspace part of an *_ex_ws call whose other arguments the family's
// _ex checks have accepted (K > 0): checks the workspace, then enqueues the
// copies of the MN-contiguous operands and sets the K-contiguous operands
// (element pointers and leading dimensions in elements) the plain call then
// takes.  Returns an error before enqueuing anything.
// fp6 operands both K-contiguous, through a workspace: the tile images of A
// then of B (gemm_mxfp6_pack), each rounded up to 256 bytes; 0 when K is
// not a multiple of 128 (no images).
inline size_t mx6_images_bytes(int64_t M, int64_t N, int64_t K) {
    const size_t a = gemm_mxfp6_packed_bytes(M, K), b = gemm_mxfp6_packed_bytes(N, K);
    if (a == 0 || b == 0) return 0;
    return (a + 255) / 256 * 256 + (b + 255) / 256 * 256;
}

inline gemm_status k_contiguous_operands(int bits, const Common &a, bool amn, bool bmn, void *ws, size_t ws_bytes,
                                         hipStream_t s, const void **A, int64_t *lda, const void **B,
                                         int64_t *ldb) {
    const size_t need = (amn ? kc_copy_bytes(bits, a.M, a.K) : 0) + (bmn ? kc_copy_bytes(bits, a.N, a.K) : 0);
    if (!ws || ws_bytes < need) return GEMM_ERR_WORKSPACE;
    if ((uintptr_t)ws % 256 != 0) return GEMM_ERR_MISALIGNED;
    const int64_t row = kc_row_bytes(bits, a.K);
    if (row >= kMaxLdBytes) return GEMM_ERR_UNSUPPORTED;
    const int64_t ld = row * 8 / bits;                 // elements: whole copy tiles
    char *p = (char *)ws;
    *A = a.A;
    *lda = a.lda;
    *B = a.B;
    *ldb = a.ldb;
    if (amn) {
        gemm_status st = launched(launch_k_contiguous_copy(bits, a.A, a.lda, a.K, a.M, p, row, s));
        if (st != GEMM_OK) return st;
        *A = p;
        *lda = ld;
        p += kc_copy_bytes(bits, a.M, a.K);
    }
    if (bmn) {
        gemm_status st = launched(launch_k_contiguous_copy(bits, a.B, a.ldb, a.K, a.N, p, row, s));
        if (st != GEMM_OK) return st;
        *B = p;
        *ldb = ld;
    }
    return GEMM_OK;
}

}  // namespace tg_api
