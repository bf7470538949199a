// C ABI: fp6 operands rewritten as the tile images the packed fp6 kernel
// loads (gemm_mxfp6_pack, gemm_mxfp6_packed_bytes).  The declarations and
// their contract are in include/tilegemm.h.
//
// Layout: a row-major operand of `rows` rows and K elements (K % 128 == 0)
// becomes ceil(rows / 256) x (K / 128) images of 24576 bytes, image (b, t)
// (rows 256 b .. 256 b + 255, elements 128 t .. 128 t + 127) at byte
// (b * (K / 128) + t) * 24576.  Its 16-byte chunk c holds bytes
// 96 t + 16 h .. 96 t + 16 h + 15 of row 256 b + c / 6, with
// h = (c % 6) ^ ((c / 6 >> 3) & 1): the order in which the fp6 kernel's LDS
// slot holds a K tile (96-byte rows, chunk pairs swapped in rows 8 .. 15 of
// every 16), so that each of its load instructions reads 1 KiB of
// consecutive bytes.  Rows past `rows` are zeros.
#include "api.hpp"
#include "common.hpp"

using namespace tg_api;
using tg::u32x4;

namespace {

constexpr int kImage = 24576;        // bytes per image: 256 rows x 96
constexpr int kChunks = kImage / 16;  // 16-byte chunks per image
// Packed operands are addressed with 32-bit offsets: K below 2^23 keeps
// (K / 128 + 2) images of one row block under 2^31 bytes.
constexpr int64_t kMaxPackedK = (int64_t)1 << 23;

// A workgroup per (row block, group of up to four K tiles), grid-stride
// over those: its threads take the group's 16-byte chunks in the order of
// the operand's storage (row by row, up to 384 bytes: whole lines when rows
// are aligned), so each wave reads a few whole rows and writes runs of
// consecutive image chunks (rows follow each other in every image).  V16:
// rows start 16-byte aligned (X aligned, row pitch a multiple of 16), so
// each chunk is one 16-byte load.
template <bool V16>
__global__ void __launch_bounds__(256)
    mx6_pack_kernel(const unsigned char *__restrict__ X, int64_t ldx_bytes, int64_t rows, int nk, int64_t units,
                    u32x4 *__restrict__ P) {
    const int ngroups = (nk + 3) / 4;
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
        const int64_t b = u / ngroups;
        const int t0 = 4 * (int)(u - b * ngroups);
        const int nt = nk - t0 < 4 ? nk - t0 : 4;
        const int per_row = 6 * nt;
        u32x4 *img = P + (b * nk + t0) * kChunks;
#pragma unroll 4
        for (int i = threadIdx.x; i < 256 * per_row; i += 256) {
            const int r = i / per_row, k = i - r * per_row;
            const int t = k / 6, h = k - 6 * t;
            const int64_t row = b * 256 + r;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row < rows) {
                const unsigned char *src = X + row * ldx_bytes + 96 * (t0 + t) + 16 * h;
                if constexpr (V16) {
                    v = *(const u32x4 *)src;
                } else {
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        v[w] = (uint32_t)src[4 * w] | ((uint32_t)src[4 * w + 1] << 8) |
                               ((uint32_t)src[4 * w + 2] << 16) | ((uint32_t)src[4 * w + 3] << 24);
                }
            }
            img[t * kChunks + 6 * r + (h ^ ((r >> 3) & 1))] = v;
        }
    }
}

int64_t packed_bytes(int64_t rows, int64_t K) { return (rows + 255) / 256 * (K / 128) * kImage; }

}  // namespace

extern "C" {

size_t gemm_mxfp6_packed_bytes(int64_t rows, int64_t K) {
    if (rows < 0 || K < 0 || K % 128 != 0 || rows >= kMaxDim || K >= kMaxPackedK) return 0;
    return (size_t)packed_bytes(rows, K);
}

gemm_status gemm_mxfp6_pack(int64_t rows, int64_t K, const void *X, int64_t ldx, void *P, size_t p_bytes,
                            hipStream_t stream) {
    if (rows < 0 || K < 0) return GEMM_ERR_INVALID_SIZE;
    if (rows >= kMaxDim || K >= kMaxPackedK || K % 128 != 0 || ldx % 4 != 0) return GEMM_ERR_UNSUPPORTED;
    if (rows == 0 || K == 0) return GEMM_OK;
    if (ldx < K) return GEMM_ERR_BAD_LD;
    if (!X || !P) return GEMM_ERR_NULL_POINTER;
    if (misaligned(P, 16)) return GEMM_ERR_MISALIGNED;
    const int64_t need = packed_bytes(rows, K);
    if ((int64_t)p_bytes < need) return GEMM_ERR_WORKSPACE;
    const int64_t ldx_bytes = ldx / 4 * 3;
    const int nk = (int)(K / 128);
    const int64_t units = (rows + 255) / 256 * ((nk + 3) / 4);
    const unsigned grid = (unsigned)(units < 65536 ? units : 65536);
    const bool v16 = (uintptr_t)X % 16 == 0 && ldx_bytes % 16 == 0;
    if (v16)
        hipLaunchKernelGGL(mx6_pack_kernel<true>, dim3(grid), dim3(256), 0, stream, (const unsigned char *)X, ldx_bytes,
                           rows, nk, units, (u32x4 *)P);
    else
        hipLaunchKernelGGL(mx6_pack_kernel<false>, dim3(grid), dim3(256), 0, stream, (const unsigned char *)X,
                           ldx_bytes, rows, nk, units, (u32x4 *)P);
    return launched(hipGetLastError());
}

}  // extern "C"
