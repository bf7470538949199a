// The K-contiguous copy kernel of the *_ex_ws entry points (transpose.hpp)
// and gemm_ex_workspace_bytes.
#include "transpose.hpp"

namespace {

// Elements per side of a copy tile: 128-byte source and destination row
// segments (fp6: 192 elements, 144 bytes), so every global access moves
// whole cache lines.
template <int W>
constexpr int copy_tile() { return W == 6 ? 192 : 1024 / W; }

// One workgroup per TE x TE elements: TE source rows (K indices k0 ..
// k0 + TE - 1), elements r0 .. r0 + TE - 1 of each, become TE destination
// rows (r0 ..), elements k0 .. of each.  Each source row segment is staged
// in LDS from the aligned 4-byte word holding its first byte (a word that
// holds a byte of the row lies on that byte's page), rows past K as zeros;
// each destination word is then assembled from the W-bit fields that fall
// in it.  The staged rows are an odd number of words apart, and (W = 16, 8,
// 4: G = 32 / W fields per word) source row e is staged at position
// (e % G) * 32 + e / G, so the rows G j + n that lanes j read for their
// n-th field are consecutive positions: different banks.
template <int W>
__global__ void __launch_bounds__(256) k_contiguous_copy_kernel(const uint8_t *src, int64_t src_row, int64_t valid,
                                                                int K, int rows, int tiles_r, uint8_t *dst,
                                                                int64_t ldd) {
    constexpr int TE = copy_tile<W>();
    constexpr int SB = TE * W / 8;                     // bytes of a row segment
    constexpr int NW = SB / 4 + 2;                     // staged words per source row (alignment slack)
    constexpr int SW = NW | 1;                         // LDS words per staged row (odd)
    constexpr int OW = SB / 4;                         // words of a destination row segment
    constexpr uint32_t MASK = (1u << W) - 1u;
    constexpr int G = 32 / W;                          // fields per word (W = 16, 8, 4)
    auto pos = [](int e) { return W == 6 ? e : (e % G) * (TE / G) + e / G; };
    static_assert(W == 6 || TE / G == 32, "32 rows per field position");
    __shared__ uint32_t stage[TE][SW];
    __shared__ int shift[TE];
    const int r0 = (int)(blockIdx.x % tiles_r) * TE, k0 = (int)(blockIdx.x / tiles_r) * TE;
    const int tid = threadIdx.x;
    // (all of a thread's loads are issued before any of them is stored to
    // LDS: stored one by one, each would wait for its own load)
    constexpr int NL = (TE * NW + 255) / 256;
    uint32_t v[NL];
#pragma unroll
    for (int n = 0; n < NL; ++n) {
        const int idx = tid + 256 * n;
        const int i = idx / NW, w = idx % NW;
        const int k = k0 + i;
        v[n] = 0;
        if (idx < TE * NW && k < K) {
            const uintptr_t row = (uintptr_t)(src + (int64_t)k * src_row);
            const uintptr_t first = row + (uintptr_t)((int64_t)r0 * W / 8);
            const uintptr_t a = (first & ~(uintptr_t)3) + 4 * (uintptr_t)w;
            if (a < row + (uintptr_t)valid) v[n] = *(const uint32_t *)a;
        }
    }
#pragma unroll
    for (int n = 0; n < NL; ++n) {
        const int idx = tid + 256 * n;
        if (idx < TE * NW) stage[pos(idx / NW)][idx % NW] = v[n];
    }
    for (int i = tid; i < TE; i += 256) {
        const uintptr_t first = (uintptr_t)(src + (int64_t)(k0 + i) * src_row) + (uintptr_t)((int64_t)r0 * W / 8);
        shift[pos(i)] = k0 + i < K ? (int)(first & 3) : 0;
    }
    __syncthreads();
    // each thread assembles four consecutive destination words (16 bytes)
    // and stores them at once
    static_assert(OW % 4 == 0, "whole 16-byte pieces");
    for (int idx = tid; idx < TE * OW / 4; idx += 256) {
        const int rr = idx / (OW / 4), j0 = (idx % (OW / 4)) * 4;
        if (r0 + rr >= rows) continue;
        uint32_t out[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int j = j0 + q;
            uint64_t acc = 0;
            const int e_lo = 32 * j / W, e_hi = (32 * j + 31) / W;
#pragma unroll
            for (int n = 0; n < 32 / W + 2; ++n) {
                const int e = e_lo + n;
                if (e > e_hi) break;
                const int pe = pos(e);
                const int bit = 8 * shift[pe] + W * rr;
                const int wi = bit >> 5, b = bit & 31;
                const uint64_t two = (uint64_t)stage[pe][wi] | ((uint64_t)stage[pe][wi + 1] << 32);
                acc |= ((two >> b) & MASK) << (W * e - 32 * j + 32);
            }
            out[q] = (uint32_t)(acc >> 32);
        }
        *(uint4 *)(dst + (int64_t)(r0 + rr) * ldd + (int64_t)k0 * W / 8 + 4 * j0) =
            make_uint4(out[0], out[1], out[2], out[3]);
    }
}

}  // namespace

namespace tg_api {

hipError_t launch_k_contiguous_copy(int bits, const void *src, int64_t lds, int64_t K, int64_t rows, void *dst,
                                    int64_t ldd_bytes, hipStream_t s) {
    const int te = bits == 16 ? copy_tile<16>() : bits == 8 ? copy_tile<8>() : bits == 6 ? copy_tile<6>()
                                                                                    : copy_tile<4>();
    const int64_t tiles_r = (rows + te - 1) / te, tiles_k = (K + te - 1) / te;
    if (tiles_r * tiles_k >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const int64_t src_row = lds * bits / 8, valid = (rows * bits + 7) / 8;
    const dim3 grid((unsigned)(tiles_r * tiles_k)), block(256);
    const uint8_t *sp = (const uint8_t *)src;
    uint8_t *dp = (uint8_t *)dst;
    switch (bits) {
    case 16:
        hipLaunchKernelGGL(k_contiguous_copy_kernel<16>, grid, block, 0, s, sp, src_row, valid, (int)K, (int)rows,
                           (int)tiles_r, dp, ldd_bytes);
        break;
    case 8:
        hipLaunchKernelGGL(k_contiguous_copy_kernel<8>, grid, block, 0, s, sp, src_row, valid, (int)K, (int)rows,
                           (int)tiles_r, dp, ldd_bytes);
        break;
    case 6:
        hipLaunchKernelGGL(k_contiguous_copy_kernel<6>, grid, block, 0, s, sp, src_row, valid, (int)K, (int)rows,
                           (int)tiles_r, dp, ldd_bytes);
        break;
    case 4:
        hipLaunchKernelGGL(k_contiguous_copy_kernel<4>, grid, block, 0, s, sp, src_row, valid, (int)K, (int)rows,
                           (int)tiles_r, dp, ldd_bytes);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tg_api

extern "C" size_t gemm_ex_workspace_bytes(int element_bits, int64_t M, int64_t N, int64_t K, int a_order,
                                          int b_order) {
    using namespace tg_api;
    if ((element_bits != 16 && element_bits != 8 && element_bits != 6 && element_bits != 4) || M < 0 || N < 0 ||
        K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim)
        return 0;
    if (element_bits == 6 && a_order == GEMM_K_CONTIGUOUS && b_order == GEMM_K_CONTIGUOUS)
        return mx6_images_bytes(M, N, K);              // (0 unless K % 128 == 0)
    return (a_order == GEMM_MN_CONTIGUOUS ? kc_copy_bytes(element_bits, M, K) : 0) +
           (b_order == GEMM_MN_CONTIGUOUS ? kc_copy_bytes(element_bits, N, K) : 0);
}
