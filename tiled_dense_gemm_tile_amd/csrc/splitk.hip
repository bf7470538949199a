// Split-K reduction: D = sum over splits s of P_s + C, where P_s is the fp32
// partial product of K range s (an M x ldw row-major slice of the caller's
// workspace, written by the four-wave kernel in split mode).  The slices
// are added in split order, then C, so the result does not depend on which
// workgroup finished first.  Memory-bound: one 16-byte vector (four columns
// of a row) per thread.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "splitk.hpp"

namespace tg {

template <bool OUT_BF16>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(SplitReduceArgs a) {
    const int64_t nvec = (int64_t)(a.N + 3) / 4;
    const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (v >= (int64_t)a.M * nvec) return;
    const int row = (int)(v / nvec);
    const int col = (int)(v - (int64_t)row * nvec) * 4;
    // partial slices: 16-byte aligned rows (ldw % 4 == 0, 256-byte aligned base)
    const float *w = a.ws + (int64_t)row * a.ldw + col;
    f32x4 s = *(const f32x4 *)w;
    for (int k = 1; k < a.splits; ++k) s += *(const f32x4 *)(w + (int64_t)k * a.slice);
    const int nv = a.N - col < 4 ? a.N - col : 4;      // columns of this vector inside N
    if (a.C) {
        if constexpr (OUT_BF16) {
            const uint16_t *c = (const uint16_t *)a.C + (int64_t)row * a.ldc + col;
            for (int i = 0; i < nv; ++i) s[i] += __builtin_bit_cast(float, (uint32_t)c[i] << 16);
        } else {
            const float *c = (const float *)a.C + (int64_t)row * a.ldc + col;
            if (nv == 4 && a.vec_c) {
                s += *(const f32x4 *)c;
            } else {
                for (int i = 0; i < nv; ++i) s[i] += c[i];
            }
        }
    }
    if constexpr (OUT_BF16) {
        uint16_t *d = (uint16_t *)a.D + (int64_t)row * a.ldd + col;
        if (nv == 4 && a.vec_d) {
            *(u32x2 *)d = u32x2{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
        } else {
            for (int i = 0; i < nv; ++i) d[i] = f32_to_bf16_rne(s[i]);
        }
    } else {
        float *d = (float *)a.D + (int64_t)row * a.ldd + col;
        if (nv == 4 && a.vec_d) {
            *(f32x4 *)d = s;
        } else {
            for (int i = 0; i < nv; ++i) d[i] = s[i];
        }
    }
}

hipError_t launch_splitk_reduce(bool out_bf16, hipStream_t stream, const SplitReduceArgs &a) {
    const int64_t nvec = (int64_t)a.M * ((a.N + 3) / 4);
    const unsigned grid = (unsigned)((nvec + 255) / 256);
    if (out_bf16)
        hipLaunchKernelGGL((splitk_reduce_kernel<true>), dim3(grid), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((splitk_reduce_kernel<false>), dim3(grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tg
