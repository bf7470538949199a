// Launcher of the block-scaled fp6 GEMM; one instance translation unit per
// output type (mx6_<out>.hip), each holding both fp6 formats.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_mx6_w4.hpp"

namespace tg {

// 256 x 256 tiles, four waves; q.g.lda / q.g.ldb in bytes; e3m2 selects
// the E3M2 format (else E2M3).
template <bool OUT_BF16>
hipError_t launch_mx6(bool e3m2, unsigned grid, hipStream_t s, const MxArgs &q, const F16Epi &e);

// Split-K partial tiles (fp32, into q.g.ws); defined in the fp32-output
// translation unit.
hipError_t launch_mx6_split(bool e3m2, unsigned grid, hipStream_t s, const MxArgs &q, const F16Epi &e);

// Persistent: `grid` workgroups (one per CU) walk all tiles; no C, D rows of
// whole 16-byte segments (q.g.N % 4 == 0, e.vec_d).
template <bool OUT_BF16>
hipError_t launch_mx6_persist(bool e3m2, unsigned grid, hipStream_t s, const MxArgs &q, const F16Epi &e);

// A and B given as their tile images (gemm_mxfp6_pack): one workgroup per
// tile, or with `persist` (conditions as launch_mx6_persist) `grid`
// workgroups walking all tiles.
template <bool OUT_BF16>
hipError_t launch_mx6_packed(bool e3m2, bool persist, unsigned grid, hipStream_t s, const MxArgs &q,
                             const F16Epi &e);

}  // namespace tg

#ifdef TG_MX6_INSTANCE
namespace tg {

template <>
hipError_t launch_mx6<TG_OUT_BF16>(bool e3m2, unsigned grid, hipStream_t s, const MxArgs &q, const F16Epi &e) {
    if (e3m2)
        hipLaunchKernelGGL((gemm_mx6_w4_kernel<TG_OUT_BF16, 3>), dim3(grid), dim3(256), 0, s, q, e);
    else
        hipLaunchKernelGGL((gemm_mx6_w4_kernel<TG_OUT_BF16, 2>), dim3(grid), dim3(256), 0, s, q, e);
    return hipGetLastError();
}

template <>
hipError_t launch_mx6_persist<TG_OUT_BF16>(bool e3m2, unsigned grid, hipStream_t s, const MxArgs &q,
                                           const F16Epi &e) {
    if (e3m2)
        hipLaunchKernelGGL((gemm_mx6_w4_kernel<TG_OUT_BF16, 3, kStoreStream, false, true>), dim3(grid), dim3(256), 0,
                           s, q, e);
    else
        hipLaunchKernelGGL((gemm_mx6_w4_kernel<TG_OUT_BF16, 2, kStoreStream, false, true>), dim3(grid), dim3(256), 0,
                           s, q, e);
    return hipGetLastError();
}

template <>
hipError_t launch_mx6_packed<TG_OUT_BF16>(bool e3m2, bool persist, unsigned grid, hipStream_t s, const MxArgs &q,
                                          const F16Epi &e) {
    if (e3m2 && persist)
        hipLaunchKernelGGL((gemm_mx6_w4_kernel<TG_OUT_BF16, 3, kStoreStream, false, true, true>), dim3(grid),
                           dim3(256), 0, s, q, e);
    else if (e3m2)
        hipLaunchKernelGGL((gemm_mx6_w4_kernel<TG_OUT_BF16, 3, kStoreStream, false, false, true>), dim3(grid),
                           dim3(256), 0, s, q, e);
    else if (persist)
        hipLaunchKernelGGL((gemm_mx6_w4_kernel<TG_OUT_BF16, 2, kStoreStream, false, true, true>), dim3(grid),
                           dim3(256), 0, s, q, e);
    else
        hipLaunchKernelGGL((gemm_mx6_w4_kernel<TG_OUT_BF16, 2, kStoreStream, false, false, true>), dim3(grid),
                           dim3(256), 0, s, q, e);
    return hipGetLastError();
}

#if !TG_OUT_BF16
hipError_t launch_mx6_split(bool e3m2, unsigned grid, hipStream_t s, const MxArgs &q, const F16Epi &e) {
    if (e3m2)
        hipLaunchKernelGGL((gemm_mx6_w4_kernel<false, 3, kStoreStream, true>), dim3(grid), dim3(256), 0, s, q, e);
    else
        hipLaunchKernelGGL((gemm_mx6_w4_kernel<false, 2, kStoreStream, true>), dim3(grid), dim3(256), 0, s, q, e);
    return hipGetLastError();
}
#endif

}  // namespace tg
#endif
