// Launcher of the block-scaled fp4 GEMM; one instance translation unit per
// output type (mx4_<out>.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_mx4_w4.hpp"

namespace tg {

// 256 x 256 tiles, four waves; q.g.lda / q.g.ldb in bytes.
template <bool OUT_BF16>
hipError_t launch_mx4(unsigned grid, hipStream_t s, const MxArgs &q, const F16Epi &e);

// Split-K partial tiles (fp32, into q.g.ws); defined in the fp32-output
// translation unit.
hipError_t launch_mx4_split(unsigned grid, hipStream_t s, const MxArgs &q, const F16Epi &e);

// Persistent: `grid` workgroups (one per CU) walk all tiles; no C, D rows of
// whole 16-byte segments (q.g.N % 4 == 0, e.vec_d).
template <bool OUT_BF16>
hipError_t launch_mx4_persist(unsigned grid, hipStream_t s, const MxArgs &q, const F16Epi &e);

}  // namespace tg

#ifdef TG_MX4_INSTANCE
namespace tg {

template <>
hipError_t launch_mx4<TG_OUT_BF16>(unsigned grid, hipStream_t s, const MxArgs &q, const F16Epi &e) {
    hipLaunchKernelGGL((gemm_mx4_w4_kernel<TG_OUT_BF16>), dim3(grid), dim3(256), 0, s, q, e);
    return hipGetLastError();
}

template <>
hipError_t launch_mx4_persist<TG_OUT_BF16>(unsigned grid, hipStream_t s, const MxArgs &q, const F16Epi &e) {
    hipLaunchKernelGGL((gemm_mx4_w4_kernel<TG_OUT_BF16, kStoreStream, false, true>), dim3(grid), dim3(256), 0, s, q,
                       e);
    return hipGetLastError();
}

#if !TG_OUT_BF16
hipError_t launch_mx4_split(unsigned grid, hipStream_t s, const MxArgs &q, const F16Epi &e) {
    hipLaunchKernelGGL((gemm_mx4_w4_kernel<false, kStoreStream, true>), dim3(grid), dim3(256), 0, s, q, e);
    return hipGetLastError();
}
#endif

}  // namespace tg
#endif
