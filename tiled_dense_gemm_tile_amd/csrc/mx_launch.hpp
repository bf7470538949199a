// Kernel configurations of the block-scaled fp8 GEMM and their launchers;
// one instance translation unit per output type (mx_<out>.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_mxfp8.hpp"
#include "gemm_mx_w4.hpp"

namespace tg {

// The configurations the kernel choice (mx_api.hip, dispatch_mx) uses:
// id, BM, BN, waves along M, waves along N, ring slots.
#define TG_MX_CONFIGS(X)        \
    X(0, 256, 256, 2, 2, 2)     \
    X(1, 128, 128, 2, 2, 2)     \
    X(2, 128, 128, 2, 2, 3)     \
    X(3, 64, 64, 2, 2, 3)

struct MxCfgInfo {
    int bm, bn, wm, wn;
};

#define TG_MX_INFO(id, bm, bn, wm, wn, ns) {bm, bn, wm, wn},
// Then the four-wave kernel (256 x 256, 128 x 128 per wave, 16x16x128
// MFMA, K % 512 == 0, 16-byte scale rows; gemm_mx_w4.hpp), one workgroup
// per tile or persistent (one per CU walking the tiles).
constexpr MxCfgInfo kMxCfgs[] = {TG_MX_CONFIGS(TG_MX_INFO){256, 256, 2, 2}, {256, 256, 2, 2}};
#undef TG_MX_INFO
constexpr int kNumMxCfgs = sizeof(kMxCfgs) / sizeof(kMxCfgs[0]);
constexpr int kMxWide = 0, kMx128 = 1, kMxDeep128 = 2, kMxDeep64 = 3, kMxFourWave = 4, kMxFourWavePersist = 5;
static_assert(kMxFourWavePersist + 1 == kNumMxCfgs, "configuration table");

template <bool OUT_BF16>
hipError_t launch_mx(int cfg, unsigned grid, hipStream_t s, const MxArgs &q, const F16Epi &e);

// The persistent four-wave kernel: `grid` workgroups walk all tiles.
template <bool OUT_BF16>
hipError_t launch_mx_persist(unsigned grid, hipStream_t s, const MxArgs &q, const F16Epi &e);

// Split-K partial tiles (fp32, into q.g.ws): the four-wave kernel with SPLIT;
// defined in the fp32-output translation unit.
hipError_t launch_mx_split(unsigned grid, hipStream_t s, const MxArgs &q, const F16Epi &e);

}  // namespace tg

#ifdef TG_MX_INSTANCE
namespace tg {

template <>
hipError_t launch_mx<TG_OUT_BF16>(int cfg, unsigned grid, hipStream_t s, const MxArgs &q, const F16Epi &e) {
    if (cfg == kMxFourWave) {
        hipLaunchKernelGGL((gemm_mx_w4_kernel<TG_OUT_BF16>), dim3(grid), dim3(256), 0, s, q, e);
        return hipGetLastError();
    }
    switch (cfg) {
#define TG_MX_CASE(id, bm, bn, wm, wn, ns)                                                              \
    case id:                                                                                            \
        hipLaunchKernelGGL((gemm_mxfp8_kernel<MxCfg<bm, bn, wm, wn, ns>, TG_OUT_BF16>), dim3(grid),     \
                           dim3(wm * wn * 64), 0, s, q, e);                                              \
        break;
        TG_MX_CONFIGS(TG_MX_CASE)
#undef TG_MX_CASE
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <>
hipError_t launch_mx_persist<TG_OUT_BF16>(unsigned grid, hipStream_t s, const MxArgs &q, const F16Epi &e) {
    hipLaunchKernelGGL((gemm_mx_w4_kernel<TG_OUT_BF16, kStoreStream, false, true>), dim3(grid), dim3(256), 0, s, q, e);
    return hipGetLastError();
}

#if !TG_OUT_BF16
hipError_t launch_mx_split(unsigned grid, hipStream_t s, const MxArgs &q, const F16Epi &e) {
    hipLaunchKernelGGL((gemm_mx_w4_kernel<false, kStoreStream, true>), dim3(grid), dim3(256), 0, s, q, e);
    return hipGetLastError();
}
#endif

}  // namespace tg
#endif
