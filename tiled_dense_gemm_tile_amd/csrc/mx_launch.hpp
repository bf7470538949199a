// Kernel configurations of the block-scaled fp8 GEMM and their launchers;
// one instance translation unit per output type (mx_<out>.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_mxfp8.hpp"
#include "gemm_mx_pp.hpp"
#include "gemm_mx_w4.hpp"

namespace tg {

// id, BM, BN, waves along M, waves along N (two-slot rings)
#define TG_MX_CONFIGS(X)     \
    X(0, 256, 256, 2, 4)     \
    X(1, 256, 256, 2, 2)     \
    X(2, 128, 128, 2, 2)     \
    X(3, 64, 64, 2, 2)

// Three-slot rings (the tile two ahead fetched), numbered after the
// ping-pong and four-wave kernels: id, BM, BN, waves along M, waves along N.
#define TG_MX_DEEP(X)        \
    X(6, 128, 128, 2, 2)     \
    X(7, 64, 64, 2, 2)

struct MxCfgInfo {
    int bm, bn, wm, wn;
};

#define TG_MX_INFO(id, bm, bn, wm, wn) {bm, bn, wm, wn},
// Then the ping-pong kernel (256 x 256, 8 waves) and the four-wave kernel
// (256 x 256, 128 x 128 per wave), both 16x16x128 MFMA, K % 512 == 0.
constexpr MxCfgInfo kMxCfgs[] = {TG_MX_CONFIGS(TG_MX_INFO){256, 256, 2, 4}, {256, 256, 2, 2},
                                  TG_MX_DEEP(TG_MX_INFO)};
#undef TG_MX_INFO
constexpr int kNumMxCfgs = sizeof(kMxCfgs) / sizeof(kMxCfgs[0]);
#define TG_MX_COUNT(...) +1
constexpr int kMxPingPong = 0 TG_MX_CONFIGS(TG_MX_COUNT), kMxFourWave = kMxPingPong + 1;
#undef TG_MX_COUNT
constexpr int kMxDeep128 = kMxFourWave + 1, kMxDeep64 = kMxFourWave + 2;
static_assert(kMxDeep64 + 1 == kNumMxCfgs && kMxDeep128 == 6, "configuration table");

template <bool OUT_BF16>
hipError_t launch_mx(int cfg, unsigned grid, hipStream_t s, const MxArgs &q, const F16Epi &e);

// Split-K partial tiles (fp32, into q.g.ws): the four-wave kernel with SPLIT;
// defined in the fp32-output translation unit.
hipError_t launch_mx_split(unsigned grid, hipStream_t s, const MxArgs &q, const F16Epi &e);

}  // namespace tg

#ifdef TG_MX_INSTANCE
namespace tg {

template <>
hipError_t launch_mx<TG_OUT_BF16>(int cfg, unsigned grid, hipStream_t s, const MxArgs &q, const F16Epi &e) {
    if (cfg == kMxPingPong) {
        hipLaunchKernelGGL((gemm_mx_pp_kernel<TG_OUT_BF16>), dim3(grid), dim3(512), 0, s, q, e);
        return hipGetLastError();
    }
    if (cfg == kMxFourWave) {
        hipLaunchKernelGGL((gemm_mx_w4_kernel<TG_OUT_BF16>), dim3(grid), dim3(256), 0, s, q, e);
        return hipGetLastError();
    }
    switch (cfg) {
#define TG_MX_CASE(id, bm, bn, wm, wn)                                                                  \
    case id:                                                                                            \
        hipLaunchKernelGGL((gemm_mxfp8_kernel<MxCfg<bm, bn, wm, wn>, TG_OUT_BF16>), dim3(grid),         \
                           dim3(wm * wn * 64), 0, s, q, e);                                              \
        break;
        TG_MX_CONFIGS(TG_MX_CASE)
#undef TG_MX_CASE
#define TG_MX_CASE(id, bm, bn, wm, wn)                                                                  \
    case id:                                                                                            \
        hipLaunchKernelGGL((gemm_mxfp8_kernel<MxCfg<bm, bn, wm, wn, 3>, TG_OUT_BF16>), dim3(grid),      \
                           dim3(wm * wn * 64), 0, s, q, e);                                              \
        break;
        TG_MX_DEEP(TG_MX_CASE)
#undef TG_MX_CASE
    default:
        return hipErrorInvalidValue;
    }
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
