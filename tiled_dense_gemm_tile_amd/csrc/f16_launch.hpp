// Kernel configurations of the 16-bit-input GEMM and their launchers.
// Each (input type, output type) pair is instantiated in its own
// translation unit (f16_<in>_<out>.hip) so they compile in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_f16.hpp"
#include "gemm_f16_dma.hpp"
#include "gemm_f16_pp.hpp"
#include "gemm_f16_w4.hpp"

namespace tg {

// Direct-to-LDS configurations: id, BM, BN, BK, waves along M, waves along N,
// LDS slots for A, LDS slots for B.
#define TG_F16_DMA_CONFIGS(X)           \
    X(0, 256, 256, 64, 2, 2, 2, 2)      \
    X(1, 256, 256, 64, 2, 2, 3, 2)      \
    X(2, 256, 256, 64, 2, 4, 2, 2)      \
    X(3, 256, 256, 64, 2, 4, 3, 2)      \
    X(4, 256, 128, 64, 2, 2, 3, 2)      \
    X(5, 128, 128, 64, 2, 2, 2, 2)      \
    X(6, 128, 128, 64, 2, 2, 3, 2)      \
    X(7, 64, 64, 64, 2, 2, 2, 2)

// Deep-ring configurations (A and B both S = 2 .. 4 tiles ahead), numbered
// after the four-wave kernels below.
#define TG_F16_DMA_DEEP(X)              \
    X(17, 128, 128, 64, 2, 2, 3, 3)     \
    X(18, 128, 128, 64, 2, 2, 4, 4)     \
    X(19, 64, 64, 64, 2, 2, 3, 3)       \
    X(20, 64, 64, 64, 2, 2, 5, 5)

// Configurations also built with 4-byte global->LDS lanes (for rows that are
// only 4-byte aligned).
constexpr bool f16_has_lane4(int id) { return id == 3 || id == 6 || id == 7; }

struct F16CfgInfo {
    int bm, bn, bk, wm, wn, na, nb;
};

#define TG_F16_INFO(id, bm, bn, bk, wm, wn, na, nb) {bm, bn, bk, wm, wn, na, nb},
// Then the ping-pong kernels (256 x 256 x 64, 8 waves in two alternating
// groups) with 32x32 and 16x16 MFMA blocks, and the four-wave kernels
// (256 x 256, 128 x 128 per wave) with 32-wide K slabs in rings of 5 or 4
// and with 64-wide K tiles in rings of 2 (A) and 2 or 3 (B); all of these
// take 16-byte lanes only.
constexpr F16CfgInfo kF16DmaCfgs[] = {TG_F16_DMA_CONFIGS(TG_F16_INFO){256, 256, 64, 2, 4, 0, 0},
                                      {256, 256, 64, 2, 4, 0, 0},
                                      {256, 256, 32, 2, 2, 5, 5},
                                      {256, 256, 32, 2, 2, 4, 4},
                                      {256, 256, 64, 2, 2, 2, 2},
                                      {256, 256, 64, 2, 2, 2, 3},
                                      {256, 256, 64, 2, 2, 2, 2},
                                      {256, 256, 64, 2, 2, 2, 3},
                                      {256, 256, 64, 2, 2, 2, 2},
                                      TG_F16_DMA_DEEP(TG_F16_INFO)};
#undef TG_F16_INFO
constexpr int kNumF16DmaCfgs = sizeof(kF16DmaCfgs) / sizeof(kF16DmaCfgs[0]);
#define TG_F16_COUNT(...) +1
constexpr int kF16PingPong32 = 0 TG_F16_DMA_CONFIGS(TG_F16_COUNT), kF16PingPong16 = kF16PingPong32 + 1;
#undef TG_F16_COUNT
constexpr int kF16FourWave5 = kF16PingPong32 + 2, kF16FourWave4 = kF16PingPong32 + 3;
constexpr int kF16FourWaveT22 = kF16PingPong32 + 4, kF16FourWaveT23 = kF16PingPong32 + 5;
constexpr int kF16FourWaveB22 = kF16PingPong32 + 6, kF16FourWaveB23 = kF16PingPong32 + 7;
// The balanced four-wave kernel for rows that are only 8-byte aligned.
constexpr int kF16FourWaveS = kF16PingPong32 + 8;
constexpr int kF16Deep2 = kF16FourWaveS + 1, kF16Deep3 = kF16FourWaveS + 2;
constexpr int kF16Deep64x2 = kF16FourWaveS + 3, kF16Deep64x4 = kF16FourWaveS + 4;
static_assert(kF16Deep64x4 + 1 == kNumF16DmaCfgs && kF16Deep2 == 17, "configuration table");
// Configurations that take rows only 4- or 8-byte aligned.
constexpr bool f16_any_rows(int id) { return f16_has_lane4(id) || id == kF16FourWaveS; }

// Register-staged fallback (any alignment): 128 x 128 x 64 tiles, 4 waves.
using StagedCfg = TileCfg<128, 128, 64, 2, 2>;

// lane_bytes: 16 or 4 (4 only for ids with f16_has_lane4).
template <bool FP16, bool OUT_BF16>
hipError_t launch_f16_dma(int cfg, int lane_bytes, unsigned grid, hipStream_t s, const F16Args &p,
                          const F16Epi &e);

// Operands stored MN-contiguous (at: A as K x M, bt: B as K x N; at least
// one set): the four-wave kernel, 16-byte rows, 256 x 256 tiles.
template <bool FP16, bool OUT_BF16>
hipError_t launch_f16_mn(bool at, bool bt, unsigned grid, hipStream_t s, const F16Args &p, const F16Epi &e);

// Split-K partial products (fp32 partial tiles into p.ws; instantiated in
// the fp32-output translation units): the four-wave kernel, 16-byte rows
// (sh false) or 8-byte rows (sh true).
template <bool FP16, bool OUT_BF16>
hipError_t launch_f16_split(bool sh, unsigned grid, hipStream_t s, const F16Args &p, const F16Epi &e);

template <bool FP16, bool OUT_BF16>
hipError_t launch_f16_staged(int vec, unsigned grid, hipStream_t s, const F16Args &p);

}  // namespace tg

// Body of one instance translation unit: define TG_FP16 and TG_OUT_BF16,
// then include this header with TG_F16_INSTANCE defined.
#ifdef TG_F16_INSTANCE
namespace tg {

template <>
hipError_t launch_f16_dma<TG_FP16, TG_OUT_BF16>(int cfg, int lane_bytes, unsigned grid, hipStream_t s,
                                                const F16Args &p, const F16Epi &e) {
    if (cfg == kF16PingPong32 || cfg == kF16PingPong16) {
        if (lane_bytes != 16) return hipErrorInvalidValue;
        if (cfg == kF16PingPong32)
            hipLaunchKernelGGL((gemm_f16_pp_kernel<32, TG_FP16, TG_OUT_BF16>), dim3(grid), dim3(512), 0, s, p, e);
        else
            hipLaunchKernelGGL((gemm_f16_pp_kernel<16, TG_FP16, TG_OUT_BF16>), dim3(grid), dim3(512), 0, s, p, e);
        return hipGetLastError();
    }
    if (cfg == kF16FourWave5 || cfg == kF16FourWave4) {
        if (lane_bytes != 16) return hipErrorInvalidValue;
        if (cfg == kF16FourWave5)
            hipLaunchKernelGGL((gemm_f16_w4_kernel<5, TG_FP16, TG_OUT_BF16>), dim3(grid), dim3(256), 0, s, p, e);
        else
            hipLaunchKernelGGL((gemm_f16_w4_kernel<4, TG_FP16, TG_OUT_BF16>), dim3(grid), dim3(256), 0, s, p, e);
        return hipGetLastError();
    }
    if (cfg == kF16FourWaveS) {
        // (lane_bytes 16 or 4: rows 16- or 8-byte aligned)
        hipLaunchKernelGGL((gemm_f16_w4t_kernel<2, 2, TG_FP16, TG_OUT_BF16, 1, kStoreStream, true>), dim3(grid),
                           dim3(256), 0, s, p, e);
        return hipGetLastError();
    }
    if (cfg == kF16FourWaveB22 || cfg == kF16FourWaveB23) {
        if (lane_bytes != 16) return hipErrorInvalidValue;
        if (cfg == kF16FourWaveB22)
            hipLaunchKernelGGL((gemm_f16_w4t_kernel<2, 2, TG_FP16, TG_OUT_BF16, 1>), dim3(grid), dim3(256), 0, s, p, e);
        else
            hipLaunchKernelGGL((gemm_f16_w4t_kernel<2, 3, TG_FP16, TG_OUT_BF16, 1>), dim3(grid), dim3(256), 0, s, p, e);
        return hipGetLastError();
    }
    if (cfg == kF16FourWaveT22 || cfg == kF16FourWaveT23) {
        if (lane_bytes != 16) return hipErrorInvalidValue;
        if (cfg == kF16FourWaveT22)
            hipLaunchKernelGGL((gemm_f16_w4t_kernel<2, 2, TG_FP16, TG_OUT_BF16>), dim3(grid), dim3(256), 0, s, p, e);
        else
            hipLaunchKernelGGL((gemm_f16_w4t_kernel<2, 3, TG_FP16, TG_OUT_BF16>), dim3(grid), dim3(256), 0, s, p, e);
        return hipGetLastError();
    }
    switch (cfg) {
#define TG_F16_CASE(id, bm, bn, bk, wm, wn, na, nb)                                                        \
    case id:                                                                                               \
        if (lane_bytes == 16) {                                                                            \
            hipLaunchKernelGGL(                                                                            \
                (gemm_f16_dma_kernel<DmaCfg<bm, bn, bk, wm, wn, na, nb>, TG_FP16, TG_OUT_BF16, 16>),       \
                dim3(grid), dim3(wm * wn * 64), 0, s, p, e);                                               \
        } else {                                                                                           \
            if constexpr (f16_has_lane4(id))                                                               \
                hipLaunchKernelGGL(                                                                        \
                    (gemm_f16_dma_kernel<DmaCfg<bm, bn, bk, wm, wn, na, nb>, TG_FP16, TG_OUT_BF16, 4>),    \
                    dim3(grid), dim3(wm * wn * 64), 0, s, p, e);                                           \
            else                                                                                           \
                return hipErrorInvalidValue;                                                               \
        }                                                                                                  \
        break;
        TG_F16_DMA_CONFIGS(TG_F16_CASE)
        TG_F16_DMA_DEEP(TG_F16_CASE)
#undef TG_F16_CASE
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <>
hipError_t launch_f16_mn<TG_FP16, TG_OUT_BF16>(bool at, bool bt, unsigned grid, hipStream_t s, const F16Args &p,
                                               const F16Epi &e) {
    if (at && bt)
        hipLaunchKernelGGL((gemm_f16_w4t_kernel<2, 2, TG_FP16, TG_OUT_BF16, 1, kStoreStream, false, false, true, true>),
                           dim3(grid), dim3(256), 0, s, p, e);
    else if (at)
        hipLaunchKernelGGL((gemm_f16_w4t_kernel<2, 2, TG_FP16, TG_OUT_BF16, 1, kStoreStream, false, false, true, false>),
                           dim3(grid), dim3(256), 0, s, p, e);
    else if (bt)
        hipLaunchKernelGGL((gemm_f16_w4t_kernel<2, 2, TG_FP16, TG_OUT_BF16, 1, kStoreStream, false, false, false, true>),
                           dim3(grid), dim3(256), 0, s, p, e);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <>
hipError_t launch_f16_split<TG_FP16, TG_OUT_BF16>(bool sh, unsigned grid, hipStream_t s, const F16Args &p,
                                                   const F16Epi &e) {
#if TG_OUT_BF16
    (void)sh, (void)grid, (void)s, (void)p, (void)e;
    return hipErrorInvalidValue;
#else
    if (sh)
        hipLaunchKernelGGL((gemm_f16_w4t_kernel<2, 2, TG_FP16, false, 1, kStoreStream, true, true>), dim3(grid),
                           dim3(256), 0, s, p, e);
    else
        hipLaunchKernelGGL((gemm_f16_w4t_kernel<2, 2, TG_FP16, false, 1, kStoreStream, false, true>), dim3(grid),
                           dim3(256), 0, s, p, e);
    return hipGetLastError();
#endif
}

template <>
hipError_t launch_f16_staged<TG_FP16, TG_OUT_BF16>(int vec, unsigned grid, hipStream_t s, const F16Args &p) {
    switch (vec) {
    case 8: hipLaunchKernelGGL((gemm_f16_kernel<StagedCfg, 8, TG_FP16, TG_OUT_BF16>), dim3(grid), dim3(StagedCfg::NT), 0, s, p); break;
    case 4: hipLaunchKernelGGL((gemm_f16_kernel<StagedCfg, 4, TG_FP16, TG_OUT_BF16>), dim3(grid), dim3(StagedCfg::NT), 0, s, p); break;
    case 2: hipLaunchKernelGGL((gemm_f16_kernel<StagedCfg, 2, TG_FP16, TG_OUT_BF16>), dim3(grid), dim3(StagedCfg::NT), 0, s, p); break;
    case 1: hipLaunchKernelGGL((gemm_f16_kernel<StagedCfg, 1, TG_FP16, TG_OUT_BF16>), dim3(grid), dim3(StagedCfg::NT), 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tg
#endif
