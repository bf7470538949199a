// Kernel configurations of the 16-bit-input GEMM and their launchers.
// Each (input type, output type) pair is instantiated in its own
// translation unit (f16_<in>_<out>.hip) so they compile in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_f16.hpp"
#include "gemm_f16_dma.hpp"
#include "gemm_f16_w4.hpp"

namespace tg {

// The configurations the kernel choice (tilegemm.hip, pick_f16_cfg) uses:
// id, BM, BN, BK, waves along M, waves along N, LDS slots for A, for B.
#define TG_F16_DMA_CONFIGS(X)                                                        \
    X(0, 256, 256, 64, 2, 4, 3, 2)   /* rows 4-byte aligned, >= 240 tiles of 256^2 */ \
    X(1, 128, 128, 64, 2, 2, 3, 2)   /* >= 240 tiles of 128^2 (two per CU)         */ \
    X(2, 64, 64, 64, 2, 2, 2, 2)     /* small grids, rows 4- or 8-byte aligned     */ \
    X(3, 128, 128, 64, 2, 2, 3, 3)   /* about one wave of 128^2 tiles              */ \
    X(4, 64, 64, 64, 2, 2, 3, 3)     /* up to 512 tiles of 64^2                    */

// Configurations built with 4-byte global->LDS lanes (rows only 4- or
// 8-byte aligned): 0 only with them, 1 and 2 with both lane widths.
constexpr bool f16_has_lane4(int id) { return id == 0 || id == 1 || id == 2; }
constexpr bool f16_has_lane16(int id) { return id != 0; }

struct F16CfgInfo {
    int bm, bn, bk, wm, wn, na, nb;
};

#define TG_F16_INFO(id, bm, bn, bk, wm, wn, na, nb) {bm, bn, bk, wm, wn, na, nb},
// Then the four-wave kernels (gemm_f16_w4.hpp): 256 x 256 tiles with
// 16-byte rows and with rows only 8-byte aligned (shifted rows), the same
// two with 192 x 256 tiles, and the persistent one (16-byte rows, 256 x 256,
// no C; launched with one workgroup per CU).
constexpr F16CfgInfo kF16DmaCfgs[] = {TG_F16_DMA_CONFIGS(TG_F16_INFO){256, 256, 64, 2, 2, 2, 2},
                                      {256, 256, 64, 2, 2, 2, 2},
                                      {192, 256, 64, 2, 2, 2, 2},
                                      {192, 256, 64, 2, 2, 2, 2},
                                      {256, 256, 64, 2, 2, 2, 2}};
#undef TG_F16_INFO
constexpr int kNumF16DmaCfgs = sizeof(kF16DmaCfgs) / sizeof(kF16DmaCfgs[0]);
constexpr int kF16Wide4Lane = 0, kF16Wide128 = 1, kF16Small64 = 2, kF16Deep128 = 3, kF16Deep64 = 4;
constexpr int kF16FourWave = 5, kF16FourWaveS = 6, kF16FourWave192 = 7, kF16FourWaveS192 = 8;
constexpr int kF16FourWavePersist = 9;
static_assert(kF16FourWavePersist + 1 == kNumF16DmaCfgs, "configuration table");
// Configurations that take rows only 4- or 8-byte aligned.
constexpr bool f16_any_rows(int id) {
    return f16_has_lane4(id) || id == kF16FourWaveS || id == kF16FourWaveS192;
}

// Register-staged fallback for rows only 2-byte aligned: 128 x 128 x 64
// tiles, 4 waves, element-wise loads.
using StagedCfg = TileCfg<128, 128, 64, 2, 2>;

// lane_bytes: 16 or 4 (see f16_has_lane4 / f16_has_lane16).
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
hipError_t launch_f16_staged(unsigned grid, hipStream_t s, const F16Args &p);

}  // namespace tg

// Body of one instance translation unit: define TG_FP16 and TG_OUT_BF16,
// then include this header with TG_F16_INSTANCE defined.
#ifdef TG_F16_INSTANCE
namespace tg {

template <>
hipError_t launch_f16_dma<TG_FP16, TG_OUT_BF16>(int cfg, int lane_bytes, unsigned grid, hipStream_t s,
                                                const F16Args &p, const F16Epi &e) {
    // (the shifted-row kernels take rows 16- or 8-byte aligned, lane_bytes 16 or 4)
    if (cfg == kF16FourWaveS) {
        hipLaunchKernelGGL((gemm_f16_w4t_kernel<TG_FP16, TG_OUT_BF16, true>), dim3(grid), dim3(256), 0, s, p, e);
        return hipGetLastError();
    }
    if (cfg == kF16FourWaveS192) {
        hipLaunchKernelGGL((gemm_f16_w4t_kernel<TG_FP16, TG_OUT_BF16, true, false, false, false, 6>), dim3(grid),
                           dim3(256), 0, s, p, e);
        return hipGetLastError();
    }
    if (cfg == kF16FourWave || cfg == kF16FourWave192 || cfg == kF16FourWavePersist) {
        if (lane_bytes != 16) return hipErrorInvalidValue;
        if (cfg == kF16FourWave)
            hipLaunchKernelGGL((gemm_f16_w4t_kernel<TG_FP16, TG_OUT_BF16>), dim3(grid), dim3(256), 0, s, p, e);
        else if (cfg == kF16FourWave192)
            hipLaunchKernelGGL((gemm_f16_w4t_kernel<TG_FP16, TG_OUT_BF16, false, false, false, false, 6>),
                               dim3(grid), dim3(256), 0, s, p, e);
        else    // (grid: one workgroup per CU, fewer than the tiles; p.C null)
            hipLaunchKernelGGL((gemm_f16_w4t_kernel<TG_FP16, TG_OUT_BF16, false, false, false, false, 8, true>),
                               dim3(grid), dim3(256), 0, s, p, e);
        return hipGetLastError();
    }
    switch (cfg) {
#define TG_F16_CASE(id, bm, bn, bk, wm, wn, na, nb)                                                        \
    case id:                                                                                               \
        if (lane_bytes == 16) {                                                                            \
            if constexpr (f16_has_lane16(id))                                                              \
                hipLaunchKernelGGL(                                                                        \
                    (gemm_f16_dma_kernel<DmaCfg<bm, bn, bk, wm, wn, na, nb>, TG_FP16, TG_OUT_BF16, 16>),   \
                    dim3(grid), dim3(wm * wn * 64), 0, s, p, e);                                           \
            else                                                                                           \
                return hipErrorInvalidValue;                                                               \
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
        hipLaunchKernelGGL((gemm_f16_w4t_kernel<TG_FP16, TG_OUT_BF16, false, false, true, true>), dim3(grid),
                           dim3(256), 0, s, p, e);
    else if (at)
        hipLaunchKernelGGL((gemm_f16_w4t_kernel<TG_FP16, TG_OUT_BF16, false, false, true, false>), dim3(grid),
                           dim3(256), 0, s, p, e);
    else if (bt)
        hipLaunchKernelGGL((gemm_f16_w4t_kernel<TG_FP16, TG_OUT_BF16, false, false, false, true>), dim3(grid),
                           dim3(256), 0, s, p, e);
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
        hipLaunchKernelGGL((gemm_f16_w4t_kernel<TG_FP16, false, true, true>), dim3(grid), dim3(256), 0, s, p, e);
    else
        hipLaunchKernelGGL((gemm_f16_w4t_kernel<TG_FP16, false, false, true>), dim3(grid), dim3(256), 0, s, p, e);
    return hipGetLastError();
#endif
}

template <>
hipError_t launch_f16_staged<TG_FP16, TG_OUT_BF16>(unsigned grid, hipStream_t s, const F16Args &p) {
    hipLaunchKernelGGL((gemm_f16_kernel<StagedCfg, 1, TG_FP16, TG_OUT_BF16>), dim3(grid), dim3(StagedCfg::NT), 0, s,
                       p);
    return hipGetLastError();
}

}  // namespace tg
#endif
