// Kernel instances of the general block-scaled GEMM (any K % 32, any
// alignment, either operand storage order): every element format, output
// type, row alignment and order.
#include "gemm_mx_any.hpp"

namespace tg {

namespace {

template <int FMT, bool OUT_BF16>
hipError_t launch_fmt(int vec, bool amn, bool bmn, bool stage, unsigned grid, hipStream_t s, const MxArgs &q) {
    if constexpr (FMT == 0) {
        if (stage) {
            // (vec: that of the K-contiguous operand, 16 or not)
            if (amn && bmn)
                hipLaunchKernelGGL((gemm_mx_any_kernel<0, OUT_BF16, 1, true, true, true>), dim3(grid), dim3(256), 0,
                                   s, q);
            else if (amn && vec >= 16)
                hipLaunchKernelGGL((gemm_mx_any_kernel<0, OUT_BF16, 16, true, false, true>), dim3(grid), dim3(256),
                                   0, s, q);
            else if (amn)
                hipLaunchKernelGGL((gemm_mx_any_kernel<0, OUT_BF16, 1, true, false, true>), dim3(grid), dim3(256), 0,
                                   s, q);
            else if (vec >= 16)
                hipLaunchKernelGGL((gemm_mx_any_kernel<0, OUT_BF16, 16, false, true, true>), dim3(grid), dim3(256),
                                   0, s, q);
            else
                hipLaunchKernelGGL((gemm_mx_any_kernel<0, OUT_BF16, 1, false, true, true>), dim3(grid), dim3(256), 0,
                                   s, q);
            return hipGetLastError();
        }
    }
    if (amn && bmn)
        hipLaunchKernelGGL((gemm_mx_any_kernel<FMT, OUT_BF16, 1, true, true>), dim3(grid), dim3(256), 0, s, q);
    else if (amn)
        hipLaunchKernelGGL((gemm_mx_any_kernel<FMT, OUT_BF16, 1, true, false>), dim3(grid), dim3(256), 0, s, q);
    else if (bmn)
        hipLaunchKernelGGL((gemm_mx_any_kernel<FMT, OUT_BF16, 1, false, true>), dim3(grid), dim3(256), 0, s, q);
    else if (vec >= 16)
        hipLaunchKernelGGL((gemm_mx_any_kernel<FMT, OUT_BF16, 16>), dim3(grid), dim3(256), 0, s, q);
    else if (vec >= 8)
        hipLaunchKernelGGL((gemm_mx_any_kernel<FMT, OUT_BF16, 8>), dim3(grid), dim3(256), 0, s, q);
    else if (vec >= 4)
        hipLaunchKernelGGL((gemm_mx_any_kernel<FMT, OUT_BF16, 4>), dim3(grid), dim3(256), 0, s, q);
    else
        hipLaunchKernelGGL((gemm_mx_any_kernel<FMT, OUT_BF16, 1>), dim3(grid), dim3(256), 0, s, q);
    return hipGetLastError();
}

template <bool OUT_BF16>
hipError_t launch_out(int fmt, int vec, bool amn, bool bmn, bool stage, unsigned grid, hipStream_t s,
                      const MxArgs &q) {
    switch (fmt) {
    case 0: return launch_fmt<0, OUT_BF16>(vec, amn, bmn, stage, grid, s, q);
    case 2: return launch_fmt<2, OUT_BF16>(vec, amn, bmn, false, grid, s, q);
    case 3: return launch_fmt<3, OUT_BF16>(vec, amn, bmn, false, grid, s, q);
    case 4: return launch_fmt<4, OUT_BF16>(vec, amn, bmn, false, grid, s, q);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_mx_any(int fmt, bool out_bf16, int vec, bool amn, bool bmn, bool stage, unsigned grid,
                         hipStream_t s, const MxArgs &q) {
    return out_bf16 ? launch_out<true>(fmt, vec, amn, bmn, stage, grid, s, q)
                    : launch_out<false>(fmt, vec, amn, bmn, stage, grid, s, q);
}

}  // namespace tg
