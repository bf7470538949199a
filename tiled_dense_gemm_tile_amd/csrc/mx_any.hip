// Kernel instances of the general block-scaled GEMM (any K % 32, any
// alignment, either operand storage order): every element format, output
// type, row alignment and order.
#include "gemm_mx_any.hpp"

namespace tg {

namespace {

template <int FMT, bool OUT_BF16>
hipError_t launch_fmt(bool aligned, bool amn, bool bmn, unsigned grid, hipStream_t s, const MxArgs &q) {
    if (amn && bmn)
        hipLaunchKernelGGL((gemm_mx_any_kernel<FMT, OUT_BF16, false, true, true>), dim3(grid), dim3(256), 0, s, q);
    else if (amn)
        hipLaunchKernelGGL((gemm_mx_any_kernel<FMT, OUT_BF16, false, true, false>), dim3(grid), dim3(256), 0, s, q);
    else if (bmn)
        hipLaunchKernelGGL((gemm_mx_any_kernel<FMT, OUT_BF16, false, false, true>), dim3(grid), dim3(256), 0, s, q);
    else if (aligned)
        hipLaunchKernelGGL((gemm_mx_any_kernel<FMT, OUT_BF16, true>), dim3(grid), dim3(256), 0, s, q);
    else
        hipLaunchKernelGGL((gemm_mx_any_kernel<FMT, OUT_BF16, false>), dim3(grid), dim3(256), 0, s, q);
    return hipGetLastError();
}

template <bool OUT_BF16>
hipError_t launch_out(int fmt, bool aligned, bool amn, bool bmn, unsigned grid, hipStream_t s, const MxArgs &q) {
    switch (fmt) {
    case 0: return launch_fmt<0, OUT_BF16>(aligned, amn, bmn, grid, s, q);
    case 2: return launch_fmt<2, OUT_BF16>(aligned, amn, bmn, grid, s, q);
    case 3: return launch_fmt<3, OUT_BF16>(aligned, amn, bmn, grid, s, q);
    case 4: return launch_fmt<4, OUT_BF16>(aligned, amn, bmn, grid, s, q);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_mx_any(int fmt, bool out_bf16, bool aligned, bool amn, bool bmn, unsigned grid, hipStream_t s,
                         const MxArgs &q) {
    return out_bf16 ? launch_out<true>(fmt, aligned, amn, bmn, grid, s, q)
                    : launch_out<false>(fmt, aligned, amn, bmn, grid, s, q);
}

}  // namespace tg
