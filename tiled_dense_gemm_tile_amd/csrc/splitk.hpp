// Split-K reduction launcher (splitk.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

struct SplitReduceArgs {
    const float *ws;       // slice s at ws + s * slice, M x ldw row-major fp32
    int64_t ldw, slice;
    int splits;
    const void *C;         // output type, M x N, ldc; or null
    int64_t ldc;
    void *D;               // output type, M x N, ldd
    int64_t ldd;
    int M, N;
    bool vec_c, vec_d;     // fp32 C / D rows allow 16-byte (bf16: 8-byte) vectors
};

hipError_t launch_splitk_reduce(bool out_bf16, hipStream_t stream, const SplitReduceArgs &a);

}  // namespace tg
