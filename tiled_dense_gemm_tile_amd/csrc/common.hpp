// Device-side building blocks shared by the gfx950 GEMM kernels:
// vector types, buffer resources, the XOR-swizzled LDS layout and the
// XCD-aware tile order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace tg {

// f(integral_constant<int, I>) for I = B .. E - 1, each call its own
// instantiation: the indices are constant expressions however large the body.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>());
        static_for<B + 1, E>(f);
    }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Offset that lies beyond every buffer resource built here (each resource
// covers less than 2^31 bytes): a buffer load from it returns zero and a
// buffer store to it is dropped.  This is how remainder tiles are predicated.
constexpr uint32_t kOOB = 0x80000000u;

// Cache-policy bits of the D stores of the full-grid kernels: nt
// (non-temporal, streamed past the caches).  A full grid writes tens to
// hundreds of MB of D that nothing re-reads during the launch; streamed, it
// no longer evicts the A and B panels the other tiles are still reading
// (measured: 16384 x 14336 x 4096 bf16 -> bf16 12 % faster, 8192^3 fp8 ->
// fp32 about 10 %, 4096^3 bf16 with fp32 C and D about 2 %).
constexpr int kStoreStream = 2;

// Third dword of a raw buffer resource on gfx9-family parts: 32-bit data
// format, no swizzle, no index stride.
constexpr int kRsrcFlags = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRsrcFlags);
}

// Bytes a resource rooted at row `r0` of a rows x cols matrix (leading
// dimension ld, element size es) must cover: up to the end of the last
// in-range element.  Clamped below 2^31 (the host guarantees the clamp is
// never reached for addressable elements).
__device__ __forceinline__ uint32_t span_bytes(int rows_left, int cols, int64_t ld, int es) {
    if (rows_left <= 0 || cols <= 0) return 0;
    int64_t b = ((int64_t)(rows_left - 1) * ld + cols) * es;
    return b >= (int64_t)kOOB ? kOOB - 1 : (uint32_t)b;
}

// fp32 -> bf16, round to nearest even (NaN stays NaN), two at a time with
// gfx950's packed conversion (v_cvt_pk_bf16_f32): lo in bits 0..15.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) { return (uint16_t)pack_bf16x2(x, 0.0f); }

// ---- LDS layout --------------------------------------------------------
// A tile of R rows x BK 16-bit elements is stored row after row, each row
// BK*2 bytes split into 16-byte chunks.  Logical chunk c of row r sits at
// physical chunk c ^ swz(r).  The swizzle makes the MFMA fragment reads
// (lanes l..l+7 or l..l+15 read the same chunk of consecutive rows)
// conflict-free whether the LDS serves 128 or 256 bytes per cycle, while a
// row's own chunks stay a permutation of the row (contiguous fills).
template <int CPR>
__device__ __forceinline__ int swz(int r) {
    if constexpr (CPR == 8) {
        return (r & 7) ^ ((r >> 3) & 1);
    } else if constexpr (CPR == 4) {
        return ((r >> 1) ^ (r >> 3)) & 3;
    } else {
        return 0;
    }
}

// Swizzle of 128-byte rows for 16x16x32 fragment reads (each quarter-wave
// reads one chunk of 16 consecutive rows): logical chunk c of row r sits at
// physical chunk c ^ (r & 7).  Measured free of bank conflicts for that
// pattern on gfx950, where swz<8> (tuned for the 32x32 pattern) is not.
__device__ __forceinline__ int swz16(int r) { return r & 7; }

// ---- tile order ---------------------------------------------------------
// Workgroup w is dispatched to XCD (w mod 8).  Renumber so each XCD owns a
// contiguous range of logical tile ids, then walk tiles in groups of
// `group_m` tile-rows so the tiles resident on one XCD at a time form a
// compact block that shares A rows and B columns in that XCD's L2.
__device__ __forceinline__ void tile_order(int wg, int nwg, int tiles_m, int tiles_n, int group_m,
                                           int &tm, int &tn) {
    const int q = nwg >> 3, r = nwg & 7, x = wg & 7;
    const int lid = x * q + (x < r ? x : r) + (wg >> 3);
    const int group_size = group_m * tiles_n;
    const int group = lid / group_size;
    const int first_m = group * group_m;
    const int gm = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int in_group = lid - group * group_size;
    tm = first_m + in_group % gm;
    tn = in_group / gm;
}

// Split-K work item of workgroup wg out of nwg = tiles * splits: the same
// The kernel's first argument, a T at offset 0 of the kernarg segment, read
// again through a pointer the compiler cannot see through: a persistent
// kernel reads what it needs for its next tile this way, so those values are
// not held in scalar registers through its main loop.  (The cast back to a
// generic pointer keeps the loads scalar constant-memory loads.)
template <class T>
__device__ __forceinline__ T kernel_arg0_reloaded() {
    using KPtr = const __attribute__((address_space(4))) T *;
    KPtr k = (KPtr)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(k));
    return *(const T *)k;
}

// XCD renumbering as tile_order, then split = id / tiles and the tile from
// id % tiles in groups of `group_m` tile-rows, so the workgroups running
// together on an XCD share the K range of their A and B panels.
__device__ __forceinline__ void tile_order_split(int wg, int nwg, int tiles_m, int tiles_n, int group_m, int &tm,
                                                 int &tn, int &split) {
    const int q = nwg >> 3, r = nwg & 7, x = wg & 7;
    const int lid = x * q + (x < r ? x : r) + (wg >> 3);
    const int tiles = tiles_m * tiles_n;
    split = lid / tiles;
    const int in_split = lid - split * tiles;
    const int group_size = group_m * tiles_n;
    const int group = in_split / group_size;
    const int first_m = group * group_m;
    const int gm = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int in_group = in_split - group * group_size;
    tm = first_m + in_group % gm;
    tn = in_group / gm;
}

}  // namespace tg
