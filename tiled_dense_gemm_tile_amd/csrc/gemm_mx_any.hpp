// Block-scaled GEMM for every call the tiled kernels do not take: any K that
// is a multiple of 32, rows and scale rows at any byte alignment, all four
// element formats (e4m3, e2m3, e3m2, e2m1), gfx950.
//
// A workgroup of four waves computes a 64 x 64 output tile, each wave a 32 x
// 32 quadrant as 2 x 2 blocks of v_mfma_scale_f32_16x16x128_f8f6f4.  There is
// no LDS: every lane loads its own operand bytes and scale bytes from memory
// with range-checked buffer loads, one 128-wide K step at a time, and feeds
// them straight to the MFMA.  Operand placement (measured): lane l supplies
// row (A) or column (B) l % 16; for fp8 its bytes 0..15 are K elements
// 16 q .. 16 q + 15 and bytes 16..31 elements 64 + 16 q .. of the step, for
// fp6 and fp4 its registers hold the 32 elements of K block q of the step
// (q = l / 16), packed as in memory; the scale of block q comes from lane
// 16 q + l % 16.  K is a multiple of 32, so a lane's bytes always lie in
// whole 32-element blocks: a block at or past K is loaded from an offset
// beyond the resource (zeros, scale code 0), and contributes nothing.  Rows
// past M or N read zeros from the per-tile resources and are not stored.
// Output: lane l of block (i, j) holds rows 4 (l / 16) .. + 3, column l % 16.
//
// AMN / BMN: A (B) is stored MN-contiguous -- K rows of lda (ldb) elements,
// element (m, k) at element k * lda + m, packed along M as along K in the
// K-contiguous form.  Each lane then gathers its 32 elements one by one
// (byte loads at the element's bit offset from a resource over the K
// step's rows) and packs them into its operand registers; elements past K
// or past M (N) are zero.
//
// STAGE (fp8 with a 16-byte-aligned MN-contiguous operand): instead, each K
// step's 128 x 64-byte panel of that operand is loaded by the workgroup with
// 16-byte loads, written to LDS (64-byte rows, one per K row) and read back
// with ds_read_b64_tr_b8, which (probed) gives output lane i of each
// 16-lane group byte i % 8 of the 8-byte reads of lanes 2b + i / 8, b = 0..7:
// when lane s of the group reads K row k + s / 2 at columns 8 (s % 2) .. + 7,
// lane i receives K values k .. k + 7 of column i, in order.  Four such reads
// (K rows 16 q, 16 q + 8, 64 + 16 q, 64 + 16 q + 8) make the lane's 32-byte
// operand in the K-contiguous layout.
#pragma once

#include "common.hpp"
#include "gemm_mxfp8.hpp"

namespace tg {

// FMT: 0 e4m3, 2 e2m3, 3 e3m2, 4 e2m1 (the MFMA's cbsz / blgp codes).
template <int FMT>
struct MxAnyFmt {
    static constexpr int kRegs = FMT == 0 ? 8 : FMT == 4 ? 4 : 6;   // operand registers per lane
};

// One scaled MFMA with scale byte 0 of each scale register; VGPR
// accumulator.  The s_nop keeps VALU writes of the operands (the unaligned
// path assembles them from bytes) out of the MFMA's read window: the
// compiler inserts no wait states around inline asm.
template <int FMT>
__device__ __forceinline__ void mx_any_mfma(f32x4 &acc, const uint32_t (&a)[MxAnyFmt<FMT>::kRegs],
                                            const uint32_t (&b)[MxAnyFmt<FMT>::kRegs], uint32_t sa, uint32_t sb) {
    if constexpr (FMT == 0) {
        const i32x8 va = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)a[4], (int)a[5], (int)a[6], (int)a[7]};
        const i32x8 vb = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], (int)b[4], (int)b[5], (int)b[6], (int)b[7]};
        asm volatile("s_nop 4\n\tv_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
                     : "+v"(acc) : "v"(va), "v"(vb), "v"(sa), "v"(sb));
    } else if constexpr (FMT == 4) {
        const u32x4 va = {a[0], a[1], a[2], a[3]}, vb = {b[0], b[1], b[2], b[3]};
        asm volatile("s_nop 4\n\tv_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
                     : "+v"(acc) : "v"(va), "v"(vb), "v"(sa), "v"(sb));
    } else {
        typedef uint32_t v6 __attribute__((ext_vector_type(6)));
        const v6 va = {a[0], a[1], a[2], a[3], a[4], a[5]}, vb = {b[0], b[1], b[2], b[3], b[4], b[5]};
        if constexpr (FMT == 2)
            asm volatile("s_nop 4\n\tv_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:2 blgp:2"
                         : "+v"(acc) : "v"(va), "v"(vb), "v"(sa), "v"(sb));
        else
            asm volatile("s_nop 4\n\tv_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:3 blgp:3"
                         : "+v"(acc) : "v"(va), "v"(vb), "v"(sa), "v"(sb));
    }
}

// N consecutive dwords at byte offset `off` of resource r, with loads of
// VEC bytes (16, 8 or 4: the offset is a multiple of VEC; 1: each dword
// from four byte loads).  off == kOOB reads zeros.
template <int N, int VEC>
__device__ __forceinline__ void mx_any_load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t *dst) {
    if constexpr (VEC == 16 && N % 4 == 0) {
#pragma unroll
        for (int d = 0; d < N; d += 4) {
            const u32x4 v = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off == kOOB ? kOOB : off + 4 * d, 0, 0));
            dst[d] = v[0], dst[d + 1] = v[1], dst[d + 2] = v[2], dst[d + 3] = v[3];
        }
        return;
    } else if constexpr (VEC >= 8 && N % 2 == 0) {
#pragma unroll
        for (int d = 0; d < N; d += 2) {
            const u32x2 v = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off == kOOB ? kOOB : off + 4 * d, 0, 0));
            dst[d] = v[0], dst[d + 1] = v[1];
        }
        return;
    }
#pragma unroll
    for (int d = 0; d < N; ++d) {
        const uint32_t o = off == kOOB ? kOOB : off + 4 * d;
        if constexpr (VEC >= 4) {
            dst[d] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, o, 0, 0);
        } else {
            uint32_t v = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint32_t ob = o == kOOB ? kOOB : o + b;
                v |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, ob, 0, 0) << (8 * b);
            }
            dst[d] = v;
        }
    }
}

// Bits per element of format FMT.
template <int FMT>
constexpr int mx_any_bits() { return FMT == 0 ? 8 : FMT == 4 ? 4 : 6; }

// The 32 elements of an MN-contiguous operand that lane (row `row` of the
// operand, quarter fq) supplies for the K step at k0 (see the placement
// above), gathered from storage X (K rows of ld_b bytes) into dst.
// `rows`: the operand's M (N).
template <int FMT>
__device__ __forceinline__ void mx_any_gather(const char *X, int64_t ld_b, int rows, int K, int row, int k0, int fq,
                                              uint32_t (&dst)[MxAnyFmt<FMT>::kRegs]) {
    constexpr int BITS = mx_any_bits<FMT>(), R = MxAnyFmt<FMT>::kRegs;
    const int nk = K - k0 < 128 ? K - k0 : 128;         // rows of this K step
    const int64_t row_bytes = ((int64_t)rows * BITS + 7) / 8;
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(X + (int64_t)k0 * ld_b, (uint32_t)((int64_t)(nk - 1) * ld_b + row_bytes));
    const uint32_t bit = (uint32_t)row * BITS;           // the element's bit offset within its storage row
#pragma unroll
    for (int d = 0; d < R; ++d) dst[d] = 0;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        const int dk = FMT == 0 ? (e < 16 ? 16 * fq + e : 64 + 16 * fq + e - 16) : 32 * fq + e;
        const bool ok = k0 + dk < K && row < rows;
        const uint32_t off = ok ? (uint32_t)(dk * ld_b) + (bit >> 3) : kOOB;
        uint32_t v = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
        if constexpr (BITS == 6)
            v |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, ok ? off + 1 : kOOB, 0, 0) << 8;
        const uint32_t code = (v >> (bit & 7)) & ((1u << BITS) - 1);
        const int pos = e * BITS, w = pos / 32, sh = pos % 32;   // constants once unrolled
        dst[w] |= code << sh;
        if (sh + BITS > 32) dst[w + 1] |= code >> (32 - sh);
    }
}

// One K step's 128 x 64-byte panel of an MN-contiguous fp8 operand (storage
// X: K rows of ld_b bytes; columns col0 .. col0 + 63 of `rows`): two 16-byte
// chunks per thread, chunk c = t and t + 256 at panel row c / 4, bytes
// 16 (c % 4) ..  Rows past K read zeros; columns past `rows` feed outputs
// that are not stored.
__device__ __forceinline__ void mx_any_panel_load(const char *X, int64_t ld_b, int rows, int K, int k0, int col0,
                                                  u32x4 (&dst)[2]) {
    const int nk = K - k0 < 128 ? K - k0 : 128;
    const int64_t cols = rows - col0 < 64 ? rows - col0 : 64;
    // through the 16-byte chunk holding the last row's last column (the base
    // is 16-byte aligned, so the chunk stays in its page)
    const uint32_t span = (uint32_t)(((int64_t)(nk - 1) * ld_b + cols + 15) & ~(int64_t)15);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(X + (int64_t)k0 * ld_b + col0, span);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = (int)threadIdx.x + 256 * h;
        const uint32_t off = (uint32_t)((c >> 2) * ld_b) + (c & 3) * 16;
        dst[h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
}

// The lane's fp8 operand for block h of its wave from a staged panel (LDS
// byte address `panel`, 64-byte rows): four transposing reads and their
// wait in one statement, so no register is used before it has landed.
__device__ __forceinline__ void mx_any_panel_frag(uint32_t panel, int col, int fr, int fq, uint32_t (&dst)[8]) {
    const uint32_t a = panel + (uint32_t)((16 * fq + (fr >> 1)) * 64 + col + 8 * (fr & 1));
    u32x2 x0, x1, x2, x3;
    asm volatile("ds_read_b64_tr_b8 %0, %4\n\t"
                 "ds_read_b64_tr_b8 %1, %4 offset:512\n\t"
                 "ds_read_b64_tr_b8 %2, %4 offset:4096\n\t"
                 "ds_read_b64_tr_b8 %3, %4 offset:4608\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3)
                 : "v"(a)
                 : "memory");
    dst[0] = x0[0], dst[1] = x0[1], dst[2] = x1[0], dst[3] = x1[1];
    dst[4] = x2[0], dst[5] = x2[1], dst[6] = x3[0], dst[7] = x3[1];
}

// q.g.lda / q.g.ldb in BYTES; q.g.K in elements (a multiple of 32).
// VEC: the widest load (16, 8, 4 or 1 bytes) every K-contiguous operand
// row allows; fp6 lanes' 24-byte blocks start at multiples of 8 only.
template <int FMT, bool OUT_BF16, int VEC, bool AMN = false, bool BMN = false, bool STAGE = false>
__global__ void __launch_bounds__(256) gemm_mx_any_kernel(MxArgs q) {
    static_assert(!STAGE || (FMT == 0 && (AMN || BMN)), "staged panels: fp8 MN-contiguous operands");
    constexpr int R = MxAnyFmt<FMT>::kRegs;
    __shared__ __attribute__((aligned(16))) char panel[STAGE ? 2 * 128 * 64 : 16];
    constexpr int V = (FMT == 2 || FMT == 3) && VEC > 8 ? 8 : VEC;
    const F16Args &p = q.g;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tm = blockIdx.x % p.tiles_m, tn = blockIdx.x / p.tiles_m;
    const int m0 = tm * 64, n0 = tn * 64;
    const int M = p.M, N = p.N, K = p.K;
    const int nblk = K / 32;
    // scales per row: one per 2^kb_shift blocks of 32 (the scale block width)
    const int kb_shift = q.kb_shift, nsc = ((nblk - 1) >> kb_shift) + 1;
    // bytes of a row's K elements
    const int64_t kbytes = FMT == 0 ? K : FMT == 4 ? K / 2 : K / 4 * 3;
    const __amdgpu_buffer_rsrc_t rA =
        make_rsrc((const char *)p.A + (int64_t)m0 * p.lda, span_bytes(M - m0, (int)kbytes, p.lda, 1));
    const __amdgpu_buffer_rsrc_t rB =
        make_rsrc((const char *)p.B + (int64_t)n0 * p.ldb, span_bytes(N - n0, (int)kbytes, p.ldb, 1));
    const __amdgpu_buffer_rsrc_t rSA =
        make_rsrc((const char *)q.SFA + (int64_t)m0 * q.ldsfa, span_bytes(M - m0, nsc, q.ldsfa, 1));
    const __amdgpu_buffer_rsrc_t rSB =
        make_rsrc((const char *)q.SFB + (int64_t)n0 * q.ldsfb, span_bytes(N - n0, nsc, q.ldsfb, 1));

    const int fr = lane & 15, fq = lane >> 4;
    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // One K step's operands and scales; the loop is software-pipelined over
    // two register sets, so step k + 1's loads are in flight while step k's
    // MFMAs run.
    struct Step {
        uint32_t fa[2][R], fb[2][R], sa[2], sb[2];
        u32x4 pa[2], pb[2];                            // staged panel chunks (STAGE)
    };
    auto load_step = [&](int k0, Step &st) __attribute__((always_inline)) {
        const int blk = k0 / 32 + fq;                  // the K block whose scale this lane supplies
        uint32_t(&fa)[2][R] = st.fa;
        uint32_t(&fb)[2][R] = st.fb;
        uint32_t(&sa)[2] = st.sa;
        uint32_t(&sb)[2] = st.sb;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int ra = 32 * wm + 16 * h + fr, rb = 32 * wn + 16 * h + fr;   // rows within the tile
            if constexpr ((AMN || BMN) && !STAGE) {
                if constexpr (AMN)
                    mx_any_gather<FMT>((const char *)p.A, p.lda, M, K, m0 + ra, k0, fq, fa[h]);
                if constexpr (BMN)
                    mx_any_gather<FMT>((const char *)p.B, p.ldb, N, K, n0 + rb, k0, fq, fb[h]);
            }
            if constexpr (FMT == 0) {
                // elements k0 + 16 q .. + 15 (block k0/32 + q/2) and k0 + 64 + 16 q .. (block k0/32 + 2 + q/2)
                const int e0 = k0 + 16 * fq, e1 = k0 + 64 + 16 * fq;
                const uint32_t oa0 = e0 < K ? (uint32_t)(ra * p.lda + e0) : kOOB;
                const uint32_t oa1 = e1 < K ? (uint32_t)(ra * p.lda + e1) : kOOB;
                const uint32_t ob0 = e0 < K ? (uint32_t)(rb * p.ldb + e0) : kOOB;
                const uint32_t ob1 = e1 < K ? (uint32_t)(rb * p.ldb + e1) : kOOB;
                if constexpr (!AMN) {
                    mx_any_load<4, V>(rA, oa0, fa[h]);
                    mx_any_load<4, V>(rA, oa1, fa[h] + 4);
                }
                if constexpr (!BMN) {
                    mx_any_load<4, V>(rB, ob0, fb[h]);
                    mx_any_load<4, V>(rB, ob1, fb[h] + 4);
                }
            } else {
                // block blk: 16 bytes (fp4) or 24 bytes (fp6)
                const int bb = FMT == 4 ? 16 : 24;
                const uint32_t oa = blk < nblk ? (uint32_t)(ra * p.lda + blk * bb) : kOOB;
                const uint32_t ob = blk < nblk ? (uint32_t)(rb * p.ldb + blk * bb) : kOOB;
                if constexpr (!AMN) mx_any_load<R, V>(rA, oa, fa[h]);
                if constexpr (!BMN) mx_any_load<R, V>(rB, ob, fb[h]);
            }
            const int sc = blk >> kb_shift;            // the block's scale (wider blocks share one)
            const uint32_t osa = blk < nblk ? (uint32_t)(ra * q.ldsfa + sc) : kOOB;
            const uint32_t osb = blk < nblk ? (uint32_t)(rb * q.ldsfb + sc) : kOOB;
            sa[h] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rSA, osa, 0, 0);
            sb[h] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rSB, osb, 0, 0);
        }
        if constexpr (STAGE && AMN) mx_any_panel_load((const char *)p.A, p.lda, M, K, k0, m0, st.pa);
        if constexpr (STAGE && BMN) mx_any_panel_load((const char *)p.B, p.ldb, N, K, k0, n0, st.pb);
    };
    // STAGE: panels to LDS, then each lane's operands by transposing reads
    auto unstage = [&](Step &st) __attribute__((always_inline)) {
        if constexpr (STAGE) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c = (int)threadIdx.x + 256 * h;
                if constexpr (AMN) *(u32x4 *)(panel + c * 16) = st.pa[h];
                if constexpr (BMN) *(u32x4 *)(panel + 8192 + c * 16) = st.pb[h];
            }
            __syncthreads();
            const uint32_t base = (uint32_t)(uintptr_t)panel;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if constexpr (AMN) mx_any_panel_frag(base, 32 * wm + 16 * h, fr, fq, st.fa[h]);
                if constexpr (BMN) mx_any_panel_frag(base + 8192, 32 * wn + 16 * h, fr, fq, st.fb[h]);
            }
            __syncthreads();                           // every read done before the next step's writes
        }
    };
    auto mfma_step = [&](Step &st) __attribute__((always_inline)) {
        unstage(st);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) mx_any_mfma<FMT>(acc[i][j], st.fa[i], st.fb[j], st.sa[i], st.sb[j]);
    };
    Step s0, s1;
    if (K > 0) load_step(0, s0);
    for (int k0 = 0; k0 < K; k0 += 256) {
        if (k0 + 128 < K) load_step(k0 + 128, s1);
        mfma_step(s0);
        if (k0 + 128 >= K) break;
        if (k0 + 256 < K) load_step(k0 + 256, s0);
        mfma_step(s1);
    }
    // the MFMA results before any other instruction reads them
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 3"
                 : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1]));

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + 32 * wn + 16 * j + fr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 32 * wm + 16 * i + 4 * fq + r;
                if (m >= M || n >= N) continue;
                float v = acc[i][j][r];
                if constexpr (OUT_BF16) {
                    if (p.C) {
                        const uint32_t c = ((const uint16_t *)p.C)[(int64_t)m * p.ldc + n];
                        v += __builtin_bit_cast(float, c << 16);
                    }
                    ((uint16_t *)p.D)[(int64_t)m * p.ldd + n] = f32_to_bf16_rne(v);
                } else {
                    if (p.C) v += ((const float *)p.C)[(int64_t)m * p.ldc + n];
                    ((float *)p.D)[(int64_t)m * p.ldd + n] = v;
                }
            }
        }
}

// Launch over ceil(M / 64) x ceil(N / 64) workgroups of 256 threads; fmt as
// FMT above, aligned: every operand row starts at a multiple of 4 bytes.
// vec: the widest load the K-contiguous operand rows allow (16, 8, 4, 1
// bytes); amn / bmn: A / B stored MN-contiguous (then vec only matters with
// stage, as 16 or not); stage: fp8 MN-contiguous operands 16-byte aligned.
hipError_t launch_mx_any(int fmt, bool out_bf16, int vec, bool amn, bool bmn, bool stage, unsigned grid,
                         hipStream_t s, const MxArgs &q);

}  // namespace tg
