/*
 * tilegemm.h -- C ABI of the tiled matrix multiply-accumulate D = A.B + C
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation (page "Tensor Core 数据布局的演进" / Evolution of Tensor Core
 * data layouts, section 概览, the equation D = AB + C; section
 * 一个具体的 fragment 映射 for the operand convention):
 *
 *     D[m][n] = C[m][n] + sum_{k<K} a(m,k) * b(k,n)     0 <= m < M, 0 <= n < N
 *
 * Layouts (all sizes and leading dimensions in ELEMENTS, not bytes):
 *   A  M x K row-major:                      a(m,k) = A[m*lda + k]
 *   B  K x N column-major, i.e. stored as N rows of K elements:
 *                                            b(k,n) = B[n*ldb + k]
 *   C  M x N row-major, element type = the output type, or NULL (C = 0)
 *   D  M x N row-major, element type given by out_type
 * Products are formed exactly and accumulated in fp32.  Summation order
 * inside the library is unspecified; integer-valued inputs whose partial sums
 * stay below 2^24 in magnitude give exact results.
 *
 * Calling convention shared by every entry point:
 *   - The caller owns every buffer (device memory) and the stream.  The
 *     library allocates nothing, keeps no per-call state and is re-entrant.
 *   - Calls are asynchronous: the work is enqueued on `stream` (NULL = the
 *     default stream) and the call returns without synchronising.
 *   - Arguments are validated before anything is enqueued.  On any status
 *     other than GEMM_OK and GEMM_ERR_HIP nothing was enqueued and D is
 *     untouched; GEMM_ERR_HIP (a failed launch) can follow kernels of the
 *     same call already enqueued (the calls that run a copy, packing or
 *     reduction kernel beside the GEMM).
 *   - M == 0 or N == 0: GEMM_OK, nothing is launched.  K == 0: D = C (or 0).
 *   - Leading dimensions: lda >= K, ldb >= K, ldc >= N, ldd >= N, else
 *     GEMM_ERR_BAD_LD.  Any such ld is accepted; the load width follows the
 *     alignment of pointers, leading dimensions and K (16-byte vectors when
 *     everything is a multiple of 16 bytes, narrower otherwise).  The
 *     remainder of M, N and K that does not fill a tile is predicated (page
 *     "（二）CUTLASS —— 掌握 TMA", section on remainder tiles: out-of-range
 *     elements are never read or written); unlike the TMA rule on that page,
 *     leading dimensions need no 16-byte padding.
 *   - Pointers: A and B must be non-NULL when M*N*K > 0, D when M*N > 0
 *     (GEMM_ERR_NULL_POINTER); each must be aligned to its element size
 *     (GEMM_ERR_MISALIGNED).
 *   - Size limits: M, N, K < 2^31 and each operand's rows may span at most
 *     2^31 / 256 bytes of leading dimension (lda*esize, ldb*esize,
 *     ldc*osize, ldd*osize < 8 MiB); larger values give
 *     GEMM_ERR_UNSUPPORTED.
 *   - Aliasing: C == D with ldc == ldd is allowed (in-place D += A.B).  Any
 *     other overlap of C with D is GEMM_ERR_UNSUPPORTED; A or B overlapping
 *     D is undefined behaviour.
 *   - A failed launch returns GEMM_ERR_HIP; gemm_last_hip_error() then gives
 *     the hipError_t of the calling thread's last failure.
 */
#ifndef TILEGEMM_H
#define TILEGEMM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_SIZE = 1,   /* M, N or K negative */
    GEMM_ERR_NULL_POINTER = 2,   /* a required pointer is NULL */
    GEMM_ERR_BAD_LD = 3,         /* a leading dimension is too small */
    GEMM_ERR_MISALIGNED = 4,     /* a pointer is not aligned to its element size */
    GEMM_ERR_UNSUPPORTED = 5,    /* valid but outside this library's limits */
    GEMM_ERR_HIP = 6,            /* the HIP runtime reported an error */
    GEMM_ERR_WORKSPACE = 7,      /* a required workspace is NULL or smaller than needed */
    GEMM_ERR_SCRATCH_LIMIT = 8   /* gemm_bf16_splitk_noalloc: partials larger than its scratch area */
} gemm_status;

typedef enum {
    GEMM_OUT_F32 = 0,            /* D (and C) are fp32 */
    GEMM_OUT_BF16 = 1            /* D (and C) are bf16; fp32 sums rounded to nearest even */
} gemm_out_type;

typedef enum {
    GEMM_K_CONTIGUOUS = 0,       /* A: a(m,k) = A[m*lda + k]   B: b(k,n) = B[n*ldb + k] */
    GEMM_MN_CONTIGUOUS = 1       /* A: a(m,k) = A[k*lda + m]   B: b(k,n) = B[k*ldb + n] */
} gemm_operand_order;

typedef enum {
    GEMM_FP6_E2M3 = 0,           /* OCP FP6 E2M3: 1 sign, 2 exponent (bias 1), 3 mantissa bits; max 7.5 */
    GEMM_FP6_E3M2 = 1            /* OCP FP6 E3M2: 1 sign, 3 exponent (bias 3), 2 mantissa bits; max 28 */
} gemm_fp6_format;

typedef enum {                   /* element formats of gemm_mx_kblock */
    GEMM_MX_E4M3 = 0,            /* as gemm_mxfp8 */
    GEMM_MX_E2M1 = 1,            /* as gemm_mxfp4 */
    GEMM_MX_E2M3 = 2,            /* as gemm_mxfp6 with GEMM_FP6_E2M3 */
    GEMM_MX_E3M2 = 3             /* as gemm_mxfp6 with GEMM_FP6_E3M2 */
} gemm_mx_format;

/*
 * gemm_bf16 -- D = A.B + C with bf16 A and B, fp32 accumulation.
 * Source: "Tensor Core 数据布局的演进", section 一个具体的 fragment 映射
 * (A row-major, B column-major, 16-bit inputs, fp32 accumulator).
 *   A: bf16, M x K row-major, lda     B: bf16, N x K (column-major K x N), ldb
 *   C: out_type, M x N row-major, ldc, or NULL
 *   D: out_type, M x N row-major, ldd
 *   out_type: GEMM_OUT_F32 or GEMM_OUT_BF16 (else GEMM_ERR_UNSUPPORTED)
 */
gemm_status gemm_bf16(int64_t M, int64_t N, int64_t K,
                      const void *A, int64_t lda,
                      const void *B, int64_t ldb,
                      const void *C, int64_t ldc,
                      void *D, int64_t ldd,
                      int out_type, hipStream_t stream);

/*
 * gemm_fp16 -- as gemm_bf16 with IEEE binary16 A and B (same page and
 * section: the fragment mapping is stated for fp16 or bf16 inputs).
 */
gemm_status gemm_fp16(int64_t M, int64_t N, int64_t K,
                      const void *A, int64_t lda,
                      const void *B, int64_t ldb,
                      const void *C, int64_t ldc,
                      void *D, int64_t ldd,
                      int out_type, hipStream_t stream);

/*
 * gemm_bf16_ex, gemm_fp16_ex -- as gemm_bf16 / gemm_fp16 with each operand's
 * storage order chosen (a_order, b_order: gemm_operand_order):
 *   A K-contiguous: M x K row-major, lda >= K (as gemm_bf16)
 *   A MN-contiguous: K x M row-major (M x K column-major), lda >= M
 *   B K-contiguous: stored N x K (K x N column-major), ldb >= K (as gemm_bf16)
 *   B MN-contiguous: K x N row-major, ldb >= N
 * Source: "Tensor Core 数据布局的演进", section ldmatrix：从 shared memory
 * 构造 fragment (the .trans form loads each 8x8 block column-major) and the
 * matrix descriptor's major modes (K-major or MN-major operand tiles); here
 * an MN-contiguous tile is read into K-ordered MFMA fragments with gfx950's
 * LDS transpose read.
 * Both K-contiguous: exactly gemm_bf16 / gemm_fp16.  Otherwise this version
 * needs A and B 16-byte aligned, lda and ldb multiples of 8 and, for a
 * K-contiguous operand, K % 8 == 0 (GEMM_ERR_UNSUPPORTED otherwise); an
 * order other than the two values is GEMM_ERR_UNSUPPORTED.  Everything
 * else as gemm_bf16 (the byte limit applies to lda*2 and ldb*2).
 */
gemm_status gemm_bf16_ex(int64_t M, int64_t N, int64_t K,
                         const void *A, int64_t lda, int a_order,
                         const void *B, int64_t ldb, int b_order,
                         const void *C, int64_t ldc,
                         void *D, int64_t ldd,
                         int out_type, hipStream_t stream);

gemm_status gemm_fp16_ex(int64_t M, int64_t N, int64_t K,
                         const void *A, int64_t lda, int a_order,
                         const void *B, int64_t ldb, int b_order,
                         const void *C, int64_t ldc,
                         void *D, int64_t ldd,
                         int out_type, hipStream_t stream);

/*
 * gemm_mxfp8 -- block-scaled fp8: D = A.B + C with
 *     a(m,k) = e4m3(A[m*lda + k]) * 2^(SFA[m*ldsfa + k/32] - 127)
 *     b(k,n) = e4m3(B[n*ldb + k]) * 2^(SFB[n*ldsfb + k/32] - 127)
 * Source: "Tensor Core 数据布局的演进", section Block-Scaled MMA 的 Scale
 * Factors: SFA(M, SFK) scales K block sfk of row m of A, SFB(N, SFK) scales
 * column n of B, one scale shared by all K elements of its block.  Here a
 * block is 32 contiguous K elements and a scale is an e8m0 code.
 *   A: OCP e4m3 (fn) bytes, M x K row-major       SFA: e8m0 bytes, M x K/32, ldsfa
 *   B: e4m3 bytes, N x K (column-major K x N)     SFB: e8m0 bytes, N x K/32, ldsfb
 *   C, D, out_type: as gemm_bf16
 * ldsfa, ldsfb >= K/32 (else GEMM_ERR_BAD_LD); SFA and SFB non-NULL when
 * M*N*K > 0 (else GEMM_ERR_NULL_POINTER).  K must be a multiple of 32 (else
 * GEMM_ERR_UNSUPPORTED); rows and scale rows may start at any byte.  The
 * tiled kernels take K % 128 == 0 with A, B and lda, ldb 16-byte aligned and
 * SFA, SFB and ldsfa, ldsfb 4-byte aligned (fastest with K % 512 == 0 and
 * 16-byte scale rows); other calls run a slower general kernel.  Scale code
 * 0xFF (NaN) and e4m3 NaN inputs give NaN in the affected outputs.
 */
gemm_status gemm_mxfp8(int64_t M, int64_t N, int64_t K,
                       const void *A, int64_t lda, const void *SFA, int64_t ldsfa,
                       const void *B, int64_t ldb, const void *SFB, int64_t ldsfb,
                       const void *C, int64_t ldc,
                       void *D, int64_t ldd,
                       int out_type, hipStream_t stream);

/*
 * gemm_mxfp4 -- block-scaled fp4: D = A.B + C with
 *     a(m,k) = e2m1(A, m*lda + k) * 2^(SFA[m*ldsfa + k/32] - 127)
 *     b(k,n) = e2m1(B, n*ldb + k) * 2^(SFB[n*ldsfb + k/32] - 127)
 * where e2m1(X, i) is the OCP FP4 E2M1 code in byte i/2 of X, low nibble
 * for even i, high nibble for odd i (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and
 * their negatives; no NaN or infinity).
 * Source: "Tensor Core 数据布局的演进", section Block-Scaled MMA 的 Scale
 * Factors (the same per-block scaling as gemm_mxfp8 with 4-bit elements).
 *   A: M x K elements row-major, lda (elements, even)
 *   B: N x K elements (column-major K x N), ldb (elements, even)
 *   SFA, SFB, C, D, out_type: as gemm_mxfp8
 * Sizes, lda and ldb count ELEMENTS (two per byte).  K must be a multiple
 * of 32 and lda, ldb even (else GEMM_ERR_UNSUPPORTED); rows and scale rows
 * may start at any byte.  The tiled kernel takes K % 512 == 0, A and B
 * 16-byte aligned, lda and ldb multiples of 32, SFA and SFB 16-byte aligned
 * and ldsfa, ldsfb multiples of 16; other calls run a slower general
 * kernel.  Byte limits of the shared convention apply to lda/2, ldb/2.
 * Scale code 0xFF (NaN) gives NaN in the affected outputs.
 */
gemm_status gemm_mxfp4(int64_t M, int64_t N, int64_t K,
                       const void *A, int64_t lda, const void *SFA, int64_t ldsfa,
                       const void *B, int64_t ldb, const void *SFB, int64_t ldsfb,
                       const void *C, int64_t ldc,
                       void *D, int64_t ldd,
                       int out_type, hipStream_t stream);

/*
 * gemm_mxfp6 -- block-scaled fp6: D = A.B + C with
 *     a(m,k) = fp6(A, m*lda + k) * 2^(SFA[m*ldsfa + k/32] - 127)
 *     b(k,n) = fp6(B, n*ldb + k) * 2^(SFB[n*ldsfb + k/32] - 127)
 * where fp6(X, i) is the six-bit code at bits 6i .. 6i+5 of X read as a
 * little-endian bit string (four elements in three bytes, the first in the
 * low six bits of the first byte), in the format given by `format`
 * (GEMM_FP6_E2M3 or GEMM_FP6_E3M2, else GEMM_ERR_UNSUPPORTED; no NaN or
 * infinity in either).  Source: "Tensor Core 数据布局的演进", section
 * Block-Scaled MMA 的 Scale Factors (the same per-block scaling as
 * gemm_mxfp8 with 6-bit elements).
 *   A: M x K elements row-major, lda (elements, a multiple of 4)
 *   B: N x K elements (column-major K x N), ldb (elements, a multiple of 4)
 *   SFA, SFB, C, D, out_type: as gemm_mxfp8
 * Sizes, lda and ldb count ELEMENTS (three bytes per four).  K must be a
 * multiple of 32 and lda, ldb multiples of 4 (else GEMM_ERR_UNSUPPORTED);
 * rows and scale rows may start at any byte.  The tiled kernel takes
 * K % 128 == 0, A and B 16-byte aligned, lda and ldb multiples of 64 (rows of
 * a multiple of 48 bytes), SFA and SFB 16-byte aligned and ldsfa, ldsfb
 * multiples of 16; other calls run a slower general kernel.  Byte limits of
 * the shared convention apply to 3*lda/4 and 3*ldb/4.  Scale code 0xFF
 * (NaN) gives NaN in the affected outputs.
 */
gemm_status gemm_mxfp6(int64_t M, int64_t N, int64_t K,
                       const void *A, int64_t lda, const void *SFA, int64_t ldsfa,
                       const void *B, int64_t ldb, const void *SFB, int64_t ldsfb,
                       const void *C, int64_t ldc,
                       void *D, int64_t ldd,
                       int format, int out_type, hipStream_t stream);

/*
 * gemm_mxfp6_pack, gemm_mxfp6_packed_bytes, gemm_mxfp6_packed -- fp6
 * operands rewritten once as the tile images the fp6 kernel loads, for
 * operands used by many calls (weights).  The tiled kernel stages a
 * 256-row, 128-element K tile of each operand in LDS as 256 rows of 96
 * bytes; from row-major storage each load instruction then fetches 96-byte
 * row pieces, from the images 1 KiB of consecutive bytes.  Source: "Tensor
 * Core 数据布局的演进", section 写回结果与对 shared memory 做 swizzle (the
 * operand staged in a swizzled shared-memory layout; here the global copy
 * is laid out the same way so the copy into it is a straight stream).
 *
 * Image layout of an operand X of `rows` rows and K elements (K % 128 ==
 * 0): ceil(rows / 256) * (K / 128) images of 24576 bytes; image (b, t)
 * (rows 256 b .. 256 b + 255, elements 128 t .. 128 t + 127) starts at byte
 * (b * (K / 128) + t) * 24576, and its 16-byte chunk c (0 .. 1535) holds
 * bytes 96 t + 16 h .. 96 t + 16 h + 15 of row 256 b + c / 6 of X's
 * storage, h = (c % 6) ^ ((c / 6 >> 3) & 1); rows past `rows` are zeros.
 *
 * gemm_mxfp6_packed_bytes(rows, K): the image bytes of such an operand; 0
 *   for rows or K negative, K % 128 != 0, rows >= 2^31 or K >= 2^23.
 * gemm_mxfp6_pack(rows, K, X, ldx, P, p_bytes, stream): enqueue the rewrite
 *   of X (rows x K fp6 elements, row-major, ldx ELEMENTS per row, a
 *   multiple of 4, >= K; any byte alignment) into P (device memory of
 *   p_bytes >= gemm_mxfp6_packed_bytes(rows, K), 16-byte aligned, not
 *   overlapping X; the caller owns both).  The codes are copied as they
 *   are: the format is the GEMM's.  rows or K == 0: nothing is enqueued.
 *   Errors: rows or K negative GEMM_ERR_INVALID_SIZE; K % 128 != 0,
 *   K >= 2^23, rows >= 2^31 or ldx % 4 != 0 GEMM_ERR_UNSUPPORTED; ldx < K
 *   GEMM_ERR_BAD_LD; X or P NULL GEMM_ERR_NULL_POINTER; P not 16-byte
 *   aligned GEMM_ERR_MISALIGNED; p_bytes too small GEMM_ERR_WORKSPACE.
 * gemm_mxfp6_packed(M, N, K, AP, SFA, ldsfa, BP, SFB, ldsfb, C, ldc, D, ldd,
 *   format, out_type, stream): gemm_mxfp6 with A and B given as images --
 *   AP of A (M rows), BP of B (N rows), both with this K, 16-byte aligned
 *   (GEMM_ERR_MISALIGNED) -- and the same result bit for bit (the same
 *   kernel and MFMA order).  Requires K % 128 == 0 and K < 2^23, SFA and
 *   SFB 16-byte aligned with ldsfa and ldsfb multiples of 16
 *   (GEMM_ERR_UNSUPPORTED otherwise; there is no general fallback for
 *   images).  SFA, SFB, C, D, format, out_type and the other checks as
 *   gemm_mxfp6.
 */
size_t gemm_mxfp6_packed_bytes(int64_t rows, int64_t K);

gemm_status gemm_mxfp6_pack(int64_t rows, int64_t K, const void *X, int64_t ldx,
                            void *P, size_t p_bytes, hipStream_t stream);

gemm_status gemm_mxfp6_packed(int64_t M, int64_t N, int64_t K,
                              const void *AP, const void *SFA, int64_t ldsfa,
                              const void *BP, const void *SFB, int64_t ldsfb,
                              const void *C, int64_t ldc,
                              void *D, int64_t ldd,
                              int format, int out_type, hipStream_t stream);

/*
 * gemm_bf16_splitk, gemm_fp16_splitk -- as gemm_bf16 / gemm_fp16, with K cut
 * into `splits` ranges computed by separate workgroups (more workgroups for
 * grids too small to fill the GPU: few output tiles, long K).  Each range's
 * fp32 partial product goes to the caller's workspace; a second kernel on
 * the same stream sums the partials in range order, adds C and writes D, so
 * the result is the same on every call.  Source: "（二）CUTLASS —— 掌握
 * Tensor Memory Accelerator（TMA）", section TMA Store Reduce (several CTAs
 * accumulating tiles into one global tile); here the accumulation is a
 * separate pass over fp32 partials rather than a reducing store.
 *   splits: 0 = the library's choice (split only grids of fewer than 128
 *     tiles of 256 x 256, up to 256 workgroups; under 16 tiles at least
 *     4096 K per range, else at least 1280 K per range and only when that
 *     gives 200 or more workgroups),
 *     1 = no split, up to 64; fewer are used when K has fewer 64-wide tiles,
 *     and none when rows are not 8-byte aligned.  Else GEMM_ERR_UNSUPPORTED.
 *   workspace: device memory, 256-byte aligned (else GEMM_ERR_MISALIGNED), of
 *     at least gemm_splitk_workspace_bytes(M, N, K, splits) bytes (else
 *     GEMM_ERR_WORKSPACE); untouched when no split is used (then it may be
 *     NULL).  Owned by the caller; its contents need no initialisation and
 *     are garbage afterwards.  Calls sharing a workspace must be ordered
 *     (e.g. on one stream); a workspace overlapping A, B, C or D is
 *     undefined behaviour.
 * Everything else (layouts, validation, out_type, C == D) is as gemm_bf16.
 */
gemm_status gemm_bf16_splitk(int64_t M, int64_t N, int64_t K,
                             const void *A, int64_t lda,
                             const void *B, int64_t ldb,
                             const void *C, int64_t ldc,
                             void *D, int64_t ldd,
                             int out_type, int splits,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);

gemm_status gemm_fp16_splitk(int64_t M, int64_t N, int64_t K,
                             const void *A, int64_t lda,
                             const void *B, int64_t ldb,
                             const void *C, int64_t ldc,
                             void *D, int64_t ldd,
                             int out_type, int splits,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * gemm_bf16_splitk_noalloc -- gemm_bf16_splitk for callers that cannot
 * allocate memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same split choice, kernels and
 * result, bit for bit, with the fp32 partials in a scratch area the library
 * holds in static device memory instead of a caller workspace.
 *   - The call allocates nothing (no hipMalloc / hipFree, no allocating
 *     library routine); the caller still passes A, B, C and D.
 *   - The scratch area holds gemm_splitk_scratch_limit() bytes (64 MiB) per
 *     GPU, kept until the process ends; its address is looked up once per
 *     GPU, on the first call there (the GPU of `stream`; NULL: the current
 *     device).  A call whose partials, gemm_splitk_workspace_bytes(M, N, K,
 *     splits), exceed it returns GEMM_ERR_SCRATCH_LIMIT with nothing
 *     enqueued.  Calls that use no split touch no scratch.
 *   - Every call on one GPU shares that GPU's area, which keeps whatever the
 *     last call left there (the partials need no initialisation): calls
 *     that may overlap on one GPU (different streams without ordering, or
 *     several host threads) race and give undefined results.
 * Everything else (splits, layouts, validation, out_type, C == D) is as
 * gemm_bf16_splitk.
 */
gemm_status gemm_bf16_splitk_noalloc(int64_t M, int64_t N, int64_t K,
                                     const void *A, int64_t lda,
                                     const void *B, int64_t ldb,
                                     const void *C, int64_t ldc,
                                     void *D, int64_t ldd,
                                     int out_type, int splits, hipStream_t stream);

/* Bytes of gemm_bf16_splitk_noalloc's scratch area per GPU. */
size_t gemm_splitk_scratch_limit(void);

/*
 * gemm_mxfp8_ex, gemm_mxfp4_ex, gemm_mxfp6_ex -- as gemm_mxfp8 / gemm_mxfp4 /
 * gemm_mxfp6 with each operand's storage order chosen (a_order, b_order:
 * gemm_operand_order):
 *   A K-contiguous: M x K row-major, lda >= K (as the plain call)
 *   A MN-contiguous: K x M row-major, element (m, k) at element k*lda + m,
 *     lda >= M
 *   B K-contiguous: N x K (as the plain call)
 *   B MN-contiguous: K x N row-major, element (k, n) at element k*ldb + n,
 *     ldb >= N
 * Elements are packed along the contiguous dimension as in the plain calls
 * (fp4 two per byte, fp6 four per three bytes; lda, ldb even for fp4 and
 * multiples of 4 for fp6), and the scales keep their layout (SFA M x K/32,
 * SFB N x K/32: one per row or column and 32-element K block).  Source:
 * "Tensor Core 数据布局的演进", the descriptors' K-major and MN-major modes
 * and the transposing fragment load.  Both K-contiguous: exactly the plain
 * call.  Otherwise the call runs the general kernel, each lane gathering its
 * K-ordered elements from the MN-contiguous storage (correct for every
 * shape; far slower than the tiled kernels).  An order other than the two
 * values is GEMM_ERR_UNSUPPORTED; everything else as the plain call.
 */
gemm_status gemm_mxfp8_ex(int64_t M, int64_t N, int64_t K,
                          const void *A, int64_t lda, int a_order, const void *SFA, int64_t ldsfa,
                          const void *B, int64_t ldb, int b_order, const void *SFB, int64_t ldsfb,
                          const void *C, int64_t ldc,
                          void *D, int64_t ldd,
                          int out_type, hipStream_t stream);

gemm_status gemm_mxfp4_ex(int64_t M, int64_t N, int64_t K,
                          const void *A, int64_t lda, int a_order, const void *SFA, int64_t ldsfa,
                          const void *B, int64_t ldb, int b_order, const void *SFB, int64_t ldsfb,
                          const void *C, int64_t ldc,
                          void *D, int64_t ldd,
                          int out_type, hipStream_t stream);

gemm_status gemm_mxfp6_ex(int64_t M, int64_t N, int64_t K,
                          const void *A, int64_t lda, int a_order, const void *SFA, int64_t ldsfa,
                          const void *B, int64_t ldb, int b_order, const void *SFB, int64_t ldsfb,
                          const void *C, int64_t ldc,
                          void *D, int64_t ldd,
                          int format, int out_type, hipStream_t stream);

/*
 * gemm_bf16_ex_ws, gemm_fp16_ex_ws, gemm_mxfp8_ex_ws, gemm_mxfp4_ex_ws,
 * gemm_mxfp6_ex_ws -- the *_ex calls with a workspace: each MN-contiguous
 * operand is first copied, by a kernel on `stream`, into the workspace as
 * its K-contiguous form (rows of K rounded up to T elements, T = 1024 / e,
 * or 192 for fp6, element i at bits e*i .. e*i + e - 1 of a row, e the
 * element's bits), and the plain
 * call then runs on the copies and its tiled kernels -- the same products
 * and sums as the *_ex call.  Source: as the *_ex calls (the descriptors'
 * K-major and MN-major modes: here an MN-major operand becomes K-major once
 * per call instead of per fragment).
 *   workspace: device memory, 256-byte aligned (else GEMM_ERR_MISALIGNED),
 *     at least gemm_ex_workspace_bytes(e, M, N, K, a_order, b_order) bytes
 *     (else GEMM_ERR_WORKSPACE), not overlapping any other argument; its
 *     contents are undefined after the call.  NULL, or both operands
 *     K-contiguous: exactly the *_ex call -- except gemm_mxfp6_ex_ws with
 *     both operands K-contiguous, K % 128 == 0, SFA and SFB 16-byte aligned
 *     with ldsfa, ldsfb multiples of 16 and a workspace of at least
 *     gemm_ex_workspace_bytes(6, M, N, K, GEMM_K_CONTIGUOUS,
 *     GEMM_K_CONTIGUOUS) bytes (the tile images of A then of B, each
 *     rounded up to 256 bytes; 0 when K % 128 != 0), 256-byte aligned: the
 *     operands are rewritten there (gemm_mxfp6_pack) and gemm_mxfp6_packed
 *     runs, the same D bit for bit (a smaller or misaligned workspace then
 *     gives the plain call).
 * Everything else (orders, leading dimensions, scales, validation,
 * out_type, C == D) is as the *_ex call; every check comes before any
 * kernel is enqueued.
 */
gemm_status gemm_bf16_ex_ws(int64_t M, int64_t N, int64_t K,
                            const void *A, int64_t lda, int a_order,
                            const void *B, int64_t ldb, int b_order,
                            const void *C, int64_t ldc,
                            void *D, int64_t ldd,
                            int out_type, void *workspace, size_t workspace_bytes, hipStream_t stream);

gemm_status gemm_fp16_ex_ws(int64_t M, int64_t N, int64_t K,
                            const void *A, int64_t lda, int a_order,
                            const void *B, int64_t ldb, int b_order,
                            const void *C, int64_t ldc,
                            void *D, int64_t ldd,
                            int out_type, void *workspace, size_t workspace_bytes, hipStream_t stream);

gemm_status gemm_mxfp8_ex_ws(int64_t M, int64_t N, int64_t K,
                             const void *A, int64_t lda, int a_order, const void *SFA, int64_t ldsfa,
                             const void *B, int64_t ldb, int b_order, const void *SFB, int64_t ldsfb,
                             const void *C, int64_t ldc,
                             void *D, int64_t ldd,
                             int out_type, void *workspace, size_t workspace_bytes, hipStream_t stream);

gemm_status gemm_mxfp4_ex_ws(int64_t M, int64_t N, int64_t K,
                             const void *A, int64_t lda, int a_order, const void *SFA, int64_t ldsfa,
                             const void *B, int64_t ldb, int b_order, const void *SFB, int64_t ldsfb,
                             const void *C, int64_t ldc,
                             void *D, int64_t ldd,
                             int out_type, void *workspace, size_t workspace_bytes, hipStream_t stream);

gemm_status gemm_mxfp6_ex_ws(int64_t M, int64_t N, int64_t K,
                             const void *A, int64_t lda, int a_order, const void *SFA, int64_t ldsfa,
                             const void *B, int64_t ldb, int b_order, const void *SFB, int64_t ldsfb,
                             const void *C, int64_t ldc,
                             void *D, int64_t ldd,
                             int format, int out_type, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Workspace bytes of the *_ex_ws calls: element_bits 16 (bf16, fp16), 8
 * (fp8), 6 (fp6) or 4 (fp4); for each MN-contiguous operand, its M (N) rows
 * of K rounded up to 1024 / element_bits elements (fp6: 192), rounded up to
 * 256 bytes; 0 for other element sizes or negative sizes. */
size_t gemm_ex_workspace_bytes(int element_bits, int64_t M, int64_t N, int64_t K, int a_order, int b_order);

/*
 * gemm_mx_kblock -- the block-scaled forms (gemm_mxfp8, gemm_mxfp4,
 * gemm_mxfp6, chosen by `format`, a gemm_mx_format) with scale blocks
 * `kblock` K elements wide instead of 32: scale j of row m of A (column n
 * of B) applies to K elements [j kblock, (j + 1) kblock).  Source:
 * "Tensor Core 数据布局的演进", section Block-Scaled MMA 的 Scale Factors
 * (one scale factor per row or column and K block, shared by the block's
 * elements; the page fixes no block width).
 *   kblock: 32, 64, 128, ... (32 times a power of two), or any multiple
 *     of 32 that is at least K: one scale per row of A and column of B;
 *     other values give GEMM_ERR_UNSUPPORTED.
 *   SFA: e8m0 codes, M x ceil(K / kblock), row-major, leading dimension
 *     ldsfa >= ceil(K / kblock) (else GEMM_ERR_BAD_LD); SFB: N x
 *     ceil(K / kblock), ldsfb likewise.
 *   kblock == 32 is the standard call (its tiled kernels); wider blocks run
 *   the general block-scaled kernel (each lane reads the one scale byte its
 *   32-element block shares), K-contiguous operands only.
 * Everything else (element formats and packing, leading dimensions in
 * elements, K % 32 == 0, validation, out_type, C == D) is as the
 * format's standard call.
 */
gemm_status gemm_mx_kblock(int format, int64_t M, int64_t N, int64_t K, int64_t kblock,
                           const void *A, int64_t lda, const void *SFA, int64_t ldsfa,
                           const void *B, int64_t ldb, const void *SFB, int64_t ldsfb,
                           const void *C, int64_t ldc,
                           void *D, int64_t ldd,
                           int out_type, hipStream_t stream);

/*
 * gemm_mx_kblock_ws -- gemm_mx_kblock on the format's tiled kernels, by
 * scale replication: a first kernel on `stream` writes each scale once per
 * 32-element K block it covers (a scale of a kblock-wide block shared by
 * its kblock / 32 blocks of 32) into the caller's workspace, and the
 * standard call (gemm_mxfp8 / gemm_mxfp4 / gemm_mxfp6) then runs on the
 * replicated scales -- the same products and sums, so the same D as
 * gemm_mx_kblock up to summation order.  Source: as gemm_mx_kblock.
 *   workspace: device memory, 256-byte aligned (else GEMM_ERR_MISALIGNED),
 *     at least gemm_mx_kblock_workspace_bytes(M, N, K) bytes (else
 *     GEMM_ERR_WORKSPACE), not overlapping any other argument; its
 *     contents are undefined after the call.  NULL: exactly gemm_mx_kblock.
 *   kblock == 32 needs no workspace (the standard call).
 * Everything else is as gemm_mx_kblock.
 */
gemm_status gemm_mx_kblock_ws(int format, int64_t M, int64_t N, int64_t K, int64_t kblock,
                              const void *A, int64_t lda, const void *SFA, int64_t ldsfa,
                              const void *B, int64_t ldb, const void *SFB, int64_t ldsfb,
                              const void *C, int64_t ldc,
                              void *D, int64_t ldd,
                              int out_type, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of gemm_mx_kblock_ws: (M + N) rows of ceil(K / 32)
 * scale bytes, each row rounded up to 16 bytes; 0 for negative sizes. */
size_t gemm_mx_kblock_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * gemm_mxfp8_splitk, gemm_mxfp4_splitk, gemm_mxfp6_splitk -- as gemm_mxfp8 /
 * gemm_mxfp4 / gemm_mxfp6, with K cut into `splits` ranges of whole groups
 * of 512 K (16 scale blocks) computed by separate workgroups, each range's
 * fp32 partial product going to the caller's workspace, and a second kernel
 * on the same stream summing the partials in range order, adding C and
 * writing D (the same result on every call).  Source: as gemm_bf16_splitk.
 *   splits: as gemm_bf16_splitk, with at most one split per 512 K; calls
 *     the tiled kernels do not take (see gemm_mxfp8 / gemm_mxfp4 /
 *     gemm_mxfp6: K % 512 == 0 -- fp6: K % 128 == 0 --, 16-byte rows and
 *     scale rows) run unsplit.
 *   workspace: as gemm_bf16_splitk; gemm_splitk_workspace_bytes(M, N, K,
 *     splits) bytes always suffice.
 * Everything else (layouts, scales, validation, out_type, C == D) is as the
 * unsplit call.
 */
gemm_status gemm_mxfp8_splitk(int64_t M, int64_t N, int64_t K,
                              const void *A, int64_t lda, const void *SFA, int64_t ldsfa,
                              const void *B, int64_t ldb, const void *SFB, int64_t ldsfb,
                              const void *C, int64_t ldc,
                              void *D, int64_t ldd,
                              int out_type, int splits,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);

gemm_status gemm_mxfp4_splitk(int64_t M, int64_t N, int64_t K,
                              const void *A, int64_t lda, const void *SFA, int64_t ldsfa,
                              const void *B, int64_t ldb, const void *SFB, int64_t ldsfb,
                              const void *C, int64_t ldc,
                              void *D, int64_t ldd,
                              int out_type, int splits,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);

gemm_status gemm_mxfp6_splitk(int64_t M, int64_t N, int64_t K,
                              const void *A, int64_t lda, const void *SFA, int64_t ldsfa,
                              const void *B, int64_t ldb, const void *SFB, int64_t ldsfb,
                              const void *C, int64_t ldc,
                              void *D, int64_t ldd,
                              int format, int out_type, int splits,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Workspace bytes the split-K calls need for these sizes and `splits` (0 =
 * the library's choice): splits_used * M * (N rounded up to a multiple of 4)
 * * 4, with splits_used counted for 64-wide K tiles (the block-scaled calls,
 * cut at multiples of 512 K, never use more); 0 when no split would be used
 * or the arguments are invalid.
 */
size_t gemm_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K, int splits);

/* Human-readable name of a status code (static storage, never NULL). */
const char *gemm_status_string(int status);

/* hipError_t of the calling thread's last GEMM_ERR_HIP (0 if none). */
int gemm_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TILEGEMM_H */
