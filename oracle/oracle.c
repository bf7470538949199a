/*
 * oracle.c -- plain CPU oracle for the tiled matrix multiply-accumulate
 *             D = A.B + C.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * What it computes (all in IEEE binary64, one output element at a time,
 * k ascending, no blocking and no reordering):
 *
 *   a(m,k) = dec_A(A[m*lda + k]) * 2^(SFA[m*ldsfa + k/kb] - 127)
 *   b(k,n) = dec_B(B[n*ldb + k]) * 2^(SFB[n*ldsfb + k/kb] - 127)
 *   D[m,n] = c(m,n) + sum_k a(m,k) * b(k,n)
 *   S[m,n] = sum_k |a(m,k) * b(k,n)|          (feeds the error bound)
 *
 * The scale factors are present only for the block-scaled forms (fp8
 * e4m3, fp4 e2m1 and fp6 e2m3 / e3m2 elements); kb is the scale block's
 * width in K elements (32 in the standard form).
 *
 * Sources on the pages:
 *  - "Tensor Core 数据布局的演进" (Evolution of Tensor Core data layouts),
 *    section 概览 (overview): the operation is the matrix multiply-accumulate
 *    D = AB + C, A and B the multiplied matrices, C the incoming accumulator.
 *  - same page, section 一个具体的 fragment 映射 (a concrete fragment
 *    mapping): A row-major, B column-major, fp16 or bf16 inputs, fp32 C/D.
 *    Here B column-major means b(k,n) lives at B[n*ldb + k].
 *  - same page, section Block-Scaled MMA 的 Scale Factors: SFA[m,sfk]
 *    scales the sfk-th K block of row m of A, SFB[n,sfk] scales column n of
 *    B, and one scale is shared by every K element of its block.  The block
 *    is kb K elements wide, 32 in the standard form, and the scale is an
 *    e8m0 power of two (the reading of the block-scaled workload; the pages
 *    do not print a width).  Coarser blocks -- kb a multiple of 32, up to
 *    one scale per row -- are the same definition with a wider block.
 *
 * Decoders are written from the format definitions (sign, biased exponent,
 * fraction), not from bit casts, so that they are an independent statement
 * of each format:
 *  - bf16: 1-8-7, bias 127 (IEEE-style, with subnormals, inf, NaN)
 *  - fp16: IEEE binary16, 1-5-10, bias 15
 *  - e4m3: OCP FP8 E4M3 ("fn"), 1-4-3, bias 7, no infinities, only
 *          S.1111.111 is NaN, max 448
 *  - e8m0: 8-bit unsigned biased exponent, value 2^(c-127), 0xFF is NaN
 *  - e2m1: OCP MX FP4, 1-2-1, bias 1, no infinities or NaN: values 0, 0.5,
 *          1, 1.5, 2, 3, 4, 6 and their negatives; two per byte, element 2i
 *          in bits 0-3 and element 2i+1 in bits 4-7 of byte i (the block-
 *          scaled fp4 reading: the pages print no element format; this is
 *          the OCP microscaling FP4 type and its packing)
 *  - e2m3: OCP MX FP6 E2M3, 1-2-3, bias 1, no infinities or NaN: max 7.5,
 *          subnormals f/8; e3m2: OCP MX FP6 E3M2, 1-3-2, bias 3, no
 *          infinities or NaN: max 28, subnormals f/16.  Packed six bits per
 *          element: element k of a row occupies bits 6k .. 6k+5 of the row
 *          read as a little-endian bit string (byte j holds bits 8j..8j+7),
 *          four elements per three bytes (the block-scaled fp6 reading, as
 *          for fp4)
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no -ffast-math: the sums must be
 * plain IEEE binary64).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum {
    ORC_BF16 = 0,
    ORC_FP16 = 1,
    ORC_E4M3 = 2,
    ORC_F32 = 3,
    ORC_E2M1 = 4,
    ORC_E2M3 = 5,
    ORC_E3M2 = 6,
};

enum {
    ORC_OK = 0,
    ORC_ERR_ARG = -1,     /* bad size, type or missing pointer */
    ORC_ERR_SCALE = -2,   /* an e8m0 scale code is NaN (0xFF) */
    ORC_ERR_KBLOCK = -3,  /* scaled form with K % 32 != 0 or a block width not a multiple of 32 */
};

/* ---- format decoders ------------------------------------------------- */

double orc_dec_bf16(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 7) & 0xFF;
    int f = h & 0x7F;
    double v;
    if (e == 0xFF)
        v = (f == 0) ? INFINITY : NAN;
    else if (e == 0)
        v = ldexp((double)f, -126 - 7);          /* f/2^7 * 2^-126 */
    else
        v = ldexp(1.0 + (double)f / 128.0, e - 127);
    return s ? -v : v;
}

double orc_dec_fp16(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0x1F)
        v = (f == 0) ? INFINITY : NAN;
    else if (e == 0)
        v = ldexp((double)f, -14 - 10);          /* f/2^10 * 2^-14 */
    else
        v = ldexp(1.0 + (double)f / 1024.0, e - 15);
    return s ? -v : v;
}

double orc_dec_e4m3(uint8_t b)
{
    int s = (b >> 7) & 1;
    int e = (b >> 3) & 0xF;
    int f = b & 0x7;
    double v;
    if (e == 0xF && f == 0x7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)f, -6 - 3);            /* f/8 * 2^-6 */
    else
        v = ldexp(1.0 + (double)f / 8.0, e - 7);
    return s ? -v : v;
}

double orc_dec_e2m1(uint8_t c)
{
    int s = (c >> 3) & 1;
    int e = (c >> 1) & 0x3;
    int f = c & 0x1;
    double v;
    if (e == 0)
        v = 0.5 * (double)f;                      /* f/2 * 2^(1-1) */
    else
        v = ldexp(1.0 + (double)f / 2.0, e - 1);
    return s ? -v : v;
}

double orc_dec_e2m3(uint8_t c)
{
    int s = (c >> 5) & 1;
    int e = (c >> 3) & 0x3;
    int f = c & 0x7;
    double v;
    if (e == 0)
        v = (double)f / 8.0;                      /* f/8 * 2^(1-1) */
    else
        v = ldexp(1.0 + (double)f / 8.0, e - 1);
    return s ? -v : v;
}

double orc_dec_e3m2(uint8_t c)
{
    int s = (c >> 5) & 1;
    int e = (c >> 2) & 0x7;
    int f = c & 0x3;
    double v;
    if (e == 0)
        v = ldexp((double)f / 4.0, 1 - 3);        /* f/4 * 2^(1-3) */
    else
        v = ldexp(1.0 + (double)f / 4.0, e - 3);
    return s ? -v : v;
}

/* Six-bit code k of a packed row: bits 6k .. 6k+5, little-endian. */
static uint8_t fp6_code(const uint8_t *base, int64_t k)
{
    const int64_t bit = 6 * k;
    const int64_t byte = bit >> 3;
    const int sh = (int)(bit & 7);
    unsigned v = base[byte];
    if (sh > 2)                                   /* the field reaches into the next byte */
        v |= (unsigned)base[byte + 1] << 8;
    return (uint8_t)((v >> sh) & 0x3F);
}

double orc_dec_e8m0(uint8_t c)
{
    if (c == 0xFF)
        return NAN;
    return ldexp(1.0, (int)c - 127);
}

double orc_dec_f32(uint32_t u)
{
    int s = (u >> 31) & 1;
    int e = (u >> 23) & 0xFF;
    uint32_t f = u & 0x7FFFFFu;
    double v;
    if (e == 0xFF)
        v = (f == 0) ? INFINITY : NAN;
    else if (e == 0)
        v = ldexp((double)f, -126 - 23);
    else
        v = ldexp(1.0 + (double)f / 8388608.0, e - 127);
    return s ? -v : v;
}

/* Round a binary64 value to the nearest bf16, ties to even (the rounding
 * the bf16 output form is defined with).  Written from the definition:
 * the representable neighbours are spaced one unit in the last place
 * (2^(e-7) in binade e, 2^-133 below 2^-126), and the value is rounded to
 * an integer multiple of that spacing with rint() in the default
 * round-to-nearest-even mode.  Overflow goes to infinity. */
uint16_t orc_rne_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0);
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80);
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);            /* a = f * 2^e2 with f in [0.5, 1) */
    int e = e2 - 1;           /* a in [2^e, 2^(e+1)) */
    if (e < -126)
        e = -126;             /* subnormal spacing is fixed at 2^-133 */
    double ulp = ldexp(1.0, e - 7);
    double q = rint(a / ulp); /* exact division: ulp is a power of two */
    double r = q * ulp;
    if (r >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80);
    /* encode r */
    if (r < ldexp(1.0, -126)) {
        int f = (int)(r / ldexp(1.0, -133));
        return (uint16_t)(sign | f);
    }
    int er2;
    double fr = frexp(r, &er2);
    int eb = er2 - 1 + 127;
    int f = (int)((fr * 2.0 - 1.0) * 128.0);
    return (uint16_t)(sign | (eb << 7) | f);
}

/* Element-wise orc_rne_bf16 over an fp32 array (each value widened exactly). */
void orc_rne_bf16_f32_array(const float *x, uint16_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_rne_bf16((double)x[i]);
}

/* ---- the operation ---------------------------------------------------- */

static double dec_elem(int type, const void *base, int64_t i)
{
    switch (type) {
    case ORC_BF16: return orc_dec_bf16(((const uint16_t *)base)[i]);
    case ORC_FP16: return orc_dec_fp16(((const uint16_t *)base)[i]);
    case ORC_E4M3: return orc_dec_e4m3(((const uint8_t *)base)[i]);
    case ORC_E2M1: {
        uint8_t byte = ((const uint8_t *)base)[i / 2];
        return orc_dec_e2m1((uint8_t)((i & 1) ? byte >> 4 : byte & 0xF));
    }
    case ORC_E2M3: return orc_dec_e2m3(fp6_code((const uint8_t *)base, i));
    case ORC_E3M2: return orc_dec_e3m2(fp6_code((const uint8_t *)base, i));
    case ORC_F32: {
        return orc_dec_f32(((const uint32_t *)base)[i]);
    }
    default: return NAN;
    }
}

/* One output element of D = A.B + C, per the definition in the header. */
static void one_element(int in_type, int64_t m, int64_t n, int64_t K,
                        const void *A, int64_t lda, const uint8_t *SFA, int64_t ldsfa,
                        const void *B, int64_t ldb, const uint8_t *SFB, int64_t ldsfb, int64_t kb,
                        int c_type, const void *C, int64_t ldc,
                        double *d_out, double *s_out)
{
    double acc = 0.0, sabs = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double a = dec_elem(in_type, A, m * lda + k);
        double b = dec_elem(in_type, B, n * ldb + k);
        if (SFA)
            a *= orc_dec_e8m0(SFA[m * ldsfa + k / kb]);
        if (SFB)
            b *= orc_dec_e8m0(SFB[n * ldsfb + k / kb]);
        double p = a * b;
        acc += p;
        sabs += fabs(p);
    }
    double c = C ? dec_elem(c_type, C, m * ldc + n) : 0.0;
    *d_out = c + acc;
    *s_out = sabs;
}

/*
 * oracle_gemm -- evaluate D_ref and S at chosen output elements.
 *
 *   in_type : ORC_BF16, ORC_FP16, ORC_E4M3, ORC_E2M1, ORC_E2M3 or ORC_E3M2
 *             (A and B share it; the fp4 and fp6 types only in the
 *             block-scaled form)
 *   A       : M x K, row-major, leading dimension lda (elements; for
 *             ORC_E2M1 even, two elements per byte; for the fp6 types a
 *             multiple of 4, four elements per three bytes)
 *   B       : column-major K x N stored as N rows of K, leading dim ldb
 *   SFA/SFB : e8m0 codes, M x ceil(K/kb) and N x ceil(K/kb), row-major
 *             with leading dims ldsfa/ldsfb; both NULL for the unscaled
 *             forms, both non-NULL for the block-scaled form
 *   kb      : scale block width in K elements, a positive multiple of 32
 *             (ignored for the unscaled forms)
 *   C       : M x N row-major of c_type (ORC_F32 or ORC_BF16), or NULL
 *   idx     : n_out flat indices m*N + n; NULL means every element in
 *             row-major order (then n_out must equal M*N)
 *   D_out, S_out : n_out binary64 results each
 *   nthreads: OpenMP threads (<= 0: the runtime default)
 *
 * Returns ORC_OK or a negative ORC_ERR_* code; on error nothing is written.
 */
int oracle_gemm(int in_type, int64_t M, int64_t N, int64_t K,
                const void *A, int64_t lda, const uint8_t *SFA, int64_t ldsfa,
                const void *B, int64_t ldb, const uint8_t *SFB, int64_t ldsfb,
                int c_type, const void *C, int64_t ldc,
                int64_t n_out, const int64_t *idx,
                double *D_out, double *S_out, int nthreads, int64_t kb)
{
    if (M < 0 || N < 0 || K < 0 || n_out < 0)
        return ORC_ERR_ARG;
    if (in_type != ORC_BF16 && in_type != ORC_FP16 && in_type != ORC_E4M3 && in_type != ORC_E2M1 &&
        in_type != ORC_E2M3 && in_type != ORC_E3M2)
        return ORC_ERR_ARG;
    if (in_type == ORC_E2M1 && (!SFA || lda % 2 != 0 || ldb % 2 != 0))
        return ORC_ERR_ARG;
    if ((in_type == ORC_E2M3 || in_type == ORC_E3M2) && (!SFA || lda % 4 != 0 || ldb % 4 != 0))
        return ORC_ERR_ARG;
    if (C && c_type != ORC_F32 && c_type != ORC_BF16)
        return ORC_ERR_ARG;
    if (!idx && n_out != M * N)
        return ORC_ERR_ARG;
    if (n_out > 0 && (!D_out || !S_out))
        return ORC_ERR_ARG;
    if (K > 0 && M > 0 && N > 0 && (!A || !B))
        return ORC_ERR_ARG;
    if ((SFA == NULL) != (SFB == NULL))
        return ORC_ERR_ARG;
    if (SFA) {
        if (K % 32 != 0 || kb <= 0 || kb % 32 != 0)
            return ORC_ERR_KBLOCK;
        const int64_t nsc = (K + kb - 1) / kb;         /* scales per row */
        for (int64_t m = 0; m < M; ++m)
            for (int64_t j = 0; j < nsc; ++j)
                if (SFA[m * ldsfa + j] == 0xFF)
                    return ORC_ERR_SCALE;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t j = 0; j < nsc; ++j)
                if (SFB[n * ldsfb + j] == 0xFF)
                    return ORC_ERR_SCALE;
    }
    if (idx) {
        for (int64_t t = 0; t < n_out; ++t)
            if (idx[t] < 0 || idx[t] >= M * N)
                return ORC_ERR_ARG;
    }
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t t = 0; t < n_out; ++t) {
        int64_t flat = idx ? idx[t] : t;
        int64_t m = flat / N, n = flat % N;
        one_element(in_type, m, n, K, A, lda, SFA, ldsfa, B, ldb, SFB, ldsfb, kb,
                    c_type, C, ldc, &D_out[t], &S_out[t]);
    }
    return ORC_OK;
}

/* Number of threads an OpenMP parallel region of this library uses. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
#else
    return 1;
#endif
}
