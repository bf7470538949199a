// C ABI of the tiled GEMM library, 16-bit inputs: argument validation,
// kernel selection and launch on the caller's stream, plus the status
// helpers.  The declarations and their contract are in include/tilegemm.h.
#include <stdlib.h>

#include <mutex>

#include "api.hpp"
#include "transpose.hpp"
#include "f16_launch.hpp"

using namespace tg_api;

namespace {

// Widest vector (in elements) that every row start and K boundary allows.
int pick_vec(const Common &a) {
    for (int v = 8; v > 1; v >>= 1) {
        const uintptr_t bytes = (uintptr_t)v * 2;
        if (((uintptr_t)a.A % bytes) == 0 && ((uintptr_t)a.B % bytes) == 0 && a.lda % v == 0 &&
            a.ldb % v == 0 && a.K % v == 0)
            return v;
    }
    return 1;
}

// Test override: TILEGEMM_F16_CONFIG=<id> forces one of the configurations
// below where its load width allows the call (read at every call; ignored
// when out of range), so the tests can reach each one on small shapes.
int forced_f16_cfg() {
    const char *e = getenv("TILEGEMM_F16_CONFIG");
    if (!e || !*e) return -1;
    const int id = atoi(e);
    return (id >= 0 && id < tg::kNumF16DmaCfgs) ? id : -1;
}

// lane_bytes 16: rows 16-byte aligned; 4: rows only 8- or 4-byte aligned.
// vec: the widest vector in elements that every row allows (8, 4 or 2 here).
int pick_f16_cfg(const Common &a, int lane_bytes, int vec) {
    const int forced = forced_f16_cfg();
    if (forced >= 0) {
        const bool ok = (forced == tg::kF16FourWaveS || forced == tg::kF16FourWaveS192) ? vec >= 4
                        : (forced == tg::kF16FourWave || forced == tg::kF16FourWave192 ||
                           forced == tg::kF16FourWavePersist)
                            ? lane_bytes == 16
                        : lane_bytes == 16 ? tg::f16_has_lane16(forced) : tg::f16_has_lane4(forced);
        if (ok) return forced;
    }
    // Four-wave 256 x 256 kernels once that grid covers half the chip: a
    // grid of 128 to 255 such tiles (part of one wave) finishes in the time
    // of a full wave, which beats the 2 to 4 waves of 128 x 128 tiles the
    // same output takes (measured at K = 4096: 144 tiles 74.9 against
    // 102.7 us, 224 tiles 92.3 against 139.5 us; equal at 128 tiles and
    // slower below).
    // Of the two four-wave tile heights, 192 x 256 tiles (0.75 of the work
    // each) when their waves of 256 workgroups cost less than those of
    // 256 x 256 tiles: 4000 x 3000 is 192 tiles of 256^2 (one wave, 3/4 of
    // the CUs busy) but 252 of 192 x 256 (one wave at 3/4 of the time).
    const int64_t t256 = tiles_of(a, 256, 256);
    const bool h192 = 3 * ((tiles_of(a, 192, 256) + 255) / 256) < 4 * ((t256 + 255) / 256);
    if (vec == 4 && t256 >= 128) return h192 ? tg::kF16FourWaveS192 : tg::kF16FourWaveS;   // 8-byte rows
    // (persistent where the grid is over one wave and the call allows it:
    // dispatch_f16)
    if (lane_bytes == 16 && t256 >= 128) return h192 ? tg::kF16FourWave192 : tg::kF16FourWavePersist;
    if (t256 >= 240) return tg::kF16Wide4Lane;                     // (rows 4-byte aligned here)
    // 128 x 128 tiles: about one wave of them (one workgroup per CU) runs
    // best with both rings two tiles ahead (2048 x 2048 x 4096: 40.0 against
    // 45.1 us); more, with two workgroups per CU sharing it, on the smaller
    // three-slot A ring (2304 x 2304 x 4096: 62.1 against 71.7 us).
    const int64_t t128 = tiles_of(a, 128, 128);
    if (lane_bytes == 16 && t128 >= 240 && t128 <= 256) return tg::kF16Deep128;
    if (t128 >= 240) return tg::kF16Wide128;
    // smaller grids: 64 x 64 tiles, both rings two tiles ahead, up to two
    // workgroups per CU (1024 x 1024 x 4096: 18.9 against 30.0 us with the
    // two-slot rings; past 512 tiles the two-slot rings are ahead again)
    if (lane_bytes == 16 && tiles_of(a, 64, 64) <= 512) return tg::kF16Deep64;
    return tg::kF16Small64;
}

template <bool FP16, bool OUT_BF16>
gemm_status dispatch_f16(const Common &a, hipStream_t s) {
    tg::F16Args p;
    p.A = a.A;
    p.B = a.B;
    p.C = a.C;
    p.D = a.D;
    p.lda = a.lda;
    p.ldb = a.ldb;
    p.ldc = a.ldc;
    p.ldd = a.ldd;
    p.M = (int)a.M;
    p.N = (int)a.N;
    p.K = (int)a.K;
    p.group_m = 4;
    // 16-byte rows: 16-byte direct-to-LDS lanes; 4- or 8-byte rows: 4-byte
    // lanes; 2-byte rows (odd K or leading dimension): register staging,
    // element by element.
    const int vec = pick_vec(a);
    const int lane_bytes = vec == 8 ? 16 : 4;
    int bm = tg::StagedCfg::BM, bn = tg::StagedCfg::BN, cfg = -1;
    if (vec >= 2) {
        cfg = pick_f16_cfg(a, lane_bytes, vec);
        bm = tg::kF16DmaCfgs[cfg].bm;
        bn = tg::kF16DmaCfgs[cfg].bn;
    }
    p.tiles_m = (int)((a.M + bm - 1) / bm);
    p.tiles_n = (int)((a.N + bn - 1) / bn);
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    if (tiles >= kMaxDim) return GEMM_ERR_UNSUPPORTED;
    if (cfg >= 0) {
        const int os = OUT_BF16 ? 2 : 4;
        const uintptr_t vb = (uintptr_t)os * 4;
        tg::F16Epi e;
        e.vec_d = ((uintptr_t)a.D % vb) == 0 && a.ldd % 4 == 0;
        e.vec_c = a.C && ((uintptr_t)a.C % vb) == 0 && a.ldc % 4 == 0;
        if (cfg == tg::kF16FourWavePersist) {
            // one workgroup per CU over grids of more tiles than CUs, without
            // C and with D rows of whole 16-byte segments (its epilogue's
            // stores); otherwise one workgroup per tile
            const int cus = cu_count(s);
            if (!a.C && e.vec_d && a.N % 4 == 0 && cus > 0 && tiles > cus)
                return launched(tg::launch_f16_dma<FP16, OUT_BF16>(cfg, lane_bytes, (unsigned)cus, s, p, e));
            cfg = tg::kF16FourWave;
        }
        return launched(tg::launch_f16_dma<FP16, OUT_BF16>(cfg, lane_bytes, (unsigned)tiles, s, p, e));
    }
    return launched(tg::launch_f16_staged<FP16, OUT_BF16>((unsigned)tiles, s, p));
}

gemm_status run_f16(bool fp16, const Common &a, hipStream_t s) {
    bool none = false;
    gemm_status st = validate(a, &none);
    if (st != GEMM_OK || none) return st;
    if (fp16)
        return a.out_type == GEMM_OUT_BF16 ? dispatch_f16<true, true>(a, s) : dispatch_f16<true, false>(a, s);
    return a.out_type == GEMM_OUT_BF16 ? dispatch_f16<false, true>(a, s) : dispatch_f16<false, false>(a, s);
}

// ---- operand storage orders (16-bit inputs) ---------------------------------

gemm_status run_f16_ex(bool fp16, const Common &a, int a_order, int b_order, hipStream_t s) {
    if ((a_order != GEMM_K_CONTIGUOUS && a_order != GEMM_MN_CONTIGUOUS) ||
        (b_order != GEMM_K_CONTIGUOUS && b_order != GEMM_MN_CONTIGUOUS))
        return GEMM_ERR_UNSUPPORTED;
    if (a_order == GEMM_K_CONTIGUOUS && b_order == GEMM_K_CONTIGUOUS) return run_f16(fp16, a, s);
    const bool at = a_order == GEMM_MN_CONTIGUOUS, bt = b_order == GEMM_MN_CONTIGUOUS;
    if (a.M < 0 || a.N < 0 || a.K < 0) return GEMM_ERR_INVALID_SIZE;
    // an MN-contiguous operand's leading dimension spans its M (N) elements
    if (a.M > 0 && a.N > 0 && ((at && a.lda < a.M) || (bt && a.ldb < a.N))) return GEMM_ERR_BAD_LD;
    Common v = a;
    if (at) v.lda = a.K;                               // checked above
    if (bt) v.ldb = a.K;
    bool none = false;
    gemm_status st = validate(v, &none);
    if (st != GEMM_OK || none) return st;
    if ((at && a.lda * 2 >= kMaxLdBytes) || (bt && a.ldb * 2 >= kMaxLdBytes)) return GEMM_ERR_UNSUPPORTED;
    // this kernel: 16-byte rows for both operands
    const bool rows16 = (uintptr_t)a.A % 16 == 0 && (uintptr_t)a.B % 16 == 0 && a.lda % 8 == 0 && a.ldb % 8 == 0 &&
                        ((at && bt) || a.K % 8 == 0);
    if (!rows16 && a.K > 0) return GEMM_ERR_UNSUPPORTED;
    tg::F16Args p;
    p.A = a.A ? a.A : a.D;                             // K == 0 reads no operand
    p.B = a.B ? a.B : a.D;
    p.C = a.C;
    p.D = a.D;
    p.lda = a.lda;
    p.ldb = a.ldb;
    p.ldc = a.ldc;
    p.ldd = a.ldd;
    p.M = (int)a.M;
    p.N = (int)a.N;
    p.K = (int)a.K;
    p.group_m = 4;
    p.tiles_m = (int)((a.M + 255) / 256);
    p.tiles_n = (int)((a.N + 255) / 256);
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    if (tiles >= kMaxDim) return GEMM_ERR_UNSUPPORTED;
    const bool bf16 = a.out_type == GEMM_OUT_BF16;
    const uintptr_t vb = (uintptr_t)(bf16 ? 2 : 4) * 4;
    tg::F16Epi e;
    e.vec_d = ((uintptr_t)a.D % vb) == 0 && a.ldd % 4 == 0;
    e.vec_c = a.C && ((uintptr_t)a.C % vb) == 0 && a.ldc % 4 == 0;
    hipError_t err;
    if (fp16)
        err = bf16 ? tg::launch_f16_mn<true, true>(at, bt, (unsigned)tiles, s, p, e)
                   : tg::launch_f16_mn<true, false>(at, bt, (unsigned)tiles, s, p, e);
    else
        err = bf16 ? tg::launch_f16_mn<false, true>(at, bt, (unsigned)tiles, s, p, e)
                   : tg::launch_f16_mn<false, false>(at, bt, (unsigned)tiles, s, p, e);
    return launched(err);
}

// ---- split-K (16-bit inputs) ------------------------------------------------

gemm_status run_f16_splitk(bool fp16, const Common &a, int splits, void *ws, size_t ws_bytes, hipStream_t s) {
    bool none = false;
    gemm_status st = validate(a, &none);
    if (st != GEMM_OK || none) return st;
    if (splits < 0 || splits > kMaxSplits) return GEMM_ERR_UNSUPPORTED;
    const int S = effective_splits(a.K, splits == 0 ? auto_splits(a.M, a.N, a.K) : splits);
    const int vec = pick_vec(a);
    // rows only 4- or 2-byte aligned have no four-wave kernel: unsplit
    if (S == 1 || vec < 4) return run_f16(fp16, a, s);
    st = check_workspace(a, S, ws, ws_bytes);
    if (st != GEMM_OK) return st;
    const int64_t ldw = splitk_ldw(a.N);
    const int64_t kt = (a.K + 63) / 64;
    tg::F16Args p;
    p.A = a.A;
    p.B = a.B;
    p.C = nullptr;
    p.D = nullptr;
    p.lda = a.lda;
    p.ldb = a.ldb;
    p.ldc = 0;
    p.ldd = 0;
    p.M = (int)a.M;
    p.N = (int)a.N;
    p.K = (int)a.K;
    p.group_m = 4;
    p.tiles_m = (int)((a.M + 255) / 256);
    p.tiles_n = (int)((a.N + 255) / 256);
    p.kt_split = (int)((kt + S - 1) / S);
    p.ws = (float *)ws;
    p.ldw = ldw;
    const int64_t grid = (int64_t)p.tiles_m * p.tiles_n * S;
    if (grid >= kMaxDim) return GEMM_ERR_UNSUPPORTED;
    tg::F16Epi e;
    e.vec_c = false;
    e.vec_d = true;                                    // 256-byte aligned base, ldw % 4 == 0
    const bool sh = vec == 4;                          // 8-byte rows: the shifted-row variant
    hipError_t err = fp16 ? tg::launch_f16_split<true, false>(sh, (unsigned)grid, s, p, e)
                          : tg::launch_f16_split<false, false>(sh, (unsigned)grid, s, p, e);
    if (err != hipSuccess) return launched(err);
    return reduce_splits(a, ws, S, s);
}

// ---- split-K with the library's static scratch area --------------------------

// fp32 split partials of gemm_bf16_splitk_noalloc: one copy of this array per
// GPU, created when the library's code is loaded there and held until the
// process ends.  In host code the name is only a host-side stand-in for the
// device symbol; the device address comes from scratch_address().
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kScratchBytes];

// Device address of the stream's GPU's copy of `scratch`, looked up once per
// device (hipGetSymbolAddress with that device current) and kept.
gemm_status scratch_address(hipStream_t s, void **out) {
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return launched(e);
    if (dev < 0 || dev >= kMaxDevices) return GEMM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return launched(e);
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return launched(e);
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return launched(e);
        addr[dev] = p;
    }
    *out = addr[dev];
    return GEMM_OK;
}

gemm_status run_bf16_splitk_noalloc(const Common &a, int splits, hipStream_t s) {
    bool none = false;
    gemm_status st = validate(a, &none);
    if (st != GEMM_OK || none) return st;
    if (splits < 0 || splits > kMaxSplits) return GEMM_ERR_UNSUPPORTED;
    // the split count and kernel choice of run_f16_splitk
    const int S = effective_splits(a.K, splits == 0 ? auto_splits(a.M, a.N, a.K) : splits);
    if (S == 1 || pick_vec(a) < 4) return run_f16(false, a, s);
    const size_t need = splitk_bytes(a.M, a.N, S);
    if (need > kScratchBytes) return GEMM_ERR_SCRATCH_LIMIT;
    void *ws = nullptr;
    st = scratch_address(s, &ws);
    if (st != GEMM_OK) return st;
    return run_f16_splitk(false, a, splits, ws, kScratchBytes, s);
}

}  // namespace

// *_ex_ws, 16-bit inputs: the _ex call's checks, then K-contiguous copies
// of the MN-contiguous operands in the workspace and the plain call.
gemm_status run_f16_ex_ws(bool fp16, const Common &a, int a_order, int b_order, void *ws, size_t ws_bytes,
                          hipStream_t s) {
    if ((a_order != GEMM_K_CONTIGUOUS && a_order != GEMM_MN_CONTIGUOUS) ||
        (b_order != GEMM_K_CONTIGUOUS && b_order != GEMM_MN_CONTIGUOUS))
        return GEMM_ERR_UNSUPPORTED;
    const bool at = a_order == GEMM_MN_CONTIGUOUS, bt = b_order == GEMM_MN_CONTIGUOUS;
    if (!ws || (!at && !bt)) return run_f16_ex(fp16, a, a_order, b_order, s);
    if (a.M < 0 || a.N < 0 || a.K < 0) return GEMM_ERR_INVALID_SIZE;
    if (a.M > 0 && a.N > 0 && ((at && a.lda < a.M) || (bt && a.ldb < a.N))) return GEMM_ERR_BAD_LD;
    Common v = a;
    if (at) v.lda = a.K;
    if (bt) v.ldb = a.K;
    bool none = false;
    gemm_status st = validate(v, &none);
    if (st != GEMM_OK || none) return st;
    if ((at && a.lda * 2 >= kMaxLdBytes) || (bt && a.ldb * 2 >= kMaxLdBytes)) return GEMM_ERR_UNSUPPORTED;
    if (a.K == 0) return run_f16_ex(fp16, a, a_order, b_order, s);
    Common k = a;
    st = k_contiguous_operands(16, a, at, bt, ws, ws_bytes, s, &k.A, &k.lda, &k.B, &k.ldb);
    if (st != GEMM_OK) return st;
    return run_f16(fp16, k, s);
}

extern "C" {

gemm_status gemm_bf16(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                      const void *C, int64_t ldc, void *D, int64_t ldd, int out_type, hipStream_t stream) {
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 2};
    return run_f16(false, a, stream);
}

gemm_status gemm_fp16(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                      const void *C, int64_t ldc, void *D, int64_t ldd, int out_type, hipStream_t stream) {
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 2};
    return run_f16(true, a, stream);
}

gemm_status gemm_bf16_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int a_order, const void *B,
                         int64_t ldb, int b_order, const void *C, int64_t ldc, void *D, int64_t ldd, int out_type,
                         hipStream_t stream) {
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 2};
    return run_f16_ex(false, a, a_order, b_order, stream);
}

gemm_status gemm_fp16_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int a_order, const void *B,
                         int64_t ldb, int b_order, const void *C, int64_t ldc, void *D, int64_t ldd, int out_type,
                         hipStream_t stream) {
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 2};
    return run_f16_ex(true, a, a_order, b_order, stream);
}

gemm_status gemm_bf16_ex_ws(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int a_order,
                            const void *B, int64_t ldb, int b_order, const void *C, int64_t ldc, void *D,
                            int64_t ldd, int out_type, void *workspace, size_t workspace_bytes,
                            hipStream_t stream) {
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 2};
    return run_f16_ex_ws(false, a, a_order, b_order, workspace, workspace_bytes, stream);
}

gemm_status gemm_fp16_ex_ws(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int a_order,
                            const void *B, int64_t ldb, int b_order, const void *C, int64_t ldc, void *D,
                            int64_t ldd, int out_type, void *workspace, size_t workspace_bytes,
                            hipStream_t stream) {
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 2};
    return run_f16_ex_ws(true, a, a_order, b_order, workspace, workspace_bytes, stream);
}

size_t gemm_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K, int splits) {
    if (M <= 0 || N <= 0 || K <= 0 || splits < 0 || splits > kMaxSplits) return 0;
    return splitk_bytes(M, N, effective_splits(K, splits == 0 ? auto_splits(M, N, K) : splits));
}

gemm_status gemm_bf16_splitk(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                             const void *C, int64_t ldc, void *D, int64_t ldd, int out_type, int splits,
                             void *workspace, size_t workspace_bytes, hipStream_t stream) {
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 2};
    return run_f16_splitk(false, a, splits, workspace, workspace_bytes, stream);
}

gemm_status gemm_fp16_splitk(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                             const void *C, int64_t ldc, void *D, int64_t ldd, int out_type, int splits,
                             void *workspace, size_t workspace_bytes, hipStream_t stream) {
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 2};
    return run_f16_splitk(true, a, splits, workspace, workspace_bytes, stream);
}

gemm_status gemm_bf16_splitk_noalloc(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                                     int64_t ldb, const void *C, int64_t ldc, void *D, int64_t ldd, int out_type,
                                     int splits, hipStream_t stream) {
    Common a{M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out_type, 2};
    return run_bf16_splitk_noalloc(a, splits, stream);
}

size_t gemm_splitk_scratch_limit(void) { return kScratchBytes; }

const char *gemm_status_string(int s) {
    switch (s) {
    case GEMM_OK: return "GEMM_OK";
    case GEMM_ERR_INVALID_SIZE: return "GEMM_ERR_INVALID_SIZE: M, N or K is negative";
    case GEMM_ERR_NULL_POINTER: return "GEMM_ERR_NULL_POINTER: a required pointer is NULL";
    case GEMM_ERR_BAD_LD: return "GEMM_ERR_BAD_LD: a leading dimension is smaller than its row";
    case GEMM_ERR_MISALIGNED: return "GEMM_ERR_MISALIGNED: a pointer is not aligned to its element size";
    case GEMM_ERR_UNSUPPORTED: return "GEMM_ERR_UNSUPPORTED: outside the library's limits";
    case GEMM_ERR_HIP: return "GEMM_ERR_HIP: the HIP runtime reported an error";
    case GEMM_ERR_WORKSPACE: return "GEMM_ERR_WORKSPACE: the workspace is missing or too small";
    case GEMM_ERR_SCRATCH_LIMIT:
        return "GEMM_ERR_SCRATCH_LIMIT: the split partials exceed the library's static scratch area";
    default: return "unknown gemm_status";
    }
}

int gemm_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
