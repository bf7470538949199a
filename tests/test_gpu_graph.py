"""The C-ABI calls under HIP graph capture, on an MI355X.

Every entry point only enqueues kernels on the caller's stream (no
allocation, no synchronisation, no memset), so a call captured into a HIP
graph must give, on every replay, the bits the same call gives eagerly.
Each case is first checked eagerly against the oracle (integer-valued
inputs, so exactly); the graph is then captured once and replayed several
times, with D overwritten by NaN and other eager GEMMs run between the
replays, and every replay must equal the eager result bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_dense_gemm_tile_amd as tg
from tiled_dense_gemm_tile_amd import inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpuutil import DEV, dev8, dev16, say, to_f64


def _c(rng, M, N):
    return rng.integers(-4, 5, size=(M, N)).astype(np.float32)


def _f16_case(t, M, N, K, seed, with_c, out, splits=None):
    rng = np.random.default_rng(seed)
    A = inputs.random_codes(rng, t, (M, K), integer=True)
    B = inputs.random_codes(rng, t, (N, K), integer=True)
    C = _c(rng, M, N) if with_c else None
    Ad, Bd = dev16(A, t), dev16(B, t)
    Cd = None if C is None else torch.from_numpy(C).to(DEV).to(out)
    ws = None
    if splits is not None:
        ws = torch.empty(tg.splitk_workspace_bytes(M, N, K, splits), dtype=torch.uint8, device=DEV)

    def call(D):
        if splits is None:
            fn = tg.gemm_bf16 if t == "bf16" else tg.gemm_fp16
            return fn(Ad, Bd, Cd, out_dtype=out, D=D)
        fn = tg.gemm_bf16_splitk if t == "bf16" else tg.gemm_fp16_splitk
        return fn(Ad, Bd, Cd, out_dtype=out, D=D, splits=splits, workspace=ws)

    Dr, _ = oracle.gemm_ref_full(t, A, B, C=C)
    return call, Dr


def _mx_case(t, M, N, K, seed, with_c, out, splits=None, b_order="k"):
    rng = np.random.default_rng(seed)
    A = inputs.random_codes(rng, t, (M, K), integer=True)
    B = inputs.random_codes(rng, t, (N, K), integer=True)
    if t == "e4m3":
        e = 0
    elif t == "e2m1":
        e = 1
    else:
        e = inputs.fp6_integer_scale(t)
    SFA = (127 + rng.integers(e, e + 2 if t in ("e4m3", "e2m1") else e + 1, size=(M, K // 32))).astype(np.uint8)
    SFB = (127 + rng.integers(e, e + 2 if t in ("e4m3", "e2m1") else e + 1, size=(N, K // 32))).astype(np.uint8)
    C = _c(rng, M, N) if with_c else None
    Ad, Bd, SFAd, SFBd = dev8(A), dev8(B), dev8(SFA), dev8(SFB)
    if b_order == "mn":
        # the same values stored K-major (N contiguous), passed as a K x N view's storage
        Bd = torch.from_numpy(np.ascontiguousarray(B.T)).to(DEV)
    Cd = None if C is None else torch.from_numpy(C).to(DEV).to(out)
    ws = None
    if splits is not None:
        ws = torch.empty(tg.splitk_workspace_bytes(M, N, K, splits), dtype=torch.uint8, device=DEV)

    def call(D):
        kw = {"out_dtype": out, "D": D}
        if t == "e4m3":
            if splits is not None:
                return tg.gemm_mxfp8_splitk(Ad, SFAd, Bd, SFBd, Cd, splits=splits, workspace=ws, **kw)
            return tg.gemm_mxfp8(Ad, SFAd, Bd, SFBd, Cd, b_order=b_order, **kw)
        if t == "e2m1":
            if splits is not None:
                return tg.gemm_mxfp4_splitk(Ad, SFAd, Bd, SFBd, Cd, splits=splits, workspace=ws, **kw)
            return tg.gemm_mxfp4(Ad, SFAd, Bd, SFBd, Cd, **kw)
        if splits is not None:
            return tg.gemm_mxfp6_splitk(Ad, SFAd, Bd, SFBd, Cd, fmt=t, splits=splits, workspace=ws, **kw)
        return tg.gemm_mxfp6(Ad, SFAd, Bd, SFBd, Cd, fmt=t, **kw)

    Dr, _ = oracle.gemm_ref_full(t, A, B, C=C, SFA=SFA, SFB=SFB)
    return call, Dr


def _ws(n):
    w = torch.empty(n + 256, dtype=torch.uint8, device=DEV)
    return w[(-w.data_ptr()) % 256:]


def _bf16_ex_ws_case():
    """A stored K x M with rows of M + 1 elements: its copy kernel, then the
    plain call, both captured."""
    M, N, K = 300, 260, 200
    rng = np.random.default_rng(8)
    A = inputs.random_codes(rng, "bf16", (M, K), integer=True)
    B = inputs.random_codes(rng, "bf16", (N, K), integer=True)
    st = np.zeros((K, M + 1), np.uint16)
    st[:, :M] = A.T
    Ad = dev16(st, "bf16")[:, :M].t()
    Bd = dev16(B, "bf16")
    ws = _ws(tg.ex_workspace_bytes(16, M, N, K, "mn", "k"))

    def call(D):
        return tg.gemm_bf16(Ad, Bd, D=D, workspace=ws)
    return call, oracle.gemm_ref_full("bf16", A, B)[0]


def _kblock_ws_case():
    """fp8 with 128-wide scale blocks: the scale replication kernel, then the
    tiled call, both captured."""
    M, N, K, kb = 520, 300, 1024, 128
    rng = np.random.default_rng(9)
    A = inputs.random_codes(rng, "e4m3", (M, K), integer=True)
    B = inputs.random_codes(rng, "e4m3", (N, K), integer=True)
    SFA = (127 + rng.integers(0, 2, size=(M, K // kb))).astype(np.uint8)
    SFB = (127 + rng.integers(0, 2, size=(N, K // kb))).astype(np.uint8)
    Ad, Bd, Sa, Sb = dev8(A), dev8(B), dev8(SFA), dev8(SFB)
    ws = _ws(tg.mx_kblock_workspace_bytes(M, N, K))

    def call(D):
        return tg.gemm_mx_kblock("e4m3", Ad, Sa, Bd, Sb, kb, D=D, workspace=ws)
    return call, oracle.gemm_ref_full("e4m3", A, B, SFA=SFA, SFB=SFB, kblock=kb)[0]


def _mxfp6_packed_case():
    """fp6 operands packed into tile images, then the packed GEMM, both
    captured (the images are rewritten on every replay)."""
    M, N, K = 300, 520, 640
    rng = np.random.default_rng(12)
    A = inputs.random_codes(rng, "e2m3", (M, K), integer=True)
    B = inputs.random_codes(rng, "e2m3", (N, K), integer=True)
    e = inputs.fp6_integer_scale("e2m3")
    SFA = np.full((M, K // 32), 127 + e, np.uint8)
    SFB = np.full((N, K // 32), 127 + e, np.uint8)
    sa = np.zeros((M, 32), np.uint8)
    sa[:, :K // 32] = SFA
    sb = np.zeros((N, 32), np.uint8)
    sb[:, :K // 32] = SFB
    Ad, Bd = dev8(A), dev8(B)
    Sa, Sb = dev8(sa)[:, :K // 32], dev8(sb)[:, :K // 32]
    AP = torch.empty(tg.mxfp6_packed_bytes(M, K), dtype=torch.uint8, device=DEV)
    BP = torch.empty(tg.mxfp6_packed_bytes(N, K), dtype=torch.uint8, device=DEV)

    def call(D):
        tg.mxfp6_pack(Ad, out=AP)
        tg.mxfp6_pack(Bd, out=BP)
        return tg.gemm_mxfp6_packed(AP, Sa, BP, Sb, M, N, K, D=D)
    return call, oracle.gemm_ref_full("e2m3", A, B, SFA=SFA, SFB=SFB)[0]


# (label, builder): whole and ragged tiles, both output types, C present and
# absent, split-K with its reduction kernel, the general scaled kernel, the
# persistent kernels, the workspace paths (a copy or replication kernel
# before the GEMM), fp6 tile images (two packing kernels before the GEMM)
CASES = {
    "bf16_c_ragged": lambda: _f16_case("bf16", 1000, 700, 1100, 1, True, torch.float32),
    "fp16_bf16out_oddk": lambda: _f16_case("fp16", 384, 520, 4100, 2, False, torch.bfloat16),
    "bf16_splitk4": lambda: _f16_case("bf16", 256, 320, 8192, 3, True, torch.float32, splits=4),
    "mxfp8_tiled": lambda: _mx_case("e4m3", 512, 512, 1024, 4, True, torch.float32),
    "mxfp8_general_mn": lambda: _mx_case("e4m3", 200, 136, 1056, 5, True, torch.bfloat16, b_order="mn"),
    "mxfp4_splitk4": lambda: _mx_case("e2m1", 256, 256, 4096, 6, False, torch.float32, splits=4),
    "mxfp6_e3m2": lambda: _mx_case("e3m2", 300, 200, 640, 7, True, torch.float32),
    "bf16_persistent": lambda: _f16_case("bf16", 4200, 4300, 256, 10, False, torch.bfloat16),
    "mxfp8_persistent": lambda: _mx_case("e4m3", 4200, 4300, 512, 11, False, torch.float32),
    "bf16_ex_ws": _bf16_ex_ws_case,
    "mxfp8_kblock_ws": _kblock_ws_case,
    "mxfp6_packed": _mxfp6_packed_case,
}


@pytest.mark.parametrize("label", list(CASES))
def test_graph_replays_equal_eager(label):
    say("graph %s" % label)
    call, Dr = CASES[label]()
    M, N = Dr.shape
    D_eager = call(None)
    torch.cuda.synchronize()
    out = D_eager.dtype
    if out == torch.float32:
        assert np.array_equal(to_f64(D_eager), Dr)
    else:
        assert np.array_equal(D_eager.cpu().view(torch.int16).numpy().view(np.uint16),
                              oracle.rne_bf16_f32(Dr.astype(np.float32)))

    D = torch.empty((M, N), dtype=out, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(D)
    torch.cuda.synchronize()

    other = torch.empty_like(D_eager)
    for r in range(4):
        D.fill_(float("nan"))
        call(other)                                   # eager work between the replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(D, D_eager), "replay %d differs" % r
        assert torch.equal(other, D_eager)
