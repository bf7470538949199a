"""MN-contiguous operands through a workspace (gemm_*_ex_ws): each
MN-contiguous operand copied K-contiguous by a kernel, then the plain call's
tiled kernels.

The logical operands are drawn as for the K-contiguous calls and only their
storage changes.  Bar: bit-exact against the oracle on integer inputs (and
equal to the K-contiguous call on the same values), otherwise
|D - D_ref| <= 2^-12 * sum|a*b| + 1e-6.  Shapes cover partial 64-element
copy tiles in both directions, storage rows that are not 16-byte multiples
(which the 16-bit _ex call refuses without a workspace), padded storage
rows, and grids large enough for the four-wave and persistent kernels.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import check
import tiled_dense_gemm_tile_amd as tg
from tiled_dense_gemm_tile_amd import inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpuutil import DEV, dev8, dev16, say, to_f64

ORDERS = [(True, False), (False, True), (True, True)]
BITS = {"bf16": 16, "fp16": 16, "e4m3": 8, "e2m3": 6, "e3m2": 6, "e2m1": 4}


def _workspace(t, M, N, K, a_mn, b_mn):
    n = tg.ex_workspace_bytes(BITS[t], M, N, K, "mn" if a_mn else "k", "mn" if b_mn else "k")
    ws = torch.empty(n + 256, dtype=torch.uint8, device=DEV)
    return ws[(-ws.data_ptr()) % 256:]


# ---- 16-bit ---------------------------------------------------------------

def _stored16(codes, t, mn, ld):
    """Device view (rows, K) of the logical codes, K-contiguous or stored as
    a K x ld array (MN-contiguous, ld >= rows)."""
    if not mn:
        return dev16(codes, t)
    rows, K = codes.shape
    st = np.zeros((K, ld), dtype=np.uint16)
    st[:, :rows] = codes.T
    return dev16(st, t)[:, :rows].t()


# (M, N, K, extra elements per MN storage row): rows of M + 3 elements
# (not 16-byte multiples), odd K, one element, grids of several waves
SHAPES16 = [(300, 200, 520, 3), (257, 129, 136, 1), (64, 40, 8, 0), (1, 1, 65, 5), (1000, 513, 100, 0),
            (4200, 4300, 1024, 0), (2048, 2304, 777, 2)]


@pytest.mark.parametrize("t", ["bf16", "fp16"])
@pytest.mark.parametrize("orders", ORDERS, ids=["a_mn", "b_mn", "both"])
@pytest.mark.parametrize("shape", SHAPES16, ids=["%dx%dx%d+%d" % s for s in SHAPES16])
def test_16bit(t, orders, shape):
    M, N, K, pad = shape
    a_mn, b_mn = orders
    big = M * N > 4 * 10 ** 6
    for integer in ((True,) if big else (True, False)):
        rng = np.random.default_rng(M + N + K + pad + 3 * a_mn + b_mn)
        A = inputs.random_codes(rng, t, (M, K), integer=integer)
        B = inputs.random_codes(rng, t, (N, K), integer=integer)
        C = None if big else (rng.integers(-4, 5, size=(M, N)) if integer
                              else rng.uniform(-1, 1, size=(M, N))).astype(np.float32)
        Cd = torch.from_numpy(C).to(DEV) if C is not None else None
        Ad, Bd = _stored16(A, t, a_mn, M + pad), _stored16(B, t, b_mn, N + pad)
        fn = tg.gemm_bf16 if t == "bf16" else tg.gemm_fp16
        say("ex_ws %s a_mn=%s b_mn=%s %dx%dx%d+%d integer=%s" % (t, a_mn, b_mn, M, N, K, pad, integer))
        D = fn(Ad, Bd, Cd, workspace=_workspace(t, M, N, K, a_mn, b_mn))
        torch.cuda.synchronize()
        if big:
            rand, forced = inputs.sample_indices(M, N, K)
            idx = np.concatenate([rand, forced])
            Dr, _ = oracle.gemm_ref(t, A, B, idx=idx)
            assert np.array_equal(to_f64(D).ravel()[idx], Dr)
            Dk = fn(dev16(A, t), dev16(B, t))
            torch.cuda.synchronize()
            assert torch.equal(D, Dk)
            continue
        Dr, S = oracle.gemm_ref_full(t, A, B, C=C)
        Dg = to_f64(D)
        if integer:
            bad = np.argwhere(Dg != Dr)
            assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()
        else:
            rep = check.report(Dg, Dr, S)
            assert rep["fail"] == 0, rep


def test_16bit_unaligned_rows_need_the_workspace():
    """MN-contiguous rows that are not 16-byte multiples: refused by the _ex
    call, computed through the workspace."""
    M, N, K = 100, 64, 96
    rng = np.random.default_rng(1)
    A = inputs.random_codes(rng, "bf16", (M, K), integer=True)
    B = inputs.random_codes(rng, "bf16", (N, K), integer=True)
    Ad = _stored16(A, "bf16", True, M + 1)
    with pytest.raises(tg.GemmError):
        tg.gemm_bf16(Ad, dev16(B, "bf16"))
    D = tg.gemm_bf16(Ad, dev16(B, "bf16"), workspace=_workspace("bf16", M, N, K, True, False))
    torch.cuda.synchronize()
    Dr, _ = oracle.gemm_ref_full("bf16", A, B)
    assert np.array_equal(to_f64(D), Dr)


# ---- block-scaled ---------------------------------------------------------

UNIT = {"e2m3": 9, "e3m2": 13}                      # fp6 codes of magnitude <= 1


def _codes(t, rng, shape, integer):
    if t == "e4m3":
        return inputs.random_codes(rng, t, shape, integer=integer)
    if t == "e2m1":
        return rng.integers(0, 16, size=shape).astype(np.uint8)
    if integer:
        return (rng.integers(0, UNIT[t], size=shape) | (rng.integers(0, 2, size=shape) << 5)).astype(np.uint8)
    return rng.integers(0, 64, size=shape).astype(np.uint8)


def _pack(t, codes):
    if t == "e4m3":
        return np.ascontiguousarray(codes)
    if t == "e2m1":
        return inputs.pack_e2m1(codes)
    return inputs.pack_fp6(codes)


def _scale_range(t, integer):
    if not integer:
        return -4, 5
    if t == "e4m3":
        return 0, 2
    if t == "e2m1":
        return 1, 3
    e = inputs.fp6_integer_scale(t)
    return e, e + 1


def _mx_call(t, A, SFA, B, SFB, C, a_mn, b_mn, ws):
    kw = {"a_order": "mn" if a_mn else "k", "b_order": "mn" if b_mn else "k", "workspace": ws}
    if t == "e4m3":
        return tg.gemm_mxfp8(A, SFA, B, SFB, C, **kw)
    if t == "e2m1":
        return tg.gemm_mxfp4(A, SFA, B, SFB, C, **kw)
    return tg.gemm_mxfp6(A, SFA, B, SFB, C, fmt=t, **kw)


# M and N multiples of 4 (the binding's byte views of fp4 / fp6 storage
# rows); K multiples of 32; partial copy tiles; K % 512 == 0 (the four-wave
# kernels) and not; a persistent grid
SHAPESMX = [(100, 36, 96), (132, 68, 544), (4, 4, 32), (256, 192, 1024), (48, 112, 2080), (4200, 4300, 512)]


@pytest.mark.parametrize("t", ["e4m3", "e2m1", "e2m3", "e3m2"])
@pytest.mark.parametrize("orders", ORDERS, ids=["a_mn", "b_mn", "both"])
@pytest.mark.parametrize("shape", SHAPESMX, ids=["%dx%dx%d" % s for s in SHAPESMX])
def test_block_scaled(t, orders, shape):
    M, N, K = shape
    a_mn, b_mn = orders
    big = M * N > 4 * 10 ** 6
    for integer in ((True,) if big else (True, False)):
        rng = np.random.default_rng(M + 3 * N + K + len(t) + 5 * a_mn + b_mn)
        a = _codes(t, rng, (M, K), integer)
        b = _codes(t, rng, (N, K), integer)
        lo, hi = _scale_range(t, integer)
        SFA = (127 + rng.integers(lo, hi, size=(M, K // 32))).astype(np.uint8)
        SFB = (127 + rng.integers(lo, hi, size=(N, K // 32))).astype(np.uint8)
        C = None if big else (rng.integers(-4, 5, size=(M, N)) if integer
                              else rng.uniform(-1, 1, size=(M, N))).astype(np.float32)
        Cd = torch.from_numpy(C).to(DEV) if C is not None else None
        A = dev8(_pack(t, a.T) if a_mn else _pack(t, a))
        B = dev8(_pack(t, b.T) if b_mn else _pack(t, b))
        say("ex_ws %s a_mn=%s b_mn=%s %dx%dx%d integer=%s" % (t, a_mn, b_mn, M, N, K, integer))
        D = _mx_call(t, A, dev8(SFA), B, dev8(SFB), Cd, a_mn, b_mn, _workspace(t, M, N, K, a_mn, b_mn))
        torch.cuda.synchronize()
        if big:
            rand, forced = inputs.sample_indices(M, N, K)
            idx = np.concatenate([rand, forced])
            Dr, _ = oracle.gemm_ref(t, _pack(t, a), _pack(t, b), idx=idx, SFA=SFA, SFB=SFB)
            assert np.array_equal(to_f64(D).ravel()[idx], Dr)
            Dk = _mx_call(t, dev8(_pack(t, a)), dev8(SFA), dev8(_pack(t, b)), dev8(SFB), None, False, False, None)
            torch.cuda.synchronize()
            assert torch.equal(D, Dk)
            continue
        Dr, S = oracle.gemm_ref_full(t, _pack(t, a), _pack(t, b), C=C, SFA=SFA, SFB=SFB)
        Dg = to_f64(D)
        if integer:
            bad = np.argwhere(Dg != Dr)
            assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()
        else:
            rep = check.report(Dg, Dr, S)
            assert rep["fail"] == 0, rep


@pytest.mark.parametrize("t", ["e2m1", "e2m3"])
def test_c_abi_odd_m_padded_storage(t):
    """Through the C ABI: M not a multiple of the packing (the last storage
    byte of each K row half used), A storage rows padded past M."""
    M, N, K = 37, 20, 96
    rng = np.random.default_rng(5)
    a, b = _codes(t, rng, (M, K), True), _codes(t, rng, (N, K), True)
    lo, hi = _scale_range(t, True)
    SFA = (127 + rng.integers(lo, hi, size=(M, K // 32))).astype(np.uint8)
    SFB = (127 + rng.integers(lo, hi, size=(N, K // 32))).astype(np.uint8)
    lda = 48
    st = np.zeros((K, lda), np.uint8)
    st[:, :M] = a.T
    A, B = dev8(_pack(t, st)), dev8(_pack(t, b))
    Sa, Sb = dev8(SFA), dev8(SFB)
    D = torch.empty((M, N), dtype=torch.float32, device=DEV)
    ws = _workspace(t, M, N, K, True, False)
    nb = ws.numel()
    if t == "e2m1":
        s = tg.raw.gemm_mxfp4_ex_ws(M, N, K, A.data_ptr(), lda, 1, Sa.data_ptr(), K // 32, B.data_ptr(), K, 0,
                                    Sb.data_ptr(), K // 32, None, 0, D.data_ptr(), N, 0, ws.data_ptr(), nb, None)
    else:
        s = tg.raw.gemm_mxfp6_ex_ws(M, N, K, A.data_ptr(), lda, 1, Sa.data_ptr(), K // 32, B.data_ptr(), K, 0,
                                    Sb.data_ptr(), K // 32, None, 0, D.data_ptr(), N, 0, 0, ws.data_ptr(), nb, None)
    torch.cuda.synchronize()
    assert s == 0
    Dr, _ = oracle.gemm_ref_full(t, _pack(t, a), _pack(t, b), SFA=SFA, SFB=SFB)
    assert np.array_equal(to_f64(D), Dr)
