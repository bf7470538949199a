"""Parity of MN-contiguous block-scaled operands (gemm_mxfp8_ex,
gemm_mxfp4_ex, gemm_mxfp6_ex and the binding's a_order / b_order) against
the oracle on an MI355X.

The logical operands are drawn as for the K-contiguous calls and only their
storage changes: A as K x M (element (m, k) at [k, m]) and/or B as K x N,
packed along the contiguous dimension; scales keep their M x K/32 and
N x K/32 layout.  The oracle sees the same logical matrices in its own
K-contiguous form.  Bar: bit-exact on integer inputs, otherwise
|D - D_ref| <= 2^-12 * sum|a*b| + 1e-6.
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
    from gpuutil import DEV, dev8, say, to_f64

TYPES = ["e4m3", "e2m1", "e2m3", "e3m2"]
UNIT = {"e2m3": 9, "e3m2": 13}                      # fp6 codes of magnitude <= 1


def _codes(t, rng, shape, integer):
    """Unpacked element codes (one per uint8)."""
    if t == "e4m3":
        return inputs.random_codes(rng, t, shape, integer=integer)
    if t == "e2m1":
        return rng.integers(0, 16, size=shape).astype(np.uint8)
    if integer:
        return (rng.integers(0, UNIT[t], size=shape) | (rng.integers(0, 2, size=shape) << 5)).astype(np.uint8)
    return rng.integers(0, 64, size=shape).astype(np.uint8)


def _pack(t, codes):
    """Pack element codes along the last axis."""
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


def _case(t, M, N, K, seed, integer):
    rng = np.random.default_rng(seed)
    a = _codes(t, rng, (M, K), integer)
    b = _codes(t, rng, (N, K), integer)
    lo, hi = _scale_range(t, integer)
    SFA = (127 + rng.integers(lo, hi, size=(M, K // 32))).astype(np.uint8)
    SFB = (127 + rng.integers(lo, hi, size=(N, K // 32))).astype(np.uint8)
    C = (rng.integers(-4, 5, size=(M, N)) if integer else rng.uniform(-1, 1, size=(M, N))).astype(np.float32)
    return a, b, SFA, SFB, C


def _run(t, a, b, SFA, SFB, C, a_mn, b_mn):
    A = dev8(_pack(t, a.T) if a_mn else _pack(t, a))
    B = dev8(_pack(t, b.T) if b_mn else _pack(t, b))
    kw = {"a_order": "mn" if a_mn else "k", "b_order": "mn" if b_mn else "k"}
    Cd = torch.from_numpy(C).to(DEV)
    if t == "e4m3":
        D = tg.gemm_mxfp8(A, dev8(SFA), B, dev8(SFB), Cd, **kw)
    elif t == "e2m1":
        D = tg.gemm_mxfp4(A, dev8(SFA), B, dev8(SFB), Cd, **kw)
    else:
        D = tg.gemm_mxfp6(A, dev8(SFA), B, dev8(SFB), Cd, fmt=t, **kw)
    torch.cuda.synchronize()
    return D


def _check(t, a, b, SFA, SFB, C, Dg, integer):
    Dr, S = oracle.gemm_ref_full(t, _pack(t, a), _pack(t, b), C=C, SFA=SFA, SFB=SFB)
    if integer:
        bad = np.argwhere(Dg != Dr)
        assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()
    else:
        rep = check.report(Dg, Dr, S)
        assert rep["fail"] == 0, rep


ORDERS = [(True, False), (False, True), (True, True)]
# M and N multiples of 4 (the binding's byte views of fp4 / fp6 storage rows);
# fp8 storage rows that are 16-byte multiples (M, N % 16 == 0) take the
# staged transposing-read path, the others byte gathers
SHAPES = [(64, 64, 128), (100, 36, 96), (132, 68, 544), (4, 4, 32), (256, 192, 1024), (96, 80, 160),
          (48, 112, 2080)]


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("orders", ORDERS)
@pytest.mark.parametrize("shape", SHAPES)
def test_orders(t, orders, shape):
    M, N, K = shape
    for integer in (True, False):
        a, b, SFA, SFB, C = _case(t, M, N, K, seed=M + 3 * N + K + len(t) + 7 * orders[0], integer=integer)
        say("mx layout %s a_mn=%s b_mn=%s %dx%dx%d integer=%s" % (t, *orders, M, N, K, integer))
        D = _run(t, a, b, SFA, SFB, C, *orders)
        _check(t, a, b, SFA, SFB, C, to_f64(D), integer)


@pytest.mark.parametrize("t", TYPES)
def test_same_values_as_k_contiguous_on_integers(t):
    a, b, SFA, SFB, C = _case(t, 160, 96, 1024, seed=11, integer=True)
    ref = _run(t, a, b, SFA, SFB, C, False, False)
    for orders in ORDERS:
        assert torch.equal(_run(t, a, b, SFA, SFB, C, *orders), ref), orders


@pytest.mark.parametrize("t", ["e2m1", "e2m3"])
def test_c_abi_odd_m_and_padded_storage(t):
    """Through the C ABI: M not a multiple of the packing (the last storage
    byte of each K row half used), A storage rows padded past M."""
    M, N, K = 37, 20, 96
    a, b, SFA, SFB, C = _case(t, M, N, K, seed=5, integer=True)
    lda = 48                                         # elements per storage row of A (>= M)
    st = np.zeros((K, lda), np.uint8)
    st[:, :M] = a.T
    A = dev8(_pack(t, st))
    B = dev8(_pack(t, b))
    Sa, Sb, Cd = dev8(SFA), dev8(SFB), torch.from_numpy(C).to(DEV)
    D = torch.empty((M, N), dtype=torch.float32, device=DEV)
    if t == "e2m1":
        s = tg.raw.gemm_mxfp4_ex(M, N, K, A.data_ptr(), lda, 1, Sa.data_ptr(), K // 32, B.data_ptr(), K, 0,
                                 Sb.data_ptr(), K // 32, Cd.data_ptr(), N, D.data_ptr(), N, 0, None)
    else:
        s = tg.raw.gemm_mxfp6_ex(M, N, K, A.data_ptr(), lda, 1, Sa.data_ptr(), K // 32, B.data_ptr(), K, 0,
                                 Sb.data_ptr(), K // 32, Cd.data_ptr(), N, D.data_ptr(), N, 0, 0, None)
    torch.cuda.synchronize()
    assert s == 0
    _check(t, a, b, SFA, SFB, C, to_f64(D), True)
