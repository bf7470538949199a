"""Parity of MN-contiguous operand storage (gemm_bf16_ex / gemm_fp16_ex, and
the binding's stride detection) against the oracle on an MI355X.

The logical operands are drawn exactly as for the K-contiguous calls and only
their storage changes: A as K x M (a(m,k) = A[k*lda + m]) and/or B as K x N
(b(k,n) = B[k*ldb + n]).  The oracle sees the same logical matrices in its
own K-contiguous form.  Bar: bit-exact on integer inputs, otherwise
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
    from gpuutil import DEV, bf16_bits, dev16, say, to_f64

TORCH = {"bf16": torch.bfloat16, "fp16": torch.float16}


def _stored(codes, in_type, mn, pad=0):
    """Device view (rows, K) of the logical codes (rows x K), stored
    K-contiguous or, when mn, as a K x ld row-major array with ld = rows
    rounded up to a multiple of 8, plus pad (16-byte rows)."""
    if not mn:
        return dev16(codes, in_type)
    rows, K = codes.shape
    st = np.zeros((K, (rows + 7) // 8 * 8 + pad), dtype=np.uint16)
    st[:, :rows] = codes.T
    return dev16(st, in_type)[:, :rows].t()


def _run(in_type, A, B, C, a_mn, b_mn, out=torch.float32, pad=0):
    fn = tg.gemm_bf16 if in_type == "bf16" else tg.gemm_fp16
    Cd = torch.from_numpy(C).to(DEV) if C is not None else None
    if Cd is not None and out == torch.bfloat16:
        Cd = Cd.to(torch.bfloat16)
    Ad, Bd = _stored(A, in_type, a_mn, pad), _stored(B, in_type, b_mn, pad)
    return fn(Ad, Bd, Cd, out_dtype=out)


def _case(in_type, M, N, K, seed, integer, with_c=True):
    rng = np.random.default_rng(seed)
    A = inputs.random_codes(rng, in_type, (M, K), integer=integer)
    B = inputs.random_codes(rng, in_type, (N, K), integer=integer)
    C = None
    if with_c:
        C = (rng.integers(-4, 5, size=(M, N)) if integer else rng.uniform(-1, 1, size=(M, N))).astype(np.float32)
    return A, B, C


def _check(in_type, A, B, C, Dg, integer):
    Dr, S = oracle.gemm_ref_full(in_type, A, B, C=C)
    if integer:
        bad = np.argwhere(Dg != Dr)
        assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()
    else:
        rep = check.report(Dg, Dr, S)
        assert rep["fail"] == 0, rep


ORDERS = [(True, False), (False, True), (True, True)]
# K-contiguous operands need K % 8 == 0 here; with both MN-contiguous any K
SHAPES = [(256, 256, 256), (300, 200, 520), (513, 1000, 1024), (1, 1, 64), (64, 40, 8), (257, 129, 136),
          (100, 300, 4104)]


@pytest.mark.parametrize("in_type", ["bf16", "fp16"])
@pytest.mark.parametrize("orders", ORDERS)
@pytest.mark.parametrize("shape", SHAPES)
def test_orders(in_type, orders, shape):
    a_mn, b_mn = orders
    M, N, K = shape
    for integer in (True, False):
        A, B, C = _case(in_type, M, N, K, seed=M + 5 * N + K + 7 * a_mn + 11 * b_mn, integer=integer)
        say("layout %s a_mn=%s b_mn=%s %dx%dx%d integer=%s" % (in_type, a_mn, b_mn, M, N, K, integer))
        D = _run(in_type, A, B, C, a_mn, b_mn)
        torch.cuda.synchronize()
        _check(in_type, A, B, C, to_f64(D), integer)


@pytest.mark.parametrize("K", [1, 7, 61, 130, 1003])
def test_both_mn_any_k(K):
    """Both operands MN-contiguous: K needs no alignment (rows past K read as
    zero from the per-tile resource)."""
    A, B, C = _case("bf16", 200, 136, K, seed=K, integer=True)
    D = _run("bf16", A, B, C, True, True)
    torch.cuda.synchronize()
    _check("bf16", A, B, C, to_f64(D), True)


def test_padded_leading_dimensions():
    A, B, C = _case("fp16", 300, 264, 1000, seed=3, integer=False)
    for orders in ORDERS:
        D = _run("fp16", A, B, C, *orders, pad=24)
        torch.cuda.synchronize()
        _check("fp16", A, B, C, to_f64(D), False)


def test_bf16_output_is_rne_of_fp32():
    A, B, _ = _case("bf16", 384, 320, 1024, seed=4, integer=False, with_c=False)
    D32 = _run("bf16", A, B, None, False, True)
    D16 = _run("bf16", A, B, None, False, True, out=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(D16), oracle.rne_bf16_f32(D32.cpu().numpy()))


def test_same_values_as_k_contiguous_on_integers():
    A, B, C = _case("bf16", 512, 768, 2048, seed=5, integer=True)
    ref = _run("bf16", A, B, C, False, False)
    for orders in ORDERS:
        D = _run("bf16", A, B, C, *orders)
        torch.cuda.synchronize()
        assert torch.equal(D, ref), orders


def test_unsupported_alignment_is_refused():
    M, N, K = 64, 64, 100                              # K % 8 != 0 with one K-contiguous operand
    A = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    Bs = torch.zeros((K, N), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(tg.GemmError) as ei:
        tg.gemm_bf16(A, Bs.t())
    assert ei.value.status == 5
    A2 = torch.zeros((M, 128), dtype=torch.bfloat16, device=DEV)
    Bs3 = torch.zeros((128, N + 4), dtype=torch.bfloat16, device=DEV)[:, :N]   # ldb % 8 != 0
    with pytest.raises(tg.GemmError) as ei:
        tg.gemm_bf16(A2, Bs3.t())
    assert ei.value.status == 5


def test_c_abi_orders_and_bad_ld():
    M, N, K = 128, 96, 64
    A = torch.zeros((K, M), dtype=torch.bfloat16, device=DEV)
    B = torch.zeros((N, K), dtype=torch.bfloat16, device=DEV)
    D = torch.empty((M, N), dtype=torch.float32, device=DEV)
    L = tg.raw
    assert L.gemm_bf16_ex(M, N, K, A.data_ptr(), M - 8, 1, B.data_ptr(), K, 0, None, 0, D.data_ptr(), N, 0, None) == 3
    assert L.gemm_bf16_ex(M, N, K, A.data_ptr(), M, 2, B.data_ptr(), K, 0, None, 0, D.data_ptr(), N, 0, None) == 5
    assert L.gemm_bf16_ex(M, N, K, A.data_ptr(), M, 1, B.data_ptr(), K, 0, None, 0, D.data_ptr(), N, 0, None) == 0
    torch.cuda.synchronize()
    assert torch.count_nonzero(D) == 0


def _big(b_mn, integer):
    w = inputs.WORKLOADS["square4096_bf16"]
    x = inputs.generate(w, integer=integer)
    say("layout square4096 b_mn=%s integer=%s" % (b_mn, integer))
    D = _run("bf16", x["A"], x["B"], x["C"], not b_mn, b_mn)
    torch.cuda.synchronize()
    Dg = D.cpu().numpy()
    rand, forced = inputs.sample_indices(w.M, w.N, w.seed)
    a, b = oracle.operands_f64("bf16", x["A"], x["B"])
    for name, idx in (("random", rand), ("forced", forced)):
        Dr, S = oracle.gemm_ref("bf16", x["A"], x["B"], C=x["C"], idx=idx)
        got = Dg.ravel()[idx].astype(np.float64)
        if integer:
            assert np.array_equal(got, Dr), name
        else:
            rep = check.report(got, Dr, S)
            assert rep["fail"] == 0, (name, rep)
    ok, ratio = check.freivalds_blocks(Dg, a, b, x["C"], block=64, integer=integer)
    say("  freivalds ok=%s worst %.3g" % (ok, ratio))
    assert ok


@pytest.mark.parametrize("b_mn", [False, True])
def test_square4096(b_mn):
    _big(b_mn, False)


def test_square4096_integer_b_mn():
    _big(True, True)
