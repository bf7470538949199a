"""Pins of the oracle's block-scaled fp4 (e2m1) form (CPU only).

a(m,k) = e2m1(A[m,k]) * 2^(SFA[m,k/32]-127), b likewise, D = C + sum_k a*b,
with A and B stored two elements per byte (element 2i in the low nibble of
byte i).  The pins below use an independent decoder (each e2m1 code mapped
field by field to the e4m3 code of the same value and decoded by torch's
float8_e4m3fn), exact rational arithmetic, the format's published value set
and one-hot operands.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tiled_dense_gemm_tile_amd import inputs

# OCP microscaling FP4 (E2M1): the eight magnitudes, codes 0..7; codes 8..15
# are their negatives.
E2M1_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def e2m1_via_e4m3(codes):
    """Decode e2m1 codes through torch's e4m3: sign, exponent and mantissa
    fields moved into the e4m3 layout (bias 1 -> 7, 1 -> 3 mantissa bits)."""
    codes = np.asarray(codes, dtype=np.uint8)
    s = (codes >> 3) & 1
    e = (codes >> 1) & 3
    m = codes & 1
    e4 = np.where(e == 0, np.where(m == 1, 0x30, 0x00),      # 0.5 = 2^-1: e4m3 exponent 6
                  ((e + 6) << 3) | (m << 2)).astype(np.uint8)
    e4 = e4 | (s << 7).astype(np.uint8)
    t = torch.from_numpy(e4.copy()).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def unpack(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def exact_fp4(A, B, SFA, SFB, C=None):
    a = e2m1_via_e4m3(unpack(A))
    b = e2m1_via_e4m3(unpack(B))
    sa = np.ldexp(1.0, SFA.astype(np.int64) - 127)
    sb = np.ldexp(1.0, SFB.astype(np.int64) - 127)
    M, K = a.shape
    N = b.shape[0]
    D = [[None] * N for _ in range(M)]
    S = [[None] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc, sab = Fraction(0), Fraction(0)
            for k in range(K):
                p = Fraction(float(a[m, k])) * Fraction(float(sa[m, k // 32])) * \
                    Fraction(float(b[n, k])) * Fraction(float(sb[n, k // 32]))
                acc += p
                sab += abs(p)
            D[m][n] = acc + (Fraction(float(C[m, n])) if C is not None else 0)
            S[m][n] = sab
    return D, S


def test_decode_e2m1_value_set():
    tab = oracle.decode_table("e2m1")
    assert list(tab[:8]) == E2M1_VALUES
    assert list(tab[8:]) == [-v for v in E2M1_VALUES]
    assert np.signbit(tab[8])                        # code 8 is -0


def test_decode_e2m1_matches_independent_route():
    codes = np.arange(16)
    assert np.array_equal(oracle.decode_table("e2m1"), e2m1_via_e4m3(codes))


@pytest.mark.parametrize("shape", [(1, 1, 32), (2, 3, 64), (3, 2, 96), (5, 4, 32), (1, 7, 128)])
def test_bruteforce_scaled_e2m1(shape):
    M, N, K = shape
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    A = inputs.random_codes(rng, "e2m1", (M, K))
    B = inputs.random_codes(rng, "e2m1", (N, K))
    SFA = (127 + rng.integers(-4, 5, size=(M, K // 32))).astype(np.uint8)
    SFB = (127 + rng.integers(-4, 5, size=(N, K // 32))).astype(np.uint8)
    C = rng.uniform(-1, 1, size=(M, N)).astype(np.float32)
    D, S = oracle.gemm_ref("e2m1", A, B, C=C, SFA=SFA, SFB=SFB)
    De, Se = exact_fp4(A, B, SFA, SFB, C)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(D[m, n]) - De[m][n]) <= (K + 1) * Fraction(1, 2 ** 53) * (Se[m][n] + 1)
            assert Fraction(S[m, n]) == Se[m][n]


def test_integer_variant_is_exact():
    w = inputs.WORKLOADS["mxfp4_8192"]
    x = inputs.generate(w, integer=True, M=6, N=5, K=256)
    D, _ = oracle.gemm_ref("e2m1", x["A"], x["B"], SFA=x["SFA"], SFB=x["SFB"])
    De, _ = exact_fp4(x["A"], x["B"], x["SFA"], x["SFB"])
    assert all(De[m][n].denominator == 1 for m in range(6) for n in range(5))
    assert all(Fraction(D[m, n]) == De[m][n] for m in range(6) for n in range(5))


@pytest.mark.parametrize("ka,kb", [(0, 0), (1, 1), (6, 7), (7, 6), (33, 33), (40, 41)])
def test_nibble_order(ka, kb):
    """Element k sits in the low nibble of byte k/2 when k is even, the high
    nibble when odd: one-hot rows meet only when their K positions agree."""
    K = 64
    a = np.zeros((1, K), np.uint8)
    b = np.zeros((1, K), np.uint8)
    a[0, ka] = 2                                       # 1.0
    b[0, kb] = 7                                       # 6.0
    A, B = inputs.pack_e2m1(a), inputs.pack_e2m1(b)
    assert A[0, ka // 2] == (2 if ka % 2 == 0 else 0x20)
    one = np.full((1, K // 32), 127, np.uint8)
    D, _ = oracle.gemm_ref("e2m1", A, B, SFA=one, SFB=one)
    assert D[0, 0] == (6.0 if ka == kb else 0.0)


def test_row_scale_is_power_of_two_factor():
    rng = np.random.default_rng(3)
    M, N, K = 4, 3, 64
    A = inputs.random_codes(rng, "e2m1", (M, K))
    B = inputs.random_codes(rng, "e2m1", (N, K))
    one_a = np.full((M, K // 32), 127, np.uint8)
    one_b = np.full((N, K // 32), 127, np.uint8)
    D0, _ = oracle.gemm_ref("e2m1", A, B, SFA=one_a, SFB=one_b)
    sa = one_a.copy()
    sa[2, :] = 127 + 3
    D1, _ = oracle.gemm_ref("e2m1", A, B, SFA=sa, SFB=one_b)
    assert np.array_equal(D1[2], 8.0 * D0[2])
    assert np.array_equal(np.delete(D1, 2, 0), np.delete(D0, 2, 0))


def test_full_form_matches_loop():
    w = inputs.WORKLOADS["mxfp4_8192"]
    x = inputs.generate(w, M=37, N=29, K=192, seed=11)
    D, S = oracle.gemm_ref("e2m1", x["A"], x["B"], SFA=x["SFA"], SFB=x["SFB"])
    Df, Sf = oracle.gemm_ref_full("e2m1", x["A"], x["B"], SFA=x["SFA"], SFB=x["SFB"])
    assert np.allclose(D, Df, rtol=0, atol=1e-9 * (1 + S.max()))
    assert np.allclose(S, Sf, rtol=1e-12)


def test_e2m1_needs_scales_and_whole_blocks():
    rng = np.random.default_rng(0)
    A = inputs.random_codes(rng, "e2m1", (2, 64))
    with pytest.raises(oracle.OracleError):
        oracle.gemm_ref("e2m1", A, A)
    one = np.full((2, 2), 127, np.uint8)
    with pytest.raises(oracle.OracleError):
        oracle.gemm_ref("e2m1", A, A, K=48, SFA=one, SFB=one)
