"""Pins of the oracle's definition of D = A.B + C (CPU only).

Each test fixes the oracle against something other than itself: exact rational
arithmetic with decoders taken from torch/numpy dtypes, closed forms, scale
special cases, and the IEEE formats' own tables.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tiled_dense_gemm_tile_amd import inputs


# ---- independent decoders (library dtypes, not oracle.c) -------------------

def lib_decode(in_type, bits):
    bits = np.asarray(bits)
    if in_type == "bf16":
        t = torch.from_numpy(bits.astype(np.uint16).view(np.int16).copy()).view(torch.bfloat16)
        return t.to(torch.float64).numpy()
    if in_type == "fp16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if in_type == "e4m3":
        t = torch.from_numpy(bits.astype(np.uint8).copy()).view(torch.float8_e4m3fn)
        return t.to(torch.float64).numpy()
    if in_type == "e8m0":
        t = torch.from_numpy(bits.astype(np.uint8).copy()).view(torch.float8_e8m0fnu)
        return t.to(torch.float64).numpy()
    raise ValueError(in_type)


def exact_gemm(in_type, A, B, C=None, SFA=None, SFB=None, K=None):
    """Exact D and S with Python Fractions, operands decoded by library dtypes."""
    M, N = A.shape[0], B.shape[0]
    K = A.shape[1] if K is None else K
    a = lib_decode(in_type, A[:, :K])
    b = lib_decode(in_type, B[:, :K])
    if SFA is not None:
        sa = lib_decode("e8m0", SFA)
        sb = lib_decode("e8m0", SFB)
    D = [[None] * N for _ in range(M)]
    S = [[None] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            sab = Fraction(0)
            for k in range(K):
                x = Fraction(float(a[m, k]))
                y = Fraction(float(b[n, k]))
                if SFA is not None:
                    x *= Fraction(float(sa[m, k // 32]))
                    y *= Fraction(float(sb[n, k // 32]))
                acc += x * y
                sab += abs(x * y)
            c = Fraction(float(C[m, n])) if C is not None else Fraction(0)
            D[m][n] = c + acc
            S[m][n] = sab
    return D, S


SHAPES = [(0, 1, 1), (1, 0, 2), (1, 1, 0), (1, 1, 1), (2, 3, 5), (3, 2, 8), (5, 5, 17),
          (8, 3, 2), (1, 17, 3), (17, 1, 5), (3, 5, 1)]


@pytest.mark.parametrize("in_type", ["bf16", "fp16"])
@pytest.mark.parametrize("shape", SHAPES)
def test_bruteforce_fraction(in_type, shape):
    M, N, K = shape
    rng = np.random.default_rng(hash(shape) % 1000 + (7 if in_type == "fp16" else 0))
    A = inputs.random_codes(rng, in_type, (M, K))
    B = inputs.random_codes(rng, in_type, (N, K))
    C = rng.uniform(-1, 1, size=(M, N)).astype(np.float32)
    D, S = oracle.gemm_ref(in_type, A, B, K=K, C=C)
    De, Se = exact_gemm(in_type, A, B, C)
    for m in range(M):
        for n in range(N):
            # fp64 sum of K exact products: error below K * 2^-53 * S (plus C)
            bound = float((K + 1) * Fraction(1, 2 ** 53) * (Se[m][n] + abs(Fraction(float(C[m, n])))))
            assert abs(Fraction(D[m, n]) - De[m][n]) <= bound
            assert S[m, n] == float(Se[m][n])  # |products| are exact, sums of these tiny sets too


@pytest.mark.parametrize("in_type", ["bf16", "fp16"])
def test_bruteforce_integer_exact(in_type):
    rng = np.random.default_rng(3)
    M, N, K = 5, 7, 17
    A = inputs.random_codes(rng, in_type, (M, K), integer=True)
    B = inputs.random_codes(rng, in_type, (N, K), integer=True)
    C = rng.integers(-4, 5, size=(M, N)).astype(np.float32)
    D, _ = oracle.gemm_ref(in_type, A, B, C=C)
    De, _ = exact_gemm(in_type, A, B, C)
    assert all(Fraction(D[m, n]) == De[m][n] for m in range(M) for n in range(N))


def test_bruteforce_scaled_e4m3():
    rng = np.random.default_rng(11)
    M, N, K = 3, 4, 64
    A = inputs.random_codes(rng, "e4m3", (M, K))
    B = inputs.random_codes(rng, "e4m3", (N, K))
    SFA = (127 + rng.integers(-4, 5, size=(M, 2))).astype(np.uint8)
    SFB = (127 + rng.integers(-4, 5, size=(N, 2))).astype(np.uint8)
    D, S = oracle.gemm_ref("e4m3", A, B, SFA=SFA, SFB=SFB)
    De, Se = exact_gemm("e4m3", A, B, SFA=SFA, SFB=SFB)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(D[m, n]) - De[m][n]) <= K * Fraction(1, 2 ** 53) * Se[m][n]
            assert Fraction(S[m, n]) == Se[m][n]


def test_padded_leading_dimensions():
    """lda/ldb larger than K: the padding never enters the sum."""
    rng = np.random.default_rng(5)
    M, N, K = 4, 6, 9
    A = inputs.random_codes(rng, "bf16", (M, K + 7))
    B = inputs.random_codes(rng, "bf16", (N, K + 3))
    D, _ = oracle.gemm_ref("bf16", A, B, K=K)
    D2, _ = oracle.gemm_ref("bf16", np.ascontiguousarray(A[:, :K]), np.ascontiguousarray(B[:, :K]))
    assert np.array_equal(D, D2)


# ---- closed forms -----------------------------------------------------------

ONE_BF16 = 0x3F80


def _eye_codes(n, in_type):
    one = ONE_BF16 if in_type == "bf16" else 0x3C00
    I = np.zeros((n, n), dtype=np.uint16)
    I[np.arange(n), np.arange(n)] = one
    return I


@pytest.mark.parametrize("in_type", ["bf16", "fp16"])
def test_identity_A(in_type):
    rng = np.random.default_rng(1)
    n, N = 9, 5
    B = inputs.random_codes(rng, in_type, (N, n))
    C = rng.integers(-4, 5, size=(n, N)).astype(np.float32)
    D, _ = oracle.gemm_ref(in_type, _eye_codes(n, in_type), B, C=C)
    # a(m,k) = delta_mk  =>  D[m,n] = b(m,n) + C[m,n] = B[n,m] + C[m,n]
    assert np.array_equal(D, lib_decode(in_type, B).T + C)


@pytest.mark.parametrize("in_type", ["bf16", "fp16"])
def test_identity_B(in_type):
    rng = np.random.default_rng(2)
    M, n = 6, 8
    A = inputs.random_codes(rng, in_type, (M, n))
    D, _ = oracle.gemm_ref(in_type, A, _eye_codes(n, in_type))
    assert np.array_equal(D, lib_decode(in_type, A))


def test_zero_A_and_K0_give_C():
    rng = np.random.default_rng(3)
    M, N, K = 5, 4, 7
    C = rng.uniform(-1, 1, size=(M, N)).astype(np.float32)
    B = inputs.random_codes(rng, "bf16", (N, K))
    D, S = oracle.gemm_ref("bf16", np.zeros((M, K), np.uint16), B, C=C)
    assert np.array_equal(D, C.astype(np.float64)) and not S.any()
    D0, S0 = oracle.gemm_ref("bf16", np.zeros((M, 0), np.uint16), np.zeros((N, 0), np.uint16), C=C)
    assert np.array_equal(D0, C.astype(np.float64)) and not S0.any()


def test_all_ones():
    M, N, K = 3, 4, 37
    A = np.full((M, K), ONE_BF16, np.uint16)
    B = np.full((N, K), ONE_BF16, np.uint16)
    C = np.arange(M * N, dtype=np.float32).reshape(M, N)
    D, S = oracle.gemm_ref("bf16", A, B, C=C)
    assert np.array_equal(D, K + C) and np.all(S == K)


def test_one_hot_row_selects_column():
    rng = np.random.default_rng(4)
    M, N, K = 4, 6, 10
    B = inputs.random_codes(rng, "bf16", (N, K))
    A = np.zeros((M, K), np.uint16)
    A[2, 7] = ONE_BF16
    D, _ = oracle.gemm_ref("bf16", A, B)
    assert np.array_equal(D[2], lib_decode("bf16", B[:, 7]))
    assert not D[[0, 1, 3]].any()


def test_sign_and_transpose_sensitivity():
    """A non-symmetric product: swapping operands or dropping a sign must change D."""
    A = np.array([[0x3F80, 0x4000]], np.uint16)       # [1, 2]
    B = np.array([[0x4040, 0xBF80]], np.uint16)       # column [3, -1]
    D, S = oracle.gemm_ref("bf16", A, B)
    assert D[0, 0] == 1 * 3 + 2 * -1 and S[0, 0] == 5


def test_bf16_C_type():
    C = np.array([[0x3FC0]], np.uint16)  # 1.5
    A = np.array([[ONE_BF16]], np.uint16)
    D, _ = oracle.gemm_ref("bf16", A, A, C=C, c_type="bf16")
    assert D[0, 0] == 2.5


# ---- decoders ---------------------------------------------------------------

def _same(x, y):
    x, y = np.asarray(x), np.asarray(y)
    return np.array_equal(np.isnan(x), np.isnan(y)) and np.array_equal(x[~np.isnan(x)], y[~np.isnan(y)]) \
        and np.array_equal(np.signbit(x[~np.isnan(x)]), np.signbit(y[~np.isnan(y)]))


def test_decode_bf16_exhaustive():
    codes = np.arange(65536)
    assert _same(oracle.decode_table("bf16"), lib_decode("bf16", codes))


def test_decode_fp16_exhaustive():
    codes = np.arange(65536)
    assert _same(oracle.decode_table("fp16"), lib_decode("fp16", codes))


def test_decode_e4m3_exhaustive():
    tab = oracle.decode_table("e4m3")
    assert _same(tab, lib_decode("e4m3", np.arange(256)))
    for c in range(256):
        s, e, f = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and f == 7:
            assert np.isnan(tab[c])
            continue
        v = (f / 8) * 2.0 ** -6 if e == 0 else (1 + f / 8) * 2.0 ** (e - 7)
        assert tab[c] == (-v if s else v)
    assert np.nanmax(tab) == 448.0


def test_decode_e8m0_exhaustive():
    tab = oracle.decode_table("e8m0")
    for c in range(255):
        assert tab[c] == 2.0 ** (c - 127)
    assert np.isnan(tab[255])
    assert _same(tab, lib_decode("e8m0", np.arange(256)))


def test_decode_f32_samples():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(2000).astype(np.float32),
                        np.array([0.0, -0.0, 1e-45, -1e-40, 3.4e38, np.inf], np.float32)])
    for v in x:
        assert oracle.dec_f32(int(v.view(np.uint32))) == float(v)


def test_rne_bf16_matches_torch():
    rng = np.random.default_rng(9)
    # random magnitudes across the range, exact ties, subnormals, near overflow
    base = rng.standard_normal(20000).astype(np.float32) * np.float32(2.0) ** rng.integers(-130, 120, 20000).astype(np.float32)
    ties = (np.arange(1, 2000, dtype=np.uint32) << 15).view(np.float32)   # low 16 bits = 0x8000 -> tie
    ties = np.concatenate([ties, ((np.arange(1, 2000, dtype=np.uint32) << 16) | 0x8000).view(np.float32)])
    extra = np.array([0.0, -0.0, 1e-41, -1e-41, 3.3895e38, 3.4e38, -3.39e38, 1.0, 1.00390625, 1.01171875],
                     np.float32)
    x = np.concatenate([base, ties, extra])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.rne_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)
    assert np.array_equal(oracle.rne_bf16_f32(x), ref)


# ---- block scales -----------------------------------------------------------

def _scaled_case(seed=21, M=4, N=5, K=96):
    rng = np.random.default_rng(seed)
    A = inputs.random_codes(rng, "e4m3", (M, K))
    B = inputs.random_codes(rng, "e4m3", (N, K))
    return rng, A, B


def test_unit_scales_equal_unscaled():
    rng, A, B = _scaled_case()
    ones = lambda r: np.full((r, 3), 127, np.uint8)
    D1, _ = oracle.gemm_ref("e4m3", A, B, SFA=ones(4), SFB=ones(5))
    D0, _ = oracle.gemm_ref("e4m3", A, B)
    assert np.array_equal(D1, D0)


def test_row_constant_scale_is_power_of_two_factor():
    rng, A, B = _scaled_case()
    SFA = np.full((4, 3), 127, np.uint8)
    SFA[1, :] = 127 + 3
    SFA[2, :] = 127 - 4
    SFB = np.full((5, 3), 127, np.uint8)
    SFB[3, :] = 127 + 2
    D, _ = oracle.gemm_ref("e4m3", A, B, SFA=SFA, SFB=SFB)
    D0, _ = oracle.gemm_ref("e4m3", A, B)
    fa = np.array([1, 8, 1 / 16, 1])[:, None]
    fb = np.array([1, 1, 1, 4, 1])[None, :]
    assert np.array_equal(D, D0 * fa * fb)


def test_one_block_perturbed_changes_only_its_products():
    rng, A, B = _scaled_case()
    SFA = np.full((4, 3), 127, np.uint8)
    SFB = np.full((5, 3), 127, np.uint8)
    D0, _ = oracle.gemm_ref("e4m3", A, B, SFA=SFA, SFB=SFB)
    SFA2 = SFA.copy()
    SFA2[2, 1] = 128          # doubles k = 32..63 of row 2
    D1, _ = oracle.gemm_ref("e4m3", A, B, SFA=SFA2, SFB=SFB)
    assert np.array_equal(np.delete(D1, 2, axis=0), np.delete(D0, 2, axis=0))
    a = lib_decode("e4m3", A[2, 32:64])
    b = lib_decode("e4m3", B[:, 32:64])
    assert np.allclose(D1[2] - D0[2], b @ a, rtol=0, atol=1e-12)


def test_scaled_errors():
    rng, A, B = _scaled_case(K=48)
    with pytest.raises(oracle.OracleError):
        oracle.gemm_ref("e4m3", A, B, SFA=np.full((4, 2), 127, np.uint8), SFB=np.full((5, 2), 127, np.uint8))
    rng, A, B = _scaled_case()
    bad = np.full((4, 3), 127, np.uint8)
    bad[0, 0] = 255
    with pytest.raises(oracle.OracleError):
        oracle.gemm_ref("e4m3", A, B, SFA=bad, SFB=np.full((5, 3), 127, np.uint8))


# ---- the whole-matrix form --------------------------------------------------

@pytest.mark.parametrize("in_type,scaled", [("bf16", False), ("fp16", False), ("e4m3", True)])
def test_full_matches_naive(in_type, scaled):
    rng = np.random.default_rng(17)
    M, N, K = 37, 29, 160
    A = inputs.random_codes(rng, in_type, (M, K))
    B = inputs.random_codes(rng, in_type, (N, K))
    C = rng.uniform(-1, 1, size=(M, N)).astype(np.float32)
    SFA = SFB = None
    if scaled:
        SFA = (127 + rng.integers(-4, 5, size=(M, K // 32))).astype(np.uint8)
        SFB = (127 + rng.integers(-4, 5, size=(N, K // 32))).astype(np.uint8)
    D, S = oracle.gemm_ref(in_type, A, B, C=C, SFA=SFA, SFB=SFB)
    Df, Sf = oracle.gemm_ref_full(in_type, A, B, C=C, SFA=SFA, SFB=SFB)
    assert np.all(np.abs(D - Df) <= 4 * K * 2.0 ** -53 * (S + np.abs(C)))
    assert np.allclose(S, Sf, rtol=1e-13, atol=0)
    idx = np.array([0, 5, M * N - 1, 100])
    Di, Si = oracle.gemm_ref(in_type, A, B, C=C, SFA=SFA, SFB=SFB, idx=idx)
    assert np.array_equal(Di, D.ravel()[idx]) and np.array_equal(Si, S.ravel()[idx])


def test_full_bf16_c_matches_naive():
    """The whole-matrix form with C given as bf16 bits: C decoded as bf16
    (bits << 16), the same as the naive loop's bf16 C; a one-element case
    whose C alone decides the result pins the decoding by value."""
    rng = np.random.default_rng(23)
    M, N, K = 19, 23, 96
    A = inputs.random_codes(rng, "bf16", (M, K))
    B = inputs.random_codes(rng, "bf16", (N, K))
    C = inputs.random_codes(rng, "bf16", (M, N))
    D, S = oracle.gemm_ref("bf16", A, B, C=C, c_type="bf16")
    Df, Sf = oracle.gemm_ref_full("bf16", A, B, C=C, c_type="bf16")
    cval = (C.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.abs(D - Df) <= 4 * K * 2.0 ** -53 * (S + np.abs(cval)))
    Z = np.zeros((1, 4), np.uint16)
    Dz, _ = oracle.gemm_ref_full("bf16", Z, Z, C=np.array([[0xC0A0]], np.uint16), c_type="bf16")
    assert Dz[0, 0] == -5.0
