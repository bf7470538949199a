"""Pins of the oracle's block-scaled fp6 forms, e2m3 and e3m2 (CPU only).

a(m,k) = fp6(A, m, k) * 2^(SFA[m,k/32]-127), b likewise, D = C + sum_k a*b,
with A and B packed six bits per element (element k at bits 6k .. 6k+5 of
the row read as a little-endian bit string).  The pins use an independent
decoder (each fp6 code moved field by field, subnormals normalised by bit
manipulation, into the e4m3 code of the same value and decoded by torch's
float8_e4m3fn), an independent per-element unpacker, exact rational
arithmetic, the formats' published extreme values and one-hot operands.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tiled_dense_gemm_tile_amd import inputs

FMT = {"e2m3": (2, 3, 1), "e3m2": (3, 2, 3)}          # exponent bits, mantissa bits, bias


def fp6_via_e4m3(codes, in_type):
    """Decode fp6 codes through torch's e4m3 (bias 7, 3 mantissa bits)."""
    eb, mb, bias = FMT[in_type]
    out = []
    for c in np.asarray(codes, dtype=np.uint8).ravel():
        s = (int(c) >> 5) & 1
        e = (int(c) >> mb) & ((1 << eb) - 1)
        m = int(c) & ((1 << mb) - 1)
        if e == 0 and m == 0:
            e4 = 0
        elif e == 0:
            h = m.bit_length() - 1                      # leading one of the subnormal significand
            frac = (m - (1 << h)) << (3 - h) if h <= 3 else 0
            e4 = ((1 - bias + h - mb + 7) << 3) | (frac & 7)
        else:
            e4 = ((e - bias + 7) << 3) | ((m << (3 - mb)) & 7)
        out.append(e4 | (s << 7))
    t = torch.tensor(out, dtype=torch.uint8).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy().reshape(np.shape(codes))


def unpack6(packed, K):
    """Per-element bit extraction (independent of the oracle's unpacker)."""
    p = np.asarray(packed, dtype=np.uint8)
    rows = p.reshape(-1, p.shape[-1])
    out = np.zeros((rows.shape[0], K), dtype=np.uint8)
    for r in range(rows.shape[0]):
        bits = np.unpackbits(rows[r], bitorder="little")
        for k in range(K):
            out[r, k] = int(sum(int(bits[6 * k + b]) << b for b in range(6)))
    return out.reshape(p.shape[:-1] + (K,))


def exact_fp6(in_type, A, B, SFA, SFB, K, C=None):
    a = fp6_via_e4m3(unpack6(A, K), in_type)
    b = fp6_via_e4m3(unpack6(B, K), in_type)
    sa = np.ldexp(1.0, SFA.astype(np.int64) - 127)
    sb = np.ldexp(1.0, SFB.astype(np.int64) - 127)
    M, N = a.shape[0], b.shape[0]
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


@pytest.mark.parametrize("in_type", ["e2m3", "e3m2"])
def test_decoder_matches_independent_route(in_type):
    assert np.array_equal(oracle.decode_table(in_type), fp6_via_e4m3(np.arange(64), in_type))


def test_published_extremes():
    t = oracle.decode_table("e2m3")
    assert t.max() == 7.5 and t.min() == -7.5
    assert min(v for v in t if v > 0) == 0.125                 # smallest subnormal
    assert min(v for v in t[8:32]) == 1.0                      # smallest normal
    t = oracle.decode_table("e3m2")
    assert t.max() == 28.0 and t.min() == -28.0
    assert min(v for v in t if v > 0) == 0.0625
    assert min(v for v in t[4:32]) == 0.25
    for f in ("e2m3", "e3m2"):
        tb = oracle.decode_table(f)
        assert np.signbit(tb[32]) and tb[32] == 0.0            # code 0x20 is -0
        assert np.array_equal(tb[32:], -tb[:32])


def test_pack_unpack_agree():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 64, size=(5, 64)).astype(np.uint8)
    packed = inputs.pack_fp6(codes)
    assert packed.shape == (5, 48)
    assert np.array_equal(oracle.unpack_fp6(packed), codes)
    assert np.array_equal(unpack6(packed, 64), codes)
    # element 1 straddles bytes 0 and 1: code 0b111111 at k = 1 sets bits 6..11
    one = np.zeros((1, 4), np.uint8)
    one[0, 1] = 0x3F
    assert list(inputs.pack_fp6(one)[0]) == [0xC0, 0x0F, 0x00]


@pytest.mark.parametrize("in_type", ["e2m3", "e3m2"])
@pytest.mark.parametrize("shape", [(1, 1, 32), (2, 3, 64), (3, 2, 96), (1, 5, 128)])
def test_bruteforce_scaled(in_type, shape):
    M, N, K = shape
    rng = np.random.default_rng(M * 100 + N * 10 + K + len(in_type))
    A = inputs.random_codes(rng, in_type, (M, K))
    B = inputs.random_codes(rng, in_type, (N, K))
    SFA = (127 + rng.integers(-4, 5, size=(M, K // 32))).astype(np.uint8)
    SFB = (127 + rng.integers(-4, 5, size=(N, K // 32))).astype(np.uint8)
    C = rng.uniform(-1, 1, size=(M, N)).astype(np.float32)
    D, S = oracle.gemm_ref(in_type, A, B, C=C, SFA=SFA, SFB=SFB)
    De, Se = exact_fp6(in_type, A, B, SFA, SFB, K, C)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(D[m, n]) - De[m][n]) <= (K + 1) * Fraction(1, 2 ** 53) * (Se[m][n] + 1)
            assert Fraction(S[m, n]) == Se[m][n]


@pytest.mark.parametrize("in_type", ["e2m3", "e3m2"])
def test_integer_variant_is_exact(in_type):
    w = inputs.WORKLOADS["mxfp6_8192"]
    w = type(w)(w.name, w.M, w.N, w.K, in_type, w.out_type, w.dist_a, w.dist_b, w.dist_c, w.seed, scaled=True)
    x = inputs.generate(w, integer=True, M=5, N=4, K=128)
    D, _ = oracle.gemm_ref(in_type, x["A"], x["B"], SFA=x["SFA"], SFB=x["SFB"])
    De, _ = exact_fp6(in_type, x["A"], x["B"], x["SFA"], x["SFB"], 128)
    assert all(De[m][n].denominator == 1 for m in range(5) for n in range(4))
    assert all(Fraction(D[m, n]) == De[m][n] for m in range(5) for n in range(4))


@pytest.mark.parametrize("ka,kb", [(0, 0), (1, 1), (2, 2), (3, 3), (5, 5), (4, 5), (30, 31), (33, 33)])
def test_one_hot_positions(ka, kb):
    """A single element in A and in B, at K positions ka and kb (fields that
    start inside a byte and straddle two bytes included): they meet only
    when the positions agree."""
    K = 64
    a = np.zeros((1, K), np.uint8)
    b = np.zeros((1, K), np.uint8)
    a[0, ka] = 0x0B                                       # e2m3 1.375
    b[0, kb] = 0x16                                       # e2m3 3.5
    one = np.full((1, K // 32), 127, np.uint8)
    D, _ = oracle.gemm_ref("e2m3", inputs.pack_fp6(a), inputs.pack_fp6(b), SFA=one, SFB=one)
    assert D[0, 0] == (1.375 * 3.5 if ka == kb else 0.0)


def test_full_form_matches_loop():
    w = inputs.WORKLOADS["mxfp6_8192"]
    x = inputs.generate(w, M=37, N=29, K=192, seed=11)
    D, S = oracle.gemm_ref("e2m3", x["A"], x["B"], SFA=x["SFA"], SFB=x["SFB"])
    Df, Sf = oracle.gemm_ref_full("e2m3", x["A"], x["B"], SFA=x["SFA"], SFB=x["SFB"])
    assert np.allclose(D, Df, rtol=0, atol=1e-9 * (1 + S.max()))
    assert np.allclose(S, Sf, rtol=1e-12)


def test_fp6_needs_scales_and_whole_byte_groups():
    rng = np.random.default_rng(0)
    A = inputs.random_codes(rng, "e2m3", (2, 64))
    with pytest.raises(oracle.OracleError):
        oracle.gemm_ref("e2m3", A, A)
    one = np.full((2, 2), 127, np.uint8)
    with pytest.raises(ValueError):
        oracle.gemm_ref("e2m3", A[:, :47], A[:, :47], SFA=one, SFB=one)
