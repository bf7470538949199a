"""Pins of the oracle's block-scaled form with scale blocks wider than 32 K
elements (CPU only).

The pages define block scaling as one scale factor per (row, K block) of A
and per (column, K block) of B ("Tensor Core 数据布局的演进", section
Block-Scaled MMA 的 Scale Factors), without fixing the block width; the
standard form uses 32.  A block width kb (a multiple of 32, up to one scale
per row) is the same definition with a wider block.  Each test fixes the
oracle against something other than itself: exact rational arithmetic with
library decoders, the equivalence with the 32-wide form on replicated
scales, per-row closed forms, and a perturbed block.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tiled_dense_gemm_tile_amd import inputs


def lib_decode(fmt, bits):
    t = torch.from_numpy(np.asarray(bits, dtype=np.uint8).copy())
    dt = {"e4m3": torch.float8_e4m3fn, "e8m0": torch.float8_e8m0fnu}[fmt]
    return t.view(dt).to(torch.float64).numpy()


def exact_scaled(A, B, SFA, SFB, kb):
    """Exact e4m3 D with Fractions; scale j of a row covers K [j kb, (j+1) kb)."""
    M, K = A.shape
    N = B.shape[0]
    a, b = lib_decode("e4m3", A), lib_decode("e4m3", B)
    sa, sb = lib_decode("e8m0", SFA), lib_decode("e8m0", SFB)
    D = np.empty((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += (Fraction(float(a[m, k])) * Fraction(float(sa[m, k // kb])) *
                        Fraction(float(b[n, k])) * Fraction(float(sb[n, k // kb])))
            D[m, n] = acc
    return D


def _case(M, N, K, kb, seed):
    rng = np.random.default_rng(seed)
    A = inputs.random_codes(rng, "e4m3", (M, K))
    B = inputs.random_codes(rng, "e4m3", (N, K))
    nsc = -(-K // kb)
    SFA = (127 + rng.integers(-4, 5, size=(M, nsc))).astype(np.uint8)
    SFB = (127 + rng.integers(-4, 5, size=(N, nsc))).astype(np.uint8)
    return A, B, SFA, SFB


@pytest.mark.parametrize("K,kb", [(64, 64), (128, 64), (96, 64), (128, 128), (160, 96), (96, 96), (64, 4096)])
def test_bruteforce_fraction(K, kb):
    A, B, SFA, SFB = _case(3, 4, K, kb, seed=K + kb)
    D, S = oracle.gemm_ref("e4m3", A, B, SFA=SFA, SFB=SFB, kblock=kb)
    De = exact_scaled(A, B, SFA, SFB, kb)
    for m in range(3):
        for n in range(4):
            assert abs(Fraction(D[m, n]) - De[m, n]) <= K * Fraction(1, 2 ** 53) * Fraction(S[m, n])


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1", "e2m3", "e3m2"])
@pytest.mark.parametrize("kb", [64, 128, 96])
def test_equals_32_wide_form_on_replicated_scales(fmt, kb):
    """Scale j of a kb-wide block applies to the 32-wide blocks j kb/32 ..
    (j+1) kb/32 - 1: the 32-wide form on the replicated scales gives the
    same D and S bit for bit."""
    rng = np.random.default_rng(kb)
    M, N, K = 5, 7, 384
    A = inputs.random_codes(rng, fmt, (M, K))
    B = inputs.random_codes(rng, fmt, (N, K))
    nsc = -(-K // kb)
    SFA = (127 + rng.integers(-4, 5, size=(M, nsc))).astype(np.uint8)
    SFB = (127 + rng.integers(-4, 5, size=(N, nsc))).astype(np.uint8)
    rep = np.arange(K // 32) * 32 // kb
    D, S = oracle.gemm_ref(fmt, A, B, SFA=SFA, SFB=SFB, kblock=kb)
    D32, S32 = oracle.gemm_ref(fmt, A, B, SFA=SFA[:, rep], SFB=SFB[:, rep])
    assert np.array_equal(D, D32) and np.array_equal(S, S32)


def test_one_scale_per_row_is_a_power_of_two_factor():
    """kb >= K: one scale per row of A and column of B, so D = 2^(sa + sb) D_unscaled."""
    rng = np.random.default_rng(3)
    M, N, K = 4, 6, 256
    A = inputs.random_codes(rng, "e4m3", (M, K))
    B = inputs.random_codes(rng, "e4m3", (N, K))
    ea, eb = rng.integers(-4, 5, size=M), rng.integers(-4, 5, size=N)
    SFA = (127 + ea[:, None]).astype(np.uint8)
    SFB = (127 + eb[:, None]).astype(np.uint8)
    D, _ = oracle.gemm_ref("e4m3", A, B, SFA=SFA, SFB=SFB, kblock=K)
    D0, _ = oracle.gemm_ref("e4m3", A, B)
    assert np.array_equal(D, D0 * np.exp2(ea)[:, None] * np.exp2(eb)[None, :])


def test_one_wide_block_perturbed_changes_only_its_products():
    rng = np.random.default_rng(9)
    M, N, K, kb = 4, 5, 256, 128
    A = inputs.random_codes(rng, "e4m3", (M, K))
    B = inputs.random_codes(rng, "e4m3", (N, K))
    SFA = np.full((M, 2), 127, np.uint8)
    SFB = np.full((N, 2), 127, np.uint8)
    D0, _ = oracle.gemm_ref("e4m3", A, B, SFA=SFA, SFB=SFB, kblock=kb)
    SFB2 = SFB.copy()
    SFB2[3, 1] = 129          # x4 on k = 128 .. 255 of column 3
    D1, _ = oracle.gemm_ref("e4m3", A, B, SFA=SFA, SFB=SFB2, kblock=kb)
    assert np.array_equal(np.delete(D1, 3, axis=1), np.delete(D0, 3, axis=1))
    a = lib_decode("e4m3", A[:, 128:])
    b = lib_decode("e4m3", B[3, 128:])
    assert np.allclose(D1[:, 3] - D0[:, 3], 3 * (a @ b), rtol=0, atol=1e-12)


def test_block_width_errors():
    A, B, SFA, SFB = _case(2, 2, 64, 64, seed=1)
    for kb in (0, 16, 48, -32):
        with pytest.raises(oracle.OracleError):
            oracle.gemm_ref("e4m3", A, B, SFA=SFA, SFB=SFB, kblock=kb)
    bad = SFA.copy()
    bad[1, 0] = 255
    with pytest.raises(oracle.OracleError):
        oracle.gemm_ref("e4m3", A, B, SFA=bad, SFB=SFB, kblock=64)
