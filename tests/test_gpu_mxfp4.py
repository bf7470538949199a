"""Parity of the block-scaled fp4 HIP path against the oracle on an MI355X.

a(m,k) = e2m1(A, m, k) * 2^(SFA[m,k/32]-127), b(k,n) = e2m1(B, n, k) * 2^(SFB[n,k/32]-127),
A and B two elements per byte (element 2i in the low nibble of byte i).
Bar: bit-exact on integer-valued inputs (any e2m1 code, scale exponents in
{1, 2}, so every product is an integer); otherwise
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
    from gpuutil import DEV, bf16_bits, dev8, say, to_f64


def _case(M, N, K, seed, integer, with_c=True):
    rng = np.random.default_rng(seed)
    A = inputs.random_codes(rng, "e2m1", (M, K))
    B = inputs.random_codes(rng, "e2m1", (N, K))
    lo, hi = (1, 3) if integer else (-4, 5)
    SFA = (127 + rng.integers(lo, hi, size=(M, K // 32))).astype(np.uint8)
    SFB = (127 + rng.integers(lo, hi, size=(N, K // 32))).astype(np.uint8)
    C = None
    if with_c:
        C = (rng.integers(-4, 5, size=(M, N)) if integer else rng.uniform(-1, 1, size=(M, N))).astype(np.float32)
    return {"A": A, "B": B, "SFA": SFA, "SFB": SFB}, C


def _run(x, C=None, out=torch.float32):
    Cd = torch.from_numpy(C).to(DEV) if C is not None else None
    return tg.gemm_mxfp4(dev8(x["A"]), dev8(x["SFA"]), dev8(x["B"]), dev8(x["SFB"]), Cd, out_dtype=out)


def _full_check(x, Dg, integer, C=None):
    Dr, S = oracle.gemm_ref_full("e2m1", x["A"], x["B"], C=C, SFA=x["SFA"], SFB=x["SFB"])
    if integer:
        bad = np.argwhere(Dg != Dr)
        assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()
    else:
        rep = check.report(Dg, Dr, S)
        assert rep["fail"] == 0, rep


# K a multiple of 512; M and N cover partial 256-row tiles, single rows and
# grids of several tiles.
SHAPES = [(64, 64, 512), (32, 32, 1024), (100, 70, 512), (256, 256, 512), (300, 260, 1536), (513, 1000, 1024),
          (1, 1, 512), (257, 129, 2560), (777, 513, 2048), (1100, 1030, 2048)]


@pytest.mark.parametrize("shape", SHAPES)
def test_small_shapes(shape):
    M, N, K = shape
    for integer in (True, False):
        x, C = _case(M, N, K, seed=M + 3 * N + K, integer=integer)
        say("mxfp4 %dx%dx%d integer=%s" % (M, N, K, integer))
        D = _run(x, C)
        torch.cuda.synchronize()
        _full_check(x, to_f64(D), integer, C)


def test_scale_structure():
    """Scales that differ per row, per column and per 32-wide K block (so a
    lane, block-row or step mix-up in the scale registers changes D)."""
    M, N, K = 256, 192, 1536
    x, _ = _case(M, N, K, seed=7, integer=True, with_c=False)
    nb = K // 32
    x["SFA"] = (128 + (np.arange(M)[:, None] + 2 * np.arange(nb)[None, :]) % 3).astype(np.uint8)
    x["SFB"] = (128 + (3 * np.arange(N)[:, None] + np.arange(nb)[None, :] // 2) % 3).astype(np.uint8)
    say("mxfp4 structured scales")
    D = _run(x)
    torch.cuda.synchronize()
    _full_check(x, to_f64(D), True)


def test_one_hot_blocks():
    """Each row of A and of B has one nonzero element, in a different 32-wide
    K block and byte half per row: D[m, n] is nonzero only where the two
    positions coincide, with the product of both block scales."""
    M, N, K = 64, 48, 1024
    rng = np.random.default_rng(12)
    ka = rng.integers(0, K, size=M)
    kb = np.concatenate([ka[:N // 2], rng.integers(0, K, size=N - N // 2)])
    a = np.zeros((M, K), np.uint8)
    b = np.zeros((N, K), np.uint8)
    a[np.arange(M), ka] = 7                       # 6.0
    b[np.arange(N), kb] = 3                       # 1.5
    x = {"A": inputs.pack_e2m1(a), "B": inputs.pack_e2m1(b),
         "SFA": (127 + rng.integers(-3, 4, size=(M, K // 32))).astype(np.uint8),
         "SFB": (127 + rng.integers(-3, 4, size=(N, K // 32))).astype(np.uint8)}
    say("mxfp4 one-hot rows")
    D = _run(x)
    torch.cuda.synchronize()
    _full_check(x, to_f64(D), True)


def test_padded_rows():
    """Leading dimensions past K: A and B rows of K + 64 elements, scale rows
    of K/32 + 16 and + 32 bytes whose padding holds NaN codes."""
    M, N, K = 300, 290, 1536
    for integer in (True, False):
        x, C = _case(M, N, K, seed=31, integer=integer)
        nb, kb = K // 32, K // 2
        A = torch.zeros((M, kb + 32), dtype=torch.uint8, device=DEV)
        B = torch.zeros((N, kb + 48), dtype=torch.uint8, device=DEV)
        A[:, :kb] = dev8(x["A"])
        B[:, :kb] = dev8(x["B"])
        A[:, kb:] = 0x77                           # 6.0 in both nibbles: must never be read
        B[:, kb:] = 0x77
        SFA = torch.full((M, nb + 16), 255, dtype=torch.uint8, device=DEV)
        SFB = torch.full((N, nb + 32), 255, dtype=torch.uint8, device=DEV)
        SFA[:, :nb] = dev8(x["SFA"])
        SFB[:, :nb] = dev8(x["SFB"])
        say("mxfp4 padded rows %dx%dx%d integer=%s" % (M, N, K, integer))
        D = tg.gemm_mxfp4(A[:, :kb], SFA[:, :nb], B[:, :kb], SFB[:, :nb], torch.from_numpy(C).to(DEV))
        torch.cuda.synchronize()
        _full_check(x, to_f64(D), integer, C)


def test_in_place_c():
    x, C = _case(260, 300, 1024, seed=9, integer=True)
    D = torch.from_numpy(C).to(DEV)
    say("mxfp4 in place")
    tg.gemm_mxfp4(dev8(x["A"]), dev8(x["SFA"]), dev8(x["B"]), dev8(x["SFB"]), D, D=D)
    torch.cuda.synchronize()
    _full_check(x, to_f64(D), True, C)


def test_bf16_output_is_rne_of_fp32():
    x, _ = _case(640, 384, 1536, seed=5, integer=False, with_c=False)
    D32 = _run(x)
    D16 = _run(x, out=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(D16), oracle.rne_bf16_f32(D32.cpu().numpy()))


def test_k_zero_gives_c():
    M, N = 40, 50
    C = torch.randn(M, N, device=DEV)
    z = torch.empty(M, 0, dtype=torch.uint8, device=DEV)
    zb = torch.empty(N, 0, dtype=torch.uint8, device=DEV)
    D = tg.gemm_mxfp4(z, z, zb, zb, C)
    torch.cuda.synchronize()
    assert torch.equal(D, C)


def _big(integer):
    w = inputs.WORKLOADS["mxfp4_8192"]
    x = inputs.generate(w, integer=integer)
    say("mxfp4 8192^3 integer=%s" % integer)
    D = _run(x)
    torch.cuda.synchronize()
    Dg = D.cpu().numpy()
    del D
    rand, forced = inputs.sample_indices(w.M, w.N, w.seed)
    a, b = oracle.operands_f64("e2m1", x["A"], x["B"], SFA=x["SFA"], SFB=x["SFB"])
    for name, idx in (("random", rand), ("forced", forced)):
        Dr, S = oracle.gemm_ref("e2m1", x["A"], x["B"], SFA=x["SFA"], SFB=x["SFB"], idx=idx)
        got = Dg.ravel()[idx].astype(np.float64)
        if integer:
            assert np.array_equal(got, Dr), name
        else:
            rep = check.report(got, Dr, S)
            say("  %s: %s" % (name, rep))
            assert rep["fail"] == 0, (name, rep)
    ok, ratio = check.freivalds_blocks(Dg, a, b, None, block=64, integer=integer)
    say("  freivalds ok=%s worst %.3g" % (ok, ratio))
    assert ok


def test_mxfp4_8192():
    _big(False)


def test_mxfp4_8192_integer():
    _big(True)
