"""Parity of the block-scaled fp6 HIP path (e2m3 and e3m2) against the oracle
on an MI355X.

a(m,k) = fp6(A, m, k) * 2^(SFA[m,k/32]-127), b(k,n) = fp6(B, n, k) * 2^(SFB[n,k/32]-127),
A and B packed four elements per three bytes (element k at bits 6k .. 6k+5
of a row read as a little-endian bit string).  Bar: bit-exact on
integer-valued inputs (codes of magnitude at most 1 and a scale exponent
that makes them integers); otherwise |D - D_ref| <= 2^-12 * sum|a*b| + 1e-6.
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

FORMATS = ["e2m3", "e3m2"]


def _case(fmt, M, N, K, seed, integer, with_c=True):
    rng = np.random.default_rng(seed)
    A = inputs.random_codes(rng, fmt, (M, K), integer=integer)
    B = inputs.random_codes(rng, fmt, (N, K), integer=integer)
    if integer:
        e = inputs.fp6_integer_scale(fmt)
        SFA = np.full((M, K // 32), 127 + e, np.uint8)
        SFB = np.full((N, K // 32), 127 + e, np.uint8)
    else:
        SFA = (127 + rng.integers(-4, 5, size=(M, K // 32))).astype(np.uint8)
        SFB = (127 + rng.integers(-4, 5, size=(N, K // 32))).astype(np.uint8)
    C = None
    if with_c:
        C = (rng.integers(-4, 5, size=(M, N)) if integer else rng.uniform(-1, 1, size=(M, N))).astype(np.float32)
    return {"A": A, "B": B, "SFA": SFA, "SFB": SFB}, C


def _run(fmt, x, C=None, out=torch.float32):
    Cd = torch.from_numpy(C).to(DEV) if C is not None else None
    return tg.gemm_mxfp6(dev8(x["A"]), dev8(x["SFA"]), dev8(x["B"]), dev8(x["SFB"]), Cd, out_dtype=out, fmt=fmt)


def _full_check(fmt, x, Dg, integer, C=None):
    Dr, S = oracle.gemm_ref_full(fmt, x["A"], x["B"], C=C, SFA=x["SFA"], SFB=x["SFB"])
    if integer:
        bad = np.argwhere(Dg != Dr)
        assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()
    else:
        rep = check.report(Dg, Dr, S)
        assert rep["fail"] == 0, rep


# K a multiple of 512; M and N cover partial 256-row tiles, single rows and
# grids of several tiles.
SHAPES = [(64, 64, 512), (100, 70, 512), (256, 256, 1024), (300, 260, 1536), (513, 1000, 1024), (1, 1, 512),
          (257, 129, 2560), (777, 513, 2048)]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", SHAPES)
def test_small_shapes(fmt, shape):
    M, N, K = shape
    for integer in (True, False):
        x, C = _case(fmt, M, N, K, seed=M + 3 * N + K + len(fmt), integer=integer)
        say("mxfp6 %s %dx%dx%d integer=%s" % (fmt, M, N, K, integer))
        D = _run(fmt, x, C)
        torch.cuda.synchronize()
        _full_check(fmt, x, to_f64(D), integer, C)


@pytest.mark.parametrize("fmt", FORMATS)
def test_scale_structure(fmt):
    """Scales that differ per row, per column and per 32-wide K block (so a
    lane, block-row or epoch mix-up in the scale registers changes D); codes
    of magnitude at most 1 with exponents 3..5 keep every product an
    integer."""
    M, N, K = 256, 192, 2048
    x, _ = _case(fmt, M, N, K, seed=7, integer=True, with_c=False)
    nb = K // 32
    e = inputs.fp6_integer_scale(fmt)
    x["SFA"] = (127 + e + (np.arange(M)[:, None] + 2 * np.arange(nb)[None, :]) % 3).astype(np.uint8)
    x["SFB"] = (127 + e + (3 * np.arange(N)[:, None] + np.arange(nb)[None, :] // 2) % 3).astype(np.uint8)
    say("mxfp6 %s structured scales" % fmt)
    D = _run(fmt, x)
    torch.cuda.synchronize()
    _full_check(fmt, x, to_f64(D), True)


@pytest.mark.parametrize("fmt", FORMATS)
def test_one_hot_positions(fmt):
    """Each row of A and of B has one nonzero element, at a K position whose
    six-bit field starts at any bit of a byte (straddling two bytes or not):
    D[m, n] is nonzero only where the two positions coincide."""
    M, N, K = 64, 48, 1024
    rng = np.random.default_rng(12)
    ka = rng.integers(0, K, size=M)
    kb = np.concatenate([ka[:N // 2], rng.integers(0, K, size=N - N // 2)])
    a = np.zeros((M, K), np.uint8)
    b = np.zeros((N, K), np.uint8)
    a[np.arange(M), ka] = 0x1B                    # e2m3 5.5 / e3m2 14
    b[np.arange(N), kb] = 0x2E                    # e2m3 -1.75 / e3m2 -1.5
    x = {"A": inputs.pack_fp6(a), "B": inputs.pack_fp6(b),
         "SFA": (127 + rng.integers(-3, 4, size=(M, K // 32))).astype(np.uint8),
         "SFB": (127 + rng.integers(-3, 4, size=(N, K // 32))).astype(np.uint8)}
    say("mxfp6 %s one-hot rows" % fmt)
    D = _run(fmt, x)
    torch.cuda.synchronize()
    _full_check(fmt, x, to_f64(D), True)


def test_formats_differ():
    """The same bytes under the two formats give the two oracles' results (the
    format argument reaches the MFMA)."""
    x, _ = _case("e2m3", 256, 256, 512, seed=3, integer=False, with_c=False)
    for fmt in FORMATS:
        D = _run(fmt, x)
        torch.cuda.synchronize()
        _full_check(fmt, x, to_f64(D), False)


@pytest.mark.parametrize("fmt", FORMATS)
def test_padded_rows(fmt):
    """Leading dimensions past K: A and B rows of K + 64 and K + 128 elements
    whose padding holds the largest code, scale rows of K/32 + 16 and + 32
    bytes whose padding holds NaN codes."""
    M, N, K = 300, 290, 1536
    for integer in (True, False):
        x, C = _case(fmt, M, N, K, seed=31, integer=integer)
        nb, kb = K // 32, K // 4 * 3
        A = torch.full((M, kb + 48), 0xFF, dtype=torch.uint8, device=DEV)
        B = torch.full((N, kb + 96), 0xFF, dtype=torch.uint8, device=DEV)
        A[:, :kb] = dev8(x["A"])
        B[:, :kb] = dev8(x["B"])
        SFA = torch.full((M, nb + 16), 255, dtype=torch.uint8, device=DEV)
        SFB = torch.full((N, nb + 32), 255, dtype=torch.uint8, device=DEV)
        SFA[:, :nb] = dev8(x["SFA"])
        SFB[:, :nb] = dev8(x["SFB"])
        say("mxfp6 %s padded rows %dx%dx%d integer=%s" % (fmt, M, N, K, integer))
        D = tg.gemm_mxfp6(A[:, :kb], SFA[:, :nb], B[:, :kb], SFB[:, :nb], torch.from_numpy(C).to(DEV), fmt=fmt)
        torch.cuda.synchronize()
        _full_check(fmt, x, to_f64(D), integer, C)


def test_in_place_c():
    x, C = _case("e3m2", 260, 300, 1024, seed=9, integer=True)
    D = torch.from_numpy(C).to(DEV)
    say("mxfp6 in place")
    tg.gemm_mxfp6(dev8(x["A"]), dev8(x["SFA"]), dev8(x["B"]), dev8(x["SFB"]), D, D=D, fmt="e3m2")
    torch.cuda.synchronize()
    _full_check("e3m2", x, to_f64(D), True, C)


@pytest.mark.parametrize("fmt", FORMATS)
def test_bf16_output_is_rne_of_fp32(fmt):
    x, _ = _case(fmt, 640, 384, 1536, seed=5, integer=False, with_c=False)
    D32 = _run(fmt, x)
    D16 = _run(fmt, x, out=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(D16), oracle.rne_bf16_f32(D32.cpu().numpy()))


def test_k_zero_gives_c():
    M, N = 40, 50
    C = torch.randn(M, N, device=DEV)
    z = torch.empty(M, 0, dtype=torch.uint8, device=DEV)
    zb = torch.empty(N, 0, dtype=torch.uint8, device=DEV)
    D = tg.gemm_mxfp6(z, z, zb, zb, C)
    torch.cuda.synchronize()
    assert torch.equal(D, C)


def _big(fmt, integer):
    w = inputs.WORKLOADS["mxfp6_8192"]
    if fmt != w.in_type:
        w = type(w)(w.name, w.M, w.N, w.K, fmt, w.out_type, w.dist_a, w.dist_b, w.dist_c, w.seed, scaled=True)
    x = inputs.generate(w, integer=integer)
    say("mxfp6 %s 8192^3 integer=%s" % (fmt, integer))
    D = _run(fmt, x)
    torch.cuda.synchronize()
    Dg = D.cpu().numpy()
    del D
    rand, forced = inputs.sample_indices(w.M, w.N, w.seed)
    a, b = oracle.operands_f64(fmt, x["A"], x["B"], SFA=x["SFA"], SFB=x["SFB"])
    for name, idx in (("random", rand), ("forced", forced)):
        Dr, S = oracle.gemm_ref(fmt, x["A"], x["B"], SFA=x["SFA"], SFB=x["SFB"], idx=idx)
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


def test_mxfp6_8192():
    _big("e2m3", False)


def test_mxfp6_8192_integer():
    _big("e2m3", True)


def test_mxfp6_e3m2_8192():
    _big("e3m2", False)
