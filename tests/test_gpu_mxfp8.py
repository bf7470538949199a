"""Parity of the block-scaled fp8 HIP path against the oracle on an MI355X.

a(m,k) = e4m3(A[m,k]) * 2^(SFA[m,k/32]-127), b(k,n) = e4m3(B[n,k]) * 2^(SFB[n,k/32]-127).
Bar: bit-exact on integer-valued inputs (e4m3 integers in [-4, 4], scale
exponents in {0, 1, 2}); otherwise |D - D_ref| <= 2^-12 * sum|a*b| + 1e-6.
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
    A = inputs.random_codes(rng, "e4m3", (M, K), integer=integer)
    B = inputs.random_codes(rng, "e4m3", (N, K), integer=integer)
    lo, hi = (0, 3) if integer else (-4, 5)
    SFA = (127 + rng.integers(lo, hi, size=(M, K // 32))).astype(np.uint8)
    SFB = (127 + rng.integers(lo, hi, size=(N, K // 32))).astype(np.uint8)
    C = None
    if with_c:
        C = (rng.integers(-4, 5, size=(M, N)) if integer else rng.uniform(-1, 1, size=(M, N))).astype(np.float32)
    return {"A": A, "B": B, "SFA": SFA, "SFB": SFB}, C


def _run(x, C=None, out=torch.float32):
    Cd = torch.from_numpy(C).to(DEV) if C is not None else None
    return tg.gemm_mxfp8(dev8(x["A"]), dev8(x["SFA"]), dev8(x["B"]), dev8(x["SFB"]), Cd, out_dtype=out)


def _full_check(x, Dg, integer, C=None):
    Dr, S = oracle.gemm_ref_full("e4m3", x["A"], x["B"], C=C, SFA=x["SFA"], SFB=x["SFB"])
    if integer:
        bad = np.argwhere(Dg != Dr)
        assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()
    else:
        rep = check.report(Dg, Dr, S)
        assert rep["fail"] == 0, rep


SHAPES = [(64, 64, 128), (32, 32, 256), (100, 70, 256), (256, 256, 128), (300, 260, 384), (513, 1000, 1024),
          (1, 1, 128), (257, 129, 640)]


@pytest.mark.parametrize("shape", SHAPES)
def test_small_shapes(shape):
    M, N, K = shape
    for integer in (True, False):
        x, C = _case(M, N, K, seed=M + 3 * N + K, integer=integer)
        say("mxfp8 %dx%dx%d integer=%s" % (M, N, K, integer))
        D = _run(x, C)
        torch.cuda.synchronize()
        _full_check(x, to_f64(D), integer, C)


def test_scale_structure():
    """Scales that differ per row, per column and per 32-wide K block in a
    pattern tied to the MFMA lane halves: a lane/block mix-up changes D."""
    M, N, K = 128, 96, 512
    x, _ = _case(M, N, K, seed=7, integer=True, with_c=False)
    nb = K // 32
    x["SFA"] = (127 + (np.arange(M)[:, None] + 2 * np.arange(nb)[None, :]) % 5 - 2).astype(np.uint8)
    x["SFB"] = (127 + (3 * np.arange(N)[:, None] + np.arange(nb)[None, :]) % 4 - 1).astype(np.uint8)
    say("mxfp8 structured scales")
    D = _run(x)
    torch.cuda.synchronize()
    _full_check(x, to_f64(D), True)


# Kernel configurations (csrc/mx_launch.hpp): 0 .. 3 the two- and
# three-slot kernels, 4 the four-wave kernel (K % 512 == 0, 16-byte scale rows).
@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_every_config(cfg, monkeypatch):
    monkeypatch.setenv("TILEGEMM_MX_CONFIG", str(cfg))
    for (M, N, K) in [(300, 520, 256), (777, 513, 1024), (520, 300, 384), (1100, 1030, 2048)]:
        for integer in (True, False):
            x, C = _case(M, N, K, seed=cfg * 13 + M, integer=integer)
            say("mx cfg %d %dx%dx%d integer=%s" % (cfg, M, N, K, integer))
            D = _run(x, C)
            torch.cuda.synchronize()
            _full_check(x, to_f64(D), integer, C)


@pytest.mark.parametrize("cfg", [0, 4])
def test_padded_scale_rows(cfg, monkeypatch):
    """Scale arrays with leading dimensions past K/32 (multiples of 16 bytes,
    so the 16-byte scale loads of the four-wave kernel apply)."""
    monkeypatch.setenv("TILEGEMM_MX_CONFIG", str(cfg))
    M, N, K = 300, 290, 1536
    for integer in (True, False):
        x, C = _case(M, N, K, seed=31 + cfg, integer=integer)
        nb = K // 32
        SFA = torch.full((M, nb + 16), 255, dtype=torch.uint8, device=DEV)   # padding is NaN codes
        SFB = torch.full((N, nb + 32), 255, dtype=torch.uint8, device=DEV)
        SFA[:, :nb] = dev8(x["SFA"])
        SFB[:, :nb] = dev8(x["SFB"])
        say("mx cfg %d padded scales %dx%dx%d integer=%s" % (cfg, M, N, K, integer))
        D = tg.gemm_mxfp8(dev8(x["A"]), SFA[:, :nb], dev8(x["B"]), SFB[:, :nb], torch.from_numpy(C).to(DEV))
        torch.cuda.synchronize()
        _full_check(x, to_f64(D), integer, C)


def test_bf16_output_is_rne_of_fp32():
    x, _ = _case(640, 384, 768, seed=5, integer=False, with_c=False)
    D32 = _run(x)
    D16 = _run(x, out=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(D16), oracle.rne_bf16_f32(D32.cpu().numpy()))


def test_k_zero_gives_c():
    M, N = 40, 50
    C = torch.randn(M, N, device=DEV)
    z = torch.empty(M, 0, dtype=torch.uint8, device=DEV)
    zb = torch.empty(N, 0, dtype=torch.uint8, device=DEV)
    D = tg.gemm_mxfp8(z, z, zb, zb, C)
    torch.cuda.synchronize()
    assert torch.equal(D, C)


def _big(integer):
    w = inputs.WORKLOADS["mxfp8_8192"]
    x = inputs.generate(w, integer=integer)
    say("mxfp8 8192^3 integer=%s" % integer)
    D = _run(x)
    torch.cuda.synchronize()
    Dg = D.cpu().numpy()
    del D
    rand, forced = inputs.sample_indices(w.M, w.N, w.seed)
    a, b = oracle.operands_f64("e4m3", x["A"], x["B"], SFA=x["SFA"], SFB=x["SFB"])
    for name, idx in (("random", rand), ("forced", forced)):
        Dr, S = oracle.gemm_ref("e4m3", x["A"], x["B"], SFA=x["SFA"], SFB=x["SFB"], idx=idx)
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


def test_mxfp8_8192():
    _big(False)


def test_mxfp8_8192_integer():
    _big(True)
