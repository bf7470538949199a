"""Block-scaled fp8, fp4 and fp6 grids of more 256 x 256 tiles than the GPU
has compute units, without C: the persistent four-wave kernels (one workgroup
per CU walking the tiles, its next tile's first loads in flight while the
finished tile's D is stored).

Bar: exact on integer-valued inputs against the oracle at 4096 seeded
samples plus the tile edges, within the tolerance on random inputs, and bit
for bit equal to the one-workgroup-per-tile kernel (same MFMAs in the same
order) over the whole of D, for fp32 and bf16 output.  Padding of a D with
ldd > N stays untouched.
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

# (M, N, K): ragged rows and columns (17 x 17 tiles); 32 x 32 tiles (four
# per CU); 17 x 16 tiles, one K group; 2 tiles past one per CU, long K
CASES = [(4200, 4300, 1024), (8192, 8192, 512), (4352, 4096, 512), (4100, 4104, 2048)]


# fp8: integer codes in [-4, 4] with scale exponents 0, 1; fp4: any code
# with exponents 1, 2; fp6: codes of magnitude at most 1 with the format's
# integer exponent (every product an integer)
def _int_exponents(fmt):
    if fmt == "e4m3":
        return 0, 2
    if fmt == "e2m1":
        return 1, 3
    e = inputs.fp6_integer_scale(fmt)
    return e, e + 1


def _inputs(M, N, K, seed, integer, fmt="e4m3"):
    rng = np.random.default_rng(seed)
    A = inputs.random_codes(rng, fmt, (M, K), integer=integer)
    B = inputs.random_codes(rng, fmt, (N, K), integer=integer)
    lo, hi = _int_exponents(fmt) if integer else (-4, 5)
    SFA = (127 + rng.integers(lo, hi, size=(M, K // 32))).astype(np.uint8)
    SFB = (127 + rng.integers(lo, hi, size=(N, K // 32))).astype(np.uint8)
    return A, B, SFA, SFB


def _call(fmt, A, SFA, B, SFB, **kw):
    if fmt in ("e2m3", "e3m2"):
        return tg.gemm_mxfp6(A, SFA, B, SFB, fmt=fmt, **kw)
    fn = tg.gemm_mxfp8 if fmt == "e4m3" else tg.gemm_mxfp4
    return fn(A, SFA, B, SFB, **kw)


def _sampled_check(A, B, SFA, SFB, Dg, integer, seed, fmt="e4m3"):
    M, N = Dg.shape
    rand, forced = inputs.sample_indices(M, N, seed)
    idx = np.concatenate([rand, forced])
    Dr, S = oracle.gemm_ref(fmt, A, B, idx=idx, SFA=SFA, SFB=SFB)
    got = Dg.ravel()[idx]
    if integer:
        assert np.array_equal(got, Dr)
    else:
        rep = check.report(got, Dr, S)
        assert rep["fail"] == 0, rep


# the switch that sends a call to the one-workgroup-per-tile kernel instead
PER_TILE = {"e4m3": ("TILEGEMM_MX_CONFIG", "4"), "e2m1": ("TILEGEMM_MX4_PERSIST", "0"),
            "e2m3": ("TILEGEMM_MX6_PERSIST", "0"), "e3m2": ("TILEGEMM_MX6_PERSIST", "0")}
FORMATS = ["e4m3", "e2m1", "e2m3", "e3m2"]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("case", CASES, ids=["%dx%dx%d" % c for c in CASES])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("integer", [True, False])
def test_persistent_grid(fmt, case, out, integer, monkeypatch):
    M, N, K = case
    A, B, SFA, SFB = _inputs(M, N, K, M + N + K + integer, integer, fmt)
    dA, dB, dSA, dSB = dev8(A), dev8(B), dev8(SFA), dev8(SFB)
    say("mx persistent %s %dx%dx%d %s integer=%s" % (fmt, M, N, K, out, integer))
    D = _call(fmt, dA, dSA, dB, dSB, out_dtype=out)
    monkeypatch.setenv(*PER_TILE[fmt])
    D1 = _call(fmt, dA, dSA, dB, dSB, out_dtype=out)
    torch.cuda.synchronize()
    assert torch.equal(D, D1)
    if out == torch.float32:
        _sampled_check(A, B, SFA, SFB, to_f64(D), integer, M + N, fmt)
    else:
        # bf16 D: the round-to-nearest-even of the fp32 result (itself
        # checked against the oracle by the float32 cases)
        monkeypatch.delenv(PER_TILE[fmt][0])
        D32 = _call(fmt, dA, dSA, dB, dSB)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(D), oracle.rne_bf16_f32(D32.cpu().numpy()))


@pytest.mark.parametrize("fmt", FORMATS)
def test_padded_d_rows_untouched(fmt):
    M, N, K, pad = 4200, 4300, 512, 68
    A, B, SFA, SFB = _inputs(M, N, K, 11, True, fmt)
    Dbig = torch.full((M, N + pad), float("nan"), dtype=torch.float32, device=DEV)
    D = Dbig[:, :N]
    say("mx persistent %s padded D" % fmt)
    _call(fmt, dev8(A), dev8(SFA), dev8(B), dev8(SFB), D=D)
    torch.cuda.synchronize()
    assert bool(torch.isnan(Dbig[:, N:]).all())
    _sampled_check(A, B, SFA, SFB, to_f64(D), True, 5, fmt)


@pytest.mark.parametrize("fmt", FORMATS)
def test_calls_in_a_row_of_different_grids(fmt):
    """Consecutive calls of the persistent kernel with different tile counts
    and a smaller second grid (each workgroup's walk ends with its grid)."""
    for (M, N, K) in [(8192, 4352, 512), (4200, 4300, 512), (4608, 4096, 1024)]:
        A, B, SFA, SFB = _inputs(M, N, K, M + 2 * N, True, fmt)
        say("mx persistent %s in a row %dx%dx%d" % (fmt, M, N, K))
        D = _call(fmt, dev8(A), dev8(SFA), dev8(B), dev8(SFB))
        torch.cuda.synchronize()
        _sampled_check(A, B, SFA, SFB, to_f64(D), True, M, fmt)


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_fp6_persistent_k_tail(fmt, monkeypatch):
    """fp6 with K % 512 != 0 (a last scale group short of 512 K, its bytes
    past K cleared after every tile change) and K of one tile (128)."""
    for (M, N, K) in [(4200, 4300, 640), (4608, 4100, 128)]:
        A, B, SFA, SFB = _inputs(M, N, K, M + K, True, fmt)
        dA, dB, dSA, dSB = dev8(A), dev8(B), dev8(SFA), dev8(SFB)
        say("mx persistent %s K tail %dx%dx%d" % (fmt, M, N, K))
        D = _call(fmt, dA, dSA, dB, dSB)
        monkeypatch.setenv(*PER_TILE[fmt])
        D1 = _call(fmt, dA, dSA, dB, dSB)
        monkeypatch.delenv(PER_TILE[fmt][0])
        torch.cuda.synchronize()
        assert torch.equal(D, D1)
        _sampled_check(A, B, SFA, SFB, to_f64(D), True, M, fmt)
