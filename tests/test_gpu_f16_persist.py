"""bf16 / fp16 grids of more 256 x 256 tiles than the GPU has compute units,
without C, with 16-byte rows: the persistent four-wave kernel (one workgroup
per CU walking the tiles, its next tile's first loads in flight while the
finished tile's D is stored).

Bar: bit for bit equal to the one-workgroup-per-tile kernel (the same MFMAs
in the same order) over the whole of D; exact on integer-valued inputs
against the oracle at 4096 seeded samples plus the tile edges (fp32 out),
within the tolerance on random inputs; bf16 D the round-to-nearest-even of
the fp32 D.  K covers a tail tile, a single K tile (the path that clears
what its loads bring from past K after each tile change) and two tiles.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import check
from tiled_dense_gemm_tile_amd import inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpuutil import DEV, bf16_bits, dev16, run16, say, to_f64

# (M, N, K): ragged rows and columns (17 x 17 tiles); 32 x 32 tiles;
# 17 x 16 tiles with a K tail (520 = 8 x 64 + 8); one K tile of 40; two K
# tiles
CASES = [(4200, 4300, 1024), (8192, 8192, 256), (4352, 4096, 520), (4608, 4100, 40), (4100, 4104, 128)]


def _inputs(t, M, N, K, seed, integer):
    rng = np.random.default_rng(seed)
    return (inputs.random_codes(rng, t, (M, K), integer=integer),
            inputs.random_codes(rng, t, (N, K), integer=integer))


def _sampled_check(t, A, B, Dg, integer, seed):
    M, N = Dg.shape
    rand, forced = inputs.sample_indices(M, N, seed)
    idx = np.concatenate([rand, forced])
    Dr, S = oracle.gemm_ref(t, A, B, idx=idx)
    got = Dg.ravel()[idx]
    if integer:
        assert np.array_equal(got, Dr)
    else:
        rep = check.report(got, Dr, S)
        assert rep["fail"] == 0, rep


@pytest.mark.parametrize("t", ["bf16", "fp16"])
@pytest.mark.parametrize("case", CASES, ids=["%dx%dx%d" % c for c in CASES])
@pytest.mark.parametrize("integer", [True, False])
def test_persistent_grid(t, case, integer, monkeypatch):
    M, N, K = case
    A, B = _inputs(t, M, N, K, M + N + K + integer, integer)
    dA, dB = dev16(A, t), dev16(B, t)
    say("f16 persistent %s %dx%dx%d integer=%s" % (t, M, N, K, integer))
    D = run16(t, dA, dB)
    D16 = run16(t, dA, dB, out="bf16")
    monkeypatch.setenv("TILEGEMM_F16_CONFIG", "5")         # one workgroup per tile
    D1 = run16(t, dA, dB)
    D161 = run16(t, dA, dB, out="bf16")
    torch.cuda.synchronize()
    assert torch.equal(D, D1)
    assert torch.equal(D16, D161)
    assert np.array_equal(bf16_bits(D16), oracle.rne_bf16_f32(D.cpu().numpy()))
    _sampled_check(t, A, B, to_f64(D), integer, M + N)


def test_padded_d_rows_untouched():
    M, N, K, pad = 4200, 4300, 512, 68
    A, B = _inputs("bf16", M, N, K, 11, True)
    Dbig = torch.full((M, N + pad), float("nan"), dtype=torch.float32, device=DEV)
    D = Dbig[:, :N]
    say("f16 persistent padded D")
    run16("bf16", dev16(A, "bf16"), dev16(B, "bf16"), D=D)
    torch.cuda.synchronize()
    assert bool(torch.isnan(Dbig[:, N:]).all())
    _sampled_check("bf16", A, B, to_f64(D), True, 5)


def test_calls_in_a_row_of_different_grids():
    for (M, N, K) in [(8192, 4352, 512), (4200, 4300, 64), (4608, 4096, 1024)]:
        A, B = _inputs("bf16", M, N, K, M + 2 * N, True)
        say("f16 persistent in a row %dx%dx%d" % (M, N, K))
        D = run16("bf16", dev16(A, "bf16"), dev16(B, "bf16"))
        torch.cuda.synchronize()
        _sampled_check("bf16", A, B, to_f64(D), True, M)
