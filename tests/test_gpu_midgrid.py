"""Grids at the library's kernel-choice boundaries: 128 to 239 output tiles
of 256 x 256 (part of one wave), which go to the four-wave kernels (with
256 x 256 or 192 x 256 tiles, whichever needs fewer waves of work), and
grids of up to one 128 x 128 (or 64 x 64) tile per CU, which go to the
deep-ring kernels.  Exact on integer-valued inputs against the oracle at 4096
seeded samples plus the tile edges, and within the tolerance on random
inputs."""
import numpy as np
import pytest
import torch

import oracle
from oracle import check
import tiled_dense_gemm_tile_amd as tg
from tiled_dense_gemm_tile_amd import inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpuutil import DEV, dev8, dev16, say, to_f64

# (in_type, M, N, K): 144 tiles with ragged edges and 16-byte rows; 8-byte
# rows (K = 516); fp8 at 132 tiles; 16-bit at exactly 128 tiles; 256 and 240
# tiles of 128 x 128 with ragged edges and K
# 192 x 256 tiles where they need fewer or cheaper waves than 256 x 256
# ones: 4000 x 3000 is 192 tiles of 256^2 and 252 of 192 x 256 (16-byte and
# 8-byte rows); 4096 x 3000 stays on 256^2 tiles (264 of 192 x 256 would be
# two waves)
CASES = [("bf16", 2900, 3000, 520), ("fp16", 3000, 3000, 516), ("e4m3", 2600, 3000, 1024), ("bf16", 2048, 4096, 256),
         ("bf16", 2000, 2000, 1000), ("fp16", 1900, 2000, 4104),
         ("e4m3", 2000, 1900, 2048), ("e4m3", 1000, 1000, 4096),
         ("bf16", 4000, 3000, 1000), ("fp16", 4000, 3000, 1036), ("bf16", 4096, 3000, 512)]


@pytest.mark.parametrize("case", CASES, ids=["%s_%dx%dx%d" % c for c in CASES])
@pytest.mark.parametrize("integer", [True, False])
def test_partial_wave_grid(case, integer):
    t, M, N, K = case
    rng = np.random.default_rng(M + N + K + integer)
    A = inputs.random_codes(rng, t, (M, K), integer=integer)
    B = inputs.random_codes(rng, t, (N, K), integer=integer)
    C = (rng.integers(-4, 5, size=(M, N)) if integer else rng.uniform(-1, 1, size=(M, N))).astype(np.float32)
    Cd = torch.from_numpy(C).to(DEV)
    say("partial-wave grid %s %dx%dx%d integer=%s" % (t, M, N, K, integer))
    kw = {}
    if t == "e4m3":
        lo, hi = (0, 2) if integer else (-4, 5)
        SFA = (127 + rng.integers(lo, hi, size=(M, K // 32))).astype(np.uint8)
        SFB = (127 + rng.integers(lo, hi, size=(N, K // 32))).astype(np.uint8)
        D = tg.gemm_mxfp8(dev8(A), dev8(SFA), dev8(B), dev8(SFB), Cd)
        kw = {"SFA": SFA, "SFB": SFB}
    else:
        fn = tg.gemm_bf16 if t == "bf16" else tg.gemm_fp16
        D = fn(dev16(A, t), dev16(B, t), Cd)
    torch.cuda.synchronize()
    rand, forced = inputs.sample_indices(M, N, M + N)
    idx = np.concatenate([rand, forced])
    Dg = to_f64(D).ravel()[idx]
    Dr, S = oracle.gemm_ref(t, A, B, C=C, idx=idx, **kw)
    if integer:
        assert np.array_equal(Dg, Dr)
    else:
        rep = check.report(Dg, Dr, S)
        assert rep["fail"] == 0, rep
