"""Parity of the split-K path (gemm_bf16_splitk / gemm_fp16_splitk) against
the oracle on an MI355X.

K is cut into ranges whose fp32 partial products are summed by a second
kernel; the bar is the same as for the unsplit calls: bit-exact on
integer-valued inputs, otherwise |D - D_ref| <= 2^-12 * sum|a*b| + 1e-6, and
bf16 output equal to RNE of the fp32 result.
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
    from gpuutil import DEV, bf16_bits, dev16, say, to_f64


def _case(in_type, M, N, K, seed, integer, with_c):
    rng = np.random.default_rng(seed)
    A = inputs.random_codes(rng, in_type, (M, K), integer=integer)
    B = inputs.random_codes(rng, in_type, (N, K), integer=integer)
    C = None
    if with_c:
        C = (rng.integers(-4, 5, size=(M, N)) if integer else rng.uniform(-1, 1, size=(M, N))).astype(np.float32)
    return A, B, C


def _split(in_type, A, B, C=None, splits=0, out=torch.float32, workspace=None, D=None):
    fn = tg.gemm_bf16_splitk if in_type == "bf16" else tg.gemm_fp16_splitk
    Cd = torch.from_numpy(C).to(DEV) if C is not None else None
    if Cd is not None and out == torch.bfloat16:
        Cd = Cd.to(torch.bfloat16)
    return fn(dev16(A, in_type), dev16(B, in_type), Cd, out_dtype=out, splits=splits, workspace=workspace, D=D)


def _check(in_type, A, B, C, Dg, integer):
    Dr, S = oracle.gemm_ref_full(in_type, A, B, C=C)
    if integer:
        bad = np.argwhere(Dg != Dr)
        assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()
    else:
        rep = check.report(Dg, Dr, S)
        assert rep["fail"] == 0, rep


# (M, N, K, splits): whole and ragged tiles, K a multiple of 64 or not, rows
# 16-byte aligned (K % 8 == 0) or only 8-byte aligned (K % 8 == 4), more
# splits than tiles, one 64-wide K tile per split, requests above the K tile
# count (clamped)
CASES = [(256, 256, 4096, 2), (256, 256, 4096, 3), (300, 200, 5000, 3), (64, 64, 8192, 7), (100, 70, 1024, 16),
         (1, 1, 4096, 4), (257, 129, 2052, 5), (513, 300, 4100, 4), (40, 1000, 640, 4), (96, 96, 320, 64)]


@pytest.mark.parametrize("in_type", ["bf16", "fp16"])
@pytest.mark.parametrize("case", CASES)
def test_explicit_splits(in_type, case):
    M, N, K, splits = case
    for integer in (True, False):
        A, B, C = _case(in_type, M, N, K, seed=M + 7 * N + K + splits, integer=integer, with_c=not integer or M > 1)
        say("splitk %s %dx%dx%d splits=%d integer=%s" % (in_type, M, N, K, splits, integer))
        D = _split(in_type, A, B, C, splits=splits)
        torch.cuda.synchronize()
        _check(in_type, A, B, C, to_f64(D), integer)


@pytest.mark.parametrize("in_type", ["bf16", "fp16"])
def test_bf16_output_is_rne_of_fp32(in_type):
    A, B, C = _case(in_type, 300, 264, 3000, seed=5, integer=False, with_c=False)
    D32 = _split(in_type, A, B, splits=4)
    D16 = _split(in_type, A, B, splits=4, out=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(D16), oracle.rne_bf16_f32(D32.cpu().numpy()))


def test_bf16_c_and_output():
    """bf16 C (added to the fp32 sum of the partials) and bf16 D, integer data:
    the fp32 sum is exact, so D is its nearest-even bf16 bit for bit."""
    A, B, C = _case("bf16", 200, 300, 4096, seed=8, integer=True, with_c=True)
    D = _split("bf16", A, B, C, splits=4, out=torch.bfloat16)
    torch.cuda.synchronize()
    Dr, _ = oracle.gemm_ref_full("bf16", A, B, C=C)
    assert np.array_equal(bf16_bits(D), oracle.rne_bf16_f32(Dr.astype(np.float32)))


def test_deterministic_and_equal_to_unsplit_on_integers():
    A, B, C = _case("bf16", 512, 512, 8192, seed=3, integer=False, with_c=True)
    d1 = _split("bf16", A, B, C, splits=8)
    d2 = _split("bf16", A, B, C, splits=8)
    torch.cuda.synchronize()
    assert torch.equal(d1, d2)                        # the partials are summed in range order
    Ai, Bi, Ci = _case("bf16", 512, 512, 8192, seed=4, integer=True, with_c=True)
    s = _split("bf16", Ai, Bi, Ci, splits=8)
    u = _split("bf16", Ai, Bi, Ci, splits=1)          # the unsplit kernel
    torch.cuda.synchronize()
    assert torch.equal(s, u)


def test_in_place_c():
    A, B, C = _case("fp16", 260, 300, 4096, seed=9, integer=True, with_c=True)
    D = torch.from_numpy(C).to(DEV)
    tg.gemm_fp16_splitk(dev16(A, "fp16"), dev16(B, "fp16"), D, D=D, splits=4)
    torch.cuda.synchronize()
    _check("fp16", A, B, C, to_f64(D), True)


def test_workspace_reused_and_oversized():
    M, N, K = 300, 300, 6144
    ws = torch.empty(tg.splitk_workspace_bytes(M, N, K, 6) + 4096, dtype=torch.uint8, device=DEV)
    ws.fill_(0xFF)                                    # NaN patterns: the contents need no initialisation
    for seed in (1, 2):
        A, B, C = _case("bf16", M, N, K, seed=seed, integer=True, with_c=True)
        D = _split("bf16", A, B, C, splits=6, workspace=ws)
        torch.cuda.synchronize()
        _check("bf16", A, B, C, to_f64(D), True)


def test_too_small_workspace_is_refused():
    A, B, _ = _case("bf16", 256, 256, 4096, seed=1, integer=True, with_c=False)
    need = tg.splitk_workspace_bytes(256, 256, 4096, 4)
    ws = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(tg.GemmError) as ei:
        _split("bf16", A, B, splits=4, workspace=ws)
    assert ei.value.status == 7


def test_unaligned_rows_run_unsplit():
    """Rows only 2-byte aligned (odd K) have no four-wave kernel: the call runs
    unsplit and needs no workspace."""
    A, B, C = _case("bf16", 130, 70, 3001, seed=2, integer=True, with_c=True)
    D = torch.empty((130, 70), dtype=torch.float32, device=DEV)
    Cd = torch.from_numpy(C).to(DEV)
    Ad, Bd = dev16(A, "bf16"), dev16(B, "bf16")       # held: the call takes raw pointers
    st = tg.raw.gemm_bf16_splitk(130, 70, 3001, Ad.data_ptr(), 3001, Bd.data_ptr(), 3001,
                                 Cd.data_ptr(), 70, D.data_ptr(), 70, 0, 4, None, 0, None)
    torch.cuda.synchronize()
    assert st == 0
    _check("bf16", A, B, C, to_f64(D), True)


def _big(integer):
    w = inputs.WORKLOADS["largek_bf16"]
    x = inputs.generate(w, integer=integer)
    say("splitk %s integer=%s splits=auto" % (w.name, integer))
    D = _split("bf16", x["A"], x["B"])
    torch.cuda.synchronize()
    Dg = D.cpu().numpy()
    rand, forced = inputs.sample_indices(w.M, w.N, w.seed)
    a, b = oracle.operands_f64("bf16", x["A"], x["B"])
    for name, idx in (("random", rand), ("forced", forced)):
        Dr, S = oracle.gemm_ref("bf16", x["A"], x["B"], idx=idx)
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


def test_largek():
    _big(False)


def test_largek_integer():
    _big(True)
