"""Parity of the block-scaled split-K calls (gemm_mxfp8_splitk,
gemm_mxfp4_splitk, gemm_mxfp6_splitk) against the oracle on an MI355X.

K is cut into ranges of whole 512-K groups whose fp32 partial products are
summed in order by a second kernel; the bar is the unsplit calls': bit-exact
on integer-valued inputs, otherwise |D - D_ref| <= 2^-12 * sum|a*b| + 1e-6,
and bf16 output equal to RNE of the fp32 result.
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

TYPES = ["e4m3", "e2m1", "e2m3", "e3m2"]


def _scale_range(t, integer):
    """Scale exponents: integer variants keep every product an integer and
    every partial sum below 2^24 at the K used here."""
    if not integer:
        return -4, 5
    if t == "e4m3":
        return 0, 2
    if t == "e2m1":
        return 1, 3
    e = inputs.fp6_integer_scale(t)
    return e, e + 1


def _case(t, M, N, K, seed, integer, with_c=True):
    rng = np.random.default_rng(seed)
    A = inputs.random_codes(rng, t, (M, K), integer=integer)
    B = inputs.random_codes(rng, t, (N, K), integer=integer)
    lo, hi = _scale_range(t, integer)
    SFA = (127 + rng.integers(lo, hi, size=(M, K // 32))).astype(np.uint8)
    SFB = (127 + rng.integers(lo, hi, size=(N, K // 32))).astype(np.uint8)
    C = None
    if with_c:
        C = (rng.integers(-4, 5, size=(M, N)) if integer else rng.uniform(-1, 1, size=(M, N))).astype(np.float32)
    return {"A": A, "B": B, "SFA": SFA, "SFB": SFB}, C


def _run(t, x, C=None, out=torch.float32, splits=0, workspace=None, D=None, split=True):
    Cd = torch.from_numpy(C).to(DEV) if C is not None else None
    if Cd is not None and out == torch.bfloat16:
        Cd = Cd.to(torch.bfloat16)
    args = (dev8(x["A"]), dev8(x["SFA"]), dev8(x["B"]), dev8(x["SFB"]), Cd)
    kw = {"out_dtype": out, "D": D}
    if split:
        kw.update(splits=splits, workspace=workspace)
    if t == "e4m3":
        return (tg.gemm_mxfp8_splitk if split else tg.gemm_mxfp8)(*args, **kw)
    if t == "e2m1":
        return (tg.gemm_mxfp4_splitk if split else tg.gemm_mxfp4)(*args, **kw)
    return (tg.gemm_mxfp6_splitk if split else tg.gemm_mxfp6)(*args, fmt=t, **kw)


def _check(t, x, Dg, integer, C=None):
    Dr, S = oracle.gemm_ref_full(t, x["A"], x["B"], C=C, SFA=x["SFA"], SFB=x["SFB"])
    if integer:
        bad = np.argwhere(Dg != Dr)
        assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()
    else:
        rep = check.report(Dg, Dr, S)
        assert rep["fail"] == 0, rep


# (M, N, K, splits): whole and ragged tiles, one 512-K group per split,
# uneven last ranges, requests above the number of 512-K groups (clamped)
CASES = [(256, 256, 2048, 2), (256, 256, 2048, 3), (300, 200, 4096, 4), (64, 64, 4096, 8), (1, 1, 1024, 2),
         (513, 300, 3072, 6), (100, 70, 1536, 16), (257, 129, 2560, 5)]


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("case", CASES)
def test_explicit_splits(t, case):
    M, N, K, splits = case
    for integer in (True, False):
        x, C = _case(t, M, N, K, seed=M + 7 * N + K + splits + len(t), integer=integer, with_c=M > 1 or not integer)
        say("mx splitk %s %dx%dx%d splits=%d integer=%s" % (t, M, N, K, splits, integer))
        D = _run(t, x, C, splits=splits)
        torch.cuda.synchronize()
        _check(t, x, to_f64(D), integer, C)


@pytest.mark.parametrize("t", TYPES)
def test_auto_split_small_grid(t):
    """Four output tiles and K = 16384: the library's choice splits K in four."""
    M, N, K = 512, 512, 16384
    assert tg.splitk_workspace_bytes(M, N, K, 0) == 4 * M * N * 4
    x, C = _case(t, M, N, K, seed=21, integer=False)
    say("mx splitk %s auto %dx%dx%d" % (t, M, N, K))
    D = _run(t, x, C)
    torch.cuda.synchronize()
    _check(t, x, to_f64(D), False, C)


@pytest.mark.parametrize("t", ["e4m3", "e2m1", "e2m3"])
def test_deterministic_and_equal_to_unsplit_on_integers(t):
    x, C = _case(t, 384, 320, 4096, seed=3, integer=False)
    d1 = _run(t, x, C, splits=8)
    d2 = _run(t, x, C, splits=8)
    torch.cuda.synchronize()
    assert torch.equal(d1, d2)                        # partials summed in range order
    xi, Ci = _case(t, 384, 320, 4096, seed=4, integer=True)
    s = _run(t, xi, Ci, splits=8)
    u = _run(t, xi, Ci, split=False)
    torch.cuda.synchronize()
    assert torch.equal(s, u)


@pytest.mark.parametrize("t", TYPES)
def test_bf16_output_is_rne_of_fp32(t):
    x, _ = _case(t, 300, 264, 3072, seed=5, integer=False, with_c=False)
    D32 = _run(t, x, splits=3)
    D16 = _run(t, x, splits=3, out=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(D16), oracle.rne_bf16_f32(D32.cpu().numpy()))


def test_bf16_c_and_output():
    x, C = _case("e4m3", 200, 300, 4096, seed=8, integer=True)
    D = _run("e4m3", x, C, splits=4, out=torch.bfloat16)
    torch.cuda.synchronize()
    Dr, _ = oracle.gemm_ref_full("e4m3", x["A"], x["B"], C=C, SFA=x["SFA"], SFB=x["SFB"])
    assert np.array_equal(bf16_bits(D), oracle.rne_bf16_f32(Dr.astype(np.float32)))


@pytest.mark.parametrize("t", ["e2m1", "e3m2"])
def test_in_place_c(t):
    x, C = _case(t, 260, 300, 4096, seed=9, integer=True)
    D = torch.from_numpy(C).to(DEV)
    args = (dev8(x["A"]), dev8(x["SFA"]), dev8(x["B"]), dev8(x["SFB"]), D)
    if t == "e2m1":
        tg.gemm_mxfp4_splitk(*args, D=D, splits=4)
    else:
        tg.gemm_mxfp6_splitk(*args, D=D, splits=4, fmt=t)
    torch.cuda.synchronize()
    _check(t, x, to_f64(D), True, C)


def test_workspace_reused_and_too_small():
    M, N, K = 300, 300, 6144
    ws = torch.empty(tg.splitk_workspace_bytes(M, N, K, 6) + 4096, dtype=torch.uint8, device=DEV)
    ws.fill_(0xFF)                                    # NaN patterns: the contents need no initialisation
    for t in TYPES:
        x, C = _case(t, M, N, K, seed=len(t), integer=True)
        D = _run(t, x, C, splits=6, workspace=ws)
        torch.cuda.synchronize()
        _check(t, x, to_f64(D), True, C)
    small = torch.empty(M * N * 4, dtype=torch.uint8, device=DEV)
    for t in TYPES:
        x, _ = _case(t, M, N, K, seed=1, integer=True, with_c=False)
        with pytest.raises(tg.GemmError) as ei:
            _run(t, x, splits=6, workspace=small)
        assert ei.value.status == 7


def test_outside_the_fast_path():
    """K % 512 != 0 has no tiled split kernel: the call runs unsplit (and
    needs no workspace), fp8 on its other kernels, fp4 and fp6 on the
    general one."""
    M, N, K = 200, 136, 640
    x, C = _case("e4m3", M, N, K, seed=2, integer=True)
    D = torch.empty((M, N), dtype=torch.float32, device=DEV)
    Cd = torch.from_numpy(C).to(DEV)
    tensors = [dev8(x[k]) for k in ("A", "SFA", "B", "SFB")]  # held: the call takes raw pointers
    st = tg.raw.gemm_mxfp8_splitk(M, N, K, tensors[0].data_ptr(), K, tensors[1].data_ptr(), K // 32,
                                  tensors[2].data_ptr(), K, tensors[3].data_ptr(), K // 32, Cd.data_ptr(), N,
                                  D.data_ptr(), N, 0, 4, None, 0, None)
    torch.cuda.synchronize()
    assert st == 0
    _check("e4m3", x, to_f64(D), True, C)
    for t in ("e2m1", "e2m3"):
        xt, _ = _case(t, 64, 64, 768, seed=1, integer=True, with_c=False)
        D = _run(t, xt, splits=2)
        torch.cuda.synchronize()
        _check(t, xt, to_f64(D), True)


def _big(integer):
    w = inputs.WORKLOADS["largek_mxfp8"]
    x = inputs.generate(w, integer=integer)
    say("mx splitk %s integer=%s splits=auto" % (w.name, integer))
    D = _run("e4m3", x)
    torch.cuda.synchronize()
    Dg = D.cpu().numpy()
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


def test_largek_mxfp8():
    _big(False)


def test_largek_mxfp8_integer():
    _big(True)
