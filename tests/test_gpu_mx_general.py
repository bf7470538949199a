"""Parity of the general block-scaled kernel against the oracle on an MI355X:
the calls the tiled kernels do not take -- K a multiple of 32 but not of
128 (fp8) or 512 (fp4, fp6), operand rows not 16-byte (or not even 4-byte)
aligned, scale rows at any alignment -- through gemm_mxfp8, gemm_mxfp4 and
gemm_mxfp6.  Bar: bit-exact on integer-valued inputs, otherwise
|D - D_ref| <= 2^-12 * sum|a*b| + 1e-6, bf16 output equal to RNE of fp32.
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
    from gpuutil import DEV, bf16_bits, say, to_f64

TYPES = ["e4m3", "e2m1", "e2m3", "e3m2"]


def _case(t, M, N, K, seed, integer, with_c=True):
    rng = np.random.default_rng(seed)
    A = inputs.random_codes(rng, t, (M, K), integer=integer)
    B = inputs.random_codes(rng, t, (N, K), integer=integer)
    # scale exponents [lo, hi): integer variants keep every product an integer
    if not integer:
        lo, hi = -4, 5
    elif t == "e4m3":
        lo, hi = 0, 2
    elif t == "e2m1":
        lo, hi = 1, 3
    else:
        lo = inputs.fp6_integer_scale(t)
        hi = lo + 1
    SFA = (127 + rng.integers(lo, hi, size=(M, K // 32))).astype(np.uint8)
    SFB = (127 + rng.integers(lo, hi, size=(N, K // 32))).astype(np.uint8)
    C = None
    if with_c:
        C = (rng.integers(-4, 5, size=(M, N)) if integer else rng.uniform(-1, 1, size=(M, N))).astype(np.float32)
    return {"A": A, "B": B, "SFA": SFA, "SFB": SFB}, C


def _dev(rows, pad=0, offset=0, fill=0xFF):
    """Device copy of a (R, W) byte array as a (R, W) view whose rows are W +
    pad bytes apart and whose first byte lies `offset` bytes into its
    allocation; the padding holds `fill` (must never be read)."""
    R, W = rows.shape
    buf = torch.full((offset + R * (W + pad) + 16,), fill, dtype=torch.uint8, device=DEV)
    view = buf[offset:offset + R * (W + pad)].view(R, W + pad)
    view[:, :W] = torch.from_numpy(np.ascontiguousarray(rows)).to(DEV)
    return view[:, :W], buf


def _call(t, A, SFA, B, SFB, C=None, out=torch.float32, D=None):
    if t == "e4m3":
        return tg.gemm_mxfp8(A, SFA, B, SFB, C, out_dtype=out, D=D)
    if t == "e2m1":
        return tg.gemm_mxfp4(A, SFA, B, SFB, C, out_dtype=out, D=D)
    return tg.gemm_mxfp6(A, SFA, B, SFB, C, out_dtype=out, D=D, fmt=t)


def _check(t, x, Dg, integer, C=None):
    Dr, S = oracle.gemm_ref_full(t, x["A"], x["B"], C=C, SFA=x["SFA"], SFB=x["SFB"])
    if integer:
        bad = np.argwhere(Dg != Dr)
        assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()
    else:
        rep = check.report(Dg, Dr, S)
        assert rep["fail"] == 0, rep


def _run(t, x, C=None, out=torch.float32, pad=0, offset=0, spad=0, soffset=0):
    A, _a = _dev(x["A"], pad, offset)                 # the buffers stay held until the call has run
    B, _b = _dev(x["B"], pad, offset)
    SFA, _sa = _dev(x["SFA"], spad, soffset)
    SFB, _sb = _dev(x["SFB"], spad, soffset)
    Cd = torch.from_numpy(C).to(DEV) if C is not None else None
    if Cd is not None and out == torch.bfloat16:
        Cd = Cd.to(torch.bfloat16)
    D = _call(t, A, SFA, B, SFB, Cd, out=out)
    torch.cuda.synchronize()
    return D


# K multiples of 32 off the tiled kernels' steps; ragged M and N
SHAPES = [(64, 64, 32), (100, 70, 96), (65, 129, 160), (1, 1, 32), (200, 136, 544), (130, 257, 1056),
          (77, 50, 2080)]


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("shape", SHAPES)
def test_any_k(t, shape):
    M, N, K = shape
    for integer in (True, False):
        x, C = _case(t, M, N, K, seed=M + 5 * N + K + len(t), integer=integer)
        say("mx general %s %dx%dx%d integer=%s" % (t, M, N, K, integer))
        D = _run(t, x, C)
        _check(t, x, to_f64(D), integer, C)


# (row padding in bytes, start offset): rows 4-byte aligned but not 16, and
# not even 4-byte aligned (fp6 row strides must stay multiples of 3 bytes)
LAYOUTS = {"e4m3": [(4, 0), (1, 1), (3, 2)], "e2m1": [(4, 4), (1, 3), (2, 1)],
           "e2m3": [(12, 4), (3, 1), (6, 2)], "e3m2": [(12, 8), (3, 3), (9, 1)]}


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("which", [0, 1, 2])
def test_unaligned_rows_and_scales(t, which):
    pad, offset = LAYOUTS[t][which]
    for K in (512, 1056):                             # a tiled-kernel K and an odd one
        for integer in (True, False):
            x, C = _case(t, 150, 90, K, seed=K + which + len(t), integer=integer)
            say("mx general %s K=%d row pad %d offset %d integer=%s" % (t, K, pad, offset, integer))
            D = _run(t, x, C, pad=pad, offset=offset, spad=which + 1, soffset=which)
            _check(t, x, to_f64(D), integer, C)


@pytest.mark.parametrize("t", TYPES)
def test_bf16_output_and_c(t):
    x, C = _case(t, 96, 80, 1056, seed=4, integer=True)
    D = _run(t, x, C, out=torch.bfloat16)
    Dr, _ = oracle.gemm_ref_full(t, x["A"], x["B"], C=C, SFA=x["SFA"], SFB=x["SFB"])
    assert np.array_equal(bf16_bits(D), oracle.rne_bf16_f32(Dr.astype(np.float32)))
    x, _ = _case(t, 96, 80, 1056, seed=5, integer=False, with_c=False)
    D32 = _run(t, x)
    D16 = _run(t, x, out=torch.bfloat16)
    assert np.array_equal(bf16_bits(D16), oracle.rne_bf16_f32(D32.cpu().numpy()))


def test_same_as_tiled_kernel_on_integers():
    """The general kernel (scales at an odd offset) and the tiled kernel
    (aligned copies) give the same bits on integer data."""
    for t in TYPES:
        x, C = _case(t, 300, 260, 1024, seed=7, integer=True)
        g = _run(t, x, C, soffset=1, spad=1)
        f = _run(t, x, C)
        assert torch.equal(g, f), t


# K off the 512 step with operand rows 16-byte multiples and scale rows
# padded to 16 bytes with NaN codes (0xFF) past each row's last block, which
# no kernel may apply: fp6 with K % 128 == 0 and fp8 with K % 128 == 0 run
# tiled kernels (fp6 the four-wave one, clearing the last scale group's
# bytes past K), the other K the general kernel
TAIL_K = {"e4m3": [32, 160, 640, 1056, 4128], "e2m1": [32, 96, 544, 1056, 4128],
          "e2m3": [128, 640, 1152], "e3m2": [128, 640, 1152]}


@pytest.mark.parametrize("t", TYPES)
def test_k_tails_with_padded_scales(t):
    for K in TAIL_K[t]:
        for M, N in ((300, 264), (64, 64)):
            for integer in (True, False):
                x, C = _case(t, M, N, K, seed=K + M + len(t), integer=integer)
                spad = (-(K // 32)) % 16
                say("mx tiled tail %s %dx%dx%d integer=%s" % (t, M, N, K, integer))
                D = _run(t, x, C, spad=spad)
                _check(t, x, to_f64(D), integer, C)


@pytest.mark.parametrize("t", ["e4m3", "e2m1", "e2m3"])
def test_k_tail_split(t):
    """Split-K with K off the 512 step: fp6 splits on the four-wave kernel
    (the last range holds the partial scale group), fp8 and fp4 run unsplit."""
    M, N, K = 256, 192, 4224
    x, C = _case(t, M, N, K, seed=3, integer=True)
    spad = (-(K // 32)) % 16
    A, _a = _dev(x["A"], 0, 0)
    B, _b = _dev(x["B"], 0, 0)
    SFA, _sa = _dev(x["SFA"], spad, 0)
    SFB, _sb = _dev(x["SFB"], spad, 0)
    Cd = torch.from_numpy(C).to(DEV)
    if t == "e4m3":
        D = tg.gemm_mxfp8_splitk(A, SFA, B, SFB, Cd, splits=5)
    elif t == "e2m1":
        D = tg.gemm_mxfp4_splitk(A, SFA, B, SFB, Cd, splits=5)
    else:
        D = tg.gemm_mxfp6_splitk(A, SFA, B, SFB, Cd, splits=5, fmt=t)
    torch.cuda.synchronize()
    _check(t, x, to_f64(D), True, C)
