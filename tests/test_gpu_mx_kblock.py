"""Parity of the block-scaled forms with scale blocks wider than 32 K
(gemm_mx_kblock) against the oracle on an MI355X.

a(m,k) = x(A, m, k) * 2^(SFA[m, k / kb] - 127), b(k,n) likewise with SFB, for
e4m3, e2m1, e2m3 and e3m2 elements.  Bar: bit-exact on integer-valued inputs;
otherwise |D - D_ref| <= 2^-12 * sum|a*b| + 1e-6; and the 32-wide call on
the replicated scales equals the wide call (exact on integers).  The
workspace path (scales replicated on the GPU, then the format's tiled
kernels) is held to the same bar and, on integer inputs, equals the general
kernel's D.
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

FORMATS = ["e4m3", "e2m1", "e2m3", "e3m2"]


def _int_exponents(fmt):
    """Scale exponents that make every product an integer (partial sums stay
    below 2^24 at these sizes)."""
    if fmt == "e4m3":
        return 0, 3
    if fmt == "e2m1":
        return 1, 3
    e = inputs.fp6_integer_scale(fmt)
    return e, e + 1


def _case(fmt, M, N, K, kb, seed, integer, with_c=True):
    rng = np.random.default_rng(seed)
    A = inputs.random_codes(rng, fmt, (M, K), integer=integer)
    B = inputs.random_codes(rng, fmt, (N, K), integer=integer)
    nsc = -(-K // kb)
    lo, hi = _int_exponents(fmt) if integer else (-4, 5)
    SFA = (127 + rng.integers(lo, hi, size=(M, nsc))).astype(np.uint8)
    SFB = (127 + rng.integers(lo, hi, size=(N, nsc))).astype(np.uint8)
    C = None
    if with_c:
        C = (rng.integers(-4, 5, size=(M, N)) if integer else rng.uniform(-1, 1, size=(M, N))).astype(np.float32)
    return {"A": A, "B": B, "SFA": SFA, "SFB": SFB}, C


def _run(fmt, x, kb, C=None, out=torch.float32):
    Cd = torch.from_numpy(C).to(DEV) if C is not None else None
    return tg.gemm_mx_kblock(fmt, dev8(x["A"]), dev8(x["SFA"]), dev8(x["B"]), dev8(x["SFB"]), kb, Cd, out_dtype=out)


def _full_check(fmt, x, kb, Dg, integer, C=None):
    Dr, S = oracle.gemm_ref_full(fmt, x["A"], x["B"], C=C, SFA=x["SFA"], SFB=x["SFB"], kblock=kb)
    if integer:
        bad = np.argwhere(Dg != Dr)
        assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()
    else:
        rep = check.report(Dg, Dr, S)
        assert rep["fail"] == 0, rep


# (M, N, K, kb): several 64 x 64 tiles with ragged edges; a last block
# shorter than kb (K = 96, kb = 64); one scale per row (kb >= K, K not a
# power of two); a long K with 512-wide blocks
CASES = [(300, 260, 384, 64), (129, 70, 1024, 128), (65, 130, 96, 64), (200, 100, 96, 96),
         (100, 300, 384, 4096), (64, 64, 4096, 512)]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("case", CASES, ids=["%dx%dx%d_kb%d" % c for c in CASES])
def test_wide_blocks(fmt, case):
    M, N, K, kb = case
    for integer in (True, False):
        x, C = _case(fmt, M, N, K, kb, seed=M + N + K + kb, integer=integer)
        say("mx kblock %s %dx%dx%d kb %d integer=%s" % (fmt, M, N, K, kb, integer))
        D = _run(fmt, x, kb, C)
        torch.cuda.synchronize()
        _full_check(fmt, x, kb, to_f64(D), integer, C)


@pytest.mark.parametrize("fmt", FORMATS)
def test_equals_standard_call_on_replicated_scales(fmt):
    """kb = 128 against the 32-wide call on each scale repeated four times
    (a different kernel for the standard form): equal on integer inputs."""
    M, N, K, kb = 260, 300, 1024, 128
    x, C = _case(fmt, M, N, K, kb, seed=7, integer=True)
    rep = np.arange(K // 32) // (kb // 32)
    x32 = dict(x, SFA=np.ascontiguousarray(x["SFA"][:, rep]), SFB=np.ascontiguousarray(x["SFB"][:, rep]))
    say("mx kblock %s against the standard call" % fmt)
    Dw = _run(fmt, x, kb, C)
    Ds = _run(fmt, x32, 32, C)
    torch.cuda.synchronize()
    assert torch.equal(Dw, Ds)


def test_kb32_is_the_standard_call_and_bf16_out():
    M, N, K = 300, 260, 512
    x, C = _case("e4m3", M, N, K, 32, seed=3, integer=False, with_c=False)
    say("mx kblock 32 and bf16 out")
    D1 = _run("e4m3", x, 32)
    D2 = tg.gemm_mxfp8(dev8(x["A"]), dev8(x["SFA"]), dev8(x["B"]), dev8(x["SFB"]))
    x, _ = _case("e2m1", M, N, K, 64, seed=4, integer=False, with_c=False)
    D32 = _run("e2m1", x, 64)
    D16 = _run("e2m1", x, 64, out=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(D1, D2)
    assert np.array_equal(bf16_bits(D16), oracle.rne_bf16_f32(D32.cpu().numpy()))


def test_unsupported_widths_raise():
    x, _ = _case("e4m3", 64, 64, 256, 32, seed=5, integer=True, with_c=False)
    with pytest.raises(tg.GemmError):
        _run("e4m3", dict(x, SFA=x["SFA"][:, :3], SFB=x["SFB"][:, :3]), 96)


# The workspace path (gemm_mx_kblock_ws): scales replicated to 32-wide blocks,
# then the format's tiled kernels.  K % 512 == 0 (the four-wave kernels),
# K % 128 only (fp8's smaller kernels, fp6's tiled path, fp4's general
# kernel), a short last block, one scale per row.
WS_CASES = [(300, 260, 512, 64), (600, 520, 1024, 128), (129, 70, 1024, 1024), (200, 100, 512, 4096),
            (257, 300, 384, 128), (300, 300, 2048, 512), (64, 96, 96, 64)]


def _run_ws(fmt, x, kb, C=None, out=torch.float32):
    M, N = x["A"].shape[0], x["B"].shape[0]
    ws = torch.empty(tg.mx_kblock_workspace_bytes(M, N, _k_of(fmt, x)) + 256, dtype=torch.uint8, device=DEV)
    ws = ws[(-ws.data_ptr()) % 256:]
    Cd = torch.from_numpy(C).to(DEV) if C is not None else None
    return tg.gemm_mx_kblock(fmt, dev8(x["A"]), dev8(x["SFA"]), dev8(x["B"]), dev8(x["SFB"]), kb, Cd, out_dtype=out,
                             workspace=ws)


def _k_of(fmt, x):
    cols = x["A"].shape[1]
    return {"e4m3": cols, "e2m1": 2 * cols}.get(fmt, cols // 3 * 4)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("case", WS_CASES, ids=["%dx%dx%d_kb%d" % c for c in WS_CASES])
def test_workspace_path(fmt, case):
    M, N, K, kb = case
    for integer in (True, False):
        x, C = _case(fmt, M, N, K, kb, seed=3 * M + N + K + kb, integer=integer)
        say("mx kblock ws %s %dx%dx%d kb %d integer=%s" % (fmt, M, N, K, kb, integer))
        Dw = _run_ws(fmt, x, kb, C)
        Dg = _run(fmt, x, kb, C)
        torch.cuda.synchronize()
        _full_check(fmt, x, kb, to_f64(Dw), integer, C)
        if integer:
            assert torch.equal(Dw, Dg)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_workspace_path_persistent_grid(fmt):
    """More 256 x 256 tiles than CUs, no C, kb = 128: the persistent
    four-wave kernel on replicated scales; exact on integer inputs at the
    sampled elements, bf16 out the RNE of fp32 out."""
    M, N, K, kb = 4200, 4300, 1024, 128
    x, _ = _case(fmt, M, N, K, kb, seed=17, integer=True, with_c=False)
    say("mx kblock ws %s persistent grid" % fmt)
    D = _run_ws(fmt, x, kb)
    D16 = _run_ws(fmt, x, kb, out=torch.bfloat16)
    torch.cuda.synchronize()
    rand, forced = inputs.sample_indices(M, N, 23)
    idx = np.concatenate([rand, forced])
    Dr, _ = oracle.gemm_ref(fmt, x["A"], x["B"], idx=idx, SFA=x["SFA"], SFB=x["SFB"], kblock=kb)
    assert np.array_equal(to_f64(D).ravel()[idx], Dr)
    assert np.array_equal(bf16_bits(D16), oracle.rne_bf16_f32(D.cpu().numpy()))


def test_workspace_too_small_raises():
    x, _ = _case("e4m3", 64, 64, 512, 64, seed=5, integer=True, with_c=False)
    ws = torch.empty(tg.mx_kblock_workspace_bytes(64, 64, 512) - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(tg.GemmError):
        tg.gemm_mx_kblock("e4m3", dev8(x["A"]), dev8(x["SFA"]), dev8(x["B"]), dev8(x["SFB"]), 64, workspace=ws)
