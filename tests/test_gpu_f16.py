"""Parity of the HIP path (bf16 / fp16 inputs) against the oracle on an MI355X.

Bar: bit-exact on integer-valued inputs; otherwise
|D - D_ref| <= 2^-12 * sum_k |a*b| + 1e-6 per element (and D finite); bf16
output equals the nearest-even rounding of the same call's fp32 result.
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


def _full_check(in_type, x, Dg, integer, C=None):
    Dr, S = oracle.gemm_ref_full(in_type, x["A"], x["B"], C=C)
    if integer:
        bad = np.argwhere(Dg != Dr)
        assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()
    else:
        rep = check.report(Dg, Dr, S)
        assert rep["fail"] == 0, rep


def _case(in_type, M, N, K, seed, integer, with_c=True):
    rng = np.random.default_rng(seed)
    x = {"A": inputs.random_codes(rng, in_type, (M, K), integer=integer),
         "B": inputs.random_codes(rng, in_type, (N, K), integer=integer)}
    C = None
    if with_c:
        C = (rng.integers(-4, 5, size=(M, N)) if integer else rng.uniform(-1, 1, size=(M, N))).astype(np.float32)
    return x, C


# ---- the small workload, every element ------------------------------------------

@pytest.mark.parametrize("integer", [False, True])
def test_square256_every_element(integer):
    w = inputs.WORKLOADS["square256_bf16"]
    x = inputs.generate(w, integer=integer)
    say("square256 bf16 integer=%s" % integer)
    D = run16("bf16", dev16(x["A"], "bf16"), dev16(x["B"], "bf16"), torch.from_numpy(x["C"]).to(DEV))
    torch.cuda.synchronize()
    Dg = to_f64(D)
    Dr, S = oracle.gemm_ref("bf16", x["A"], x["B"], C=x["C"])   # naive loop, every element
    if integer:
        assert np.array_equal(Dg, Dr)
    else:
        rep = check.report(Dg, Dr, S)
        assert rep["fail"] == 0, rep


# ---- ragged shapes -------------------------------------------------------------------

RAGGED = [(1, 1, 1), (1, 17, 3), (7, 5, 9), (17, 13, 65), (63, 64, 65), (64, 64, 64), (65, 63, 127),
          (130, 70, 8), (255, 257, 256), (257, 255, 300), (129, 200, 4100), (300, 40, 1000),
          (70, 70, 1), (70, 70, 15), (70, 70, 16), (70, 70, 17), (70, 70, 63), (70, 70, 129)]


@pytest.mark.parametrize("in_type", ["bf16", "fp16"])
@pytest.mark.parametrize("shape", RAGGED)
def test_ragged(in_type, shape):
    M, N, K = shape
    for integer in (True, False):
        x, C = _case(in_type, M, N, K, seed=M * 7 + N * 3 + K, integer=integer)
        say("ragged %s %dx%dx%d integer=%s" % (in_type, M, N, K, integer))
        D = run16(in_type, dev16(x["A"], in_type), dev16(x["B"], in_type), torch.from_numpy(C).to(DEV))
        torch.cuda.synchronize()
        _full_check(in_type, x, to_f64(D), integer, C)


# ---- leading dimensions and misaligned bases -------------------------------------------

@pytest.mark.parametrize("pad_a,pad_b,off", [(0, 0, 0), (2, 0, 0), (4, 6, 0), (1, 3, 0), (0, 0, 1), (8, 8, 2),
                                             (6, 2, 4), (0, 1, 3)])
def test_leading_dims_and_offsets(pad_a, pad_b, off):
    M, N, K = 300, 260, 200
    in_type = "bf16"
    x, C = _case(in_type, M, N, K, seed=99 + pad_a + pad_b + off, integer=True)
    lda, ldb = K + pad_a, K + pad_b
    rng = np.random.default_rng(1)
    Abuf = inputs.random_codes(rng, in_type, (M * lda + off,), integer=True)
    Bbuf = inputs.random_codes(rng, in_type, (N * ldb + off,), integer=True)
    Abuf[off:].reshape(M, lda)[:, :K] = x["A"]
    Bbuf[off:].reshape(N, ldb)[:, :K] = x["B"]
    Ad = dev16(Abuf, in_type)[off:].view(M, lda)[:, :K]
    Bd = dev16(Bbuf, in_type)[off:].view(N, ldb)[:, :K]
    say("ld lda=%d ldb=%d off=%d" % (lda, ldb, off))
    D = run16(in_type, Ad, Bd, torch.from_numpy(C).to(DEV))
    torch.cuda.synchronize()
    _full_check(in_type, x, to_f64(D), True, C)


# ---- C handling, in-place, K = 0, empty outputs, canaries --------------------------------

def test_c_null_equals_zero_buffer_and_in_place():
    M, N, K = 333, 280, 190
    x, C = _case("bf16", M, N, K, seed=5, integer=False)
    A, B = dev16(x["A"], "bf16"), dev16(x["B"], "bf16")
    say("C null / zero / in-place")
    D0 = run16("bf16", A, B, None)
    Dz = run16("bf16", A, B, torch.zeros(M, N, device=DEV))
    Cd = torch.from_numpy(C).to(DEV)
    Dc = run16("bf16", A, B, Cd)
    inplace = Cd.clone()
    run16("bf16", A, B, inplace, D=inplace)
    torch.cuda.synchronize()
    assert torch.equal(D0, Dz)
    assert torch.equal(Dc, inplace)
    _full_check("bf16", x, to_f64(Dc), False, C)


def test_k_zero_gives_c():
    M, N = 100, 77
    C = torch.randn(M, N, device=DEV)
    A = torch.empty(M, 0, dtype=torch.bfloat16, device=DEV)
    B = torch.empty(N, 0, dtype=torch.bfloat16, device=DEV)
    say("K=0")
    D = run16("bf16", A, B, C)
    D0 = run16("bf16", A, B, None)
    torch.cuda.synchronize()
    assert torch.equal(D, C) and not D0.any()


def test_empty_outputs_do_nothing():
    D = torch.full((4, 4), 7.0, device=DEV)
    A = torch.ones(0, 8, dtype=torch.bfloat16, device=DEV)
    B = torch.ones(4, 8, dtype=torch.bfloat16, device=DEV)
    run16("bf16", A, B, None, D=D[:0])
    run16("bf16", B, A, None, D=D[:, :0])
    torch.cuda.synchronize()
    assert torch.all(D == 7.0)


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(200, 136, 328), (1000, 1000, 64), (513, 1030, 96)])
def test_guard_band_untouched(out, shape):
    M, N, K = shape
    x, _ = _case("bf16", M, N, K, seed=3, integer=True, with_c=False)
    ldd = N + 5
    dt = torch.float32 if out == "f32" else torch.bfloat16
    buf = torch.full((M + 2, ldd), float("nan"), dtype=dt, device=DEV)
    D = buf[1:M + 1, :N]
    say("guard %s %s" % (out, shape))
    run16("bf16", dev16(x["A"], "bf16"), dev16(x["B"], "bf16"), None, out=out, D=D)
    torch.cuda.synchronize()
    assert torch.isnan(buf[0]).all() and torch.isnan(buf[M + 1]).all() and torch.isnan(buf[:, N:]).all()
    assert not torch.isnan(D).any()
    Dr, _ = oracle.gemm_ref_full("bf16", x["A"], x["B"])
    if out == "f32":
        assert np.array_equal(to_f64(D), Dr)
    else:   # the exact integer sum, rounded once to bf16
        assert np.array_equal(bf16_bits(D), oracle.rne_bf16_f32(Dr.astype(np.float32)))


def test_deterministic():
    x, C = _case("bf16", 1024, 768, 1000, seed=8, integer=False)
    A, B, Cd = dev16(x["A"], "bf16"), dev16(x["B"], "bf16"), torch.from_numpy(C).to(DEV)
    say("determinism")
    D1 = run16("bf16", A, B, Cd)
    D2 = run16("bf16", A, B, Cd)
    torch.cuda.synchronize()
    assert torch.equal(D1.view(torch.int32), D2.view(torch.int32))


@pytest.mark.parametrize("shape", [(300, 200, 500), (2048, 2048, 256)])
def test_bf16_output_is_rne_of_fp32(shape):
    M, N, K = shape
    x, C = _case("bf16", M, N, K, seed=21, integer=False, with_c=False)
    A, B = dev16(x["A"], "bf16"), dev16(x["B"], "bf16")
    say("bf16 out %s" % (shape,))
    D32 = run16("bf16", A, B, None, out="f32")
    D16 = run16("bf16", A, B, None, out="bf16")
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(D16), oracle.rne_bf16_f32(D32.cpu().numpy()))
    _full_check("bf16", x, to_f64(D32), False)


# ---- the large workloads --------------------------------------------------------------------

def _sampled(w, x, Dg_flat, extra_rel=0.0):
    rand, forced = inputs.sample_indices(x["M"], x["N"], w.seed)
    for name, idx in (("random", rand), ("forced", forced)):
        Dr, S = oracle.gemm_ref(w.in_type, x["A"], x["B"], C=x["C"], idx=idx)
        rep = check.report(Dg_flat[idx], Dr, S, extra_rel=extra_rel)
        say("  %s: %s" % (name, rep))
        assert rep["fail"] == 0, (name, rep)


def test_square4096():
    w = inputs.WORKLOADS["square4096_bf16"]
    x = inputs.generate(w)
    say("square4096 bf16")
    D = run16("bf16", dev16(x["A"], "bf16"), dev16(x["B"], "bf16"), torch.from_numpy(x["C"]).to(DEV))
    torch.cuda.synchronize()
    Dg = D.cpu().numpy()
    _sampled(w, x, Dg.ravel().astype(np.float64))
    a, b = oracle.operands_f64("bf16", x["A"], x["B"])
    ok, ratio = check.freivalds_blocks(Dg, a, b, x["C"], block=64)
    say("  freivalds worst ratio %.3g" % ratio)
    assert ok


def test_square4096_integer():
    w = inputs.WORKLOADS["square4096_bf16"]
    x = inputs.generate(w, integer=True)
    say("square4096 bf16 integer")
    D = run16("bf16", dev16(x["A"], "bf16"), dev16(x["B"], "bf16"), torch.from_numpy(x["C"]).to(DEV))
    torch.cuda.synchronize()
    Dg = D.cpu().numpy()
    a, b = oracle.operands_f64("bf16", x["A"], x["B"])
    ok, _ = check.freivalds_blocks(Dg, a, b, x["C"], integer=True)
    assert ok
    rand, forced = inputs.sample_indices(4096, 4096, w.seed)
    idx = np.concatenate([rand, forced])
    Dr, _ = oracle.gemm_ref("bf16", x["A"], x["B"], C=x["C"], idx=idx)
    assert np.array_equal(Dg.ravel()[idx].astype(np.float64), Dr)


def test_ragged_fp16_every_element():
    w = inputs.WORKLOADS["ragged_fp16"]
    x = inputs.generate(w)
    say("ragged fp16 4000x3000x4100")
    D = run16("fp16", dev16(x["A"], "fp16"), dev16(x["B"], "fp16"), None)
    torch.cuda.synchronize()
    Dg = to_f64(D)
    _sampled(w, x, Dg.ravel())
    Dr, S = oracle.gemm_ref_full("fp16", x["A"], x["B"])
    rep = check.report(Dg, Dr, S)
    say("  full: %s" % rep)
    assert rep["fail"] == 0


def test_ragged_fp16_integer_every_element():
    """The ragged workload's shape and launch with integer inputs in [-4, 4]:
    every element bit-exact against the float64 product (exact here: every
    partial sum is an integer below 2^24), the samples against the naive loop."""
    w = inputs.WORKLOADS["ragged_fp16"]
    x = inputs.generate(w, integer=True)
    say("ragged fp16 4000x3000x4100 integer")
    D = run16("fp16", dev16(x["A"], "fp16"), dev16(x["B"], "fp16"), None)
    torch.cuda.synchronize()
    Dg = to_f64(D)
    Dr, _ = oracle.gemm_ref_full("fp16", x["A"], x["B"])
    bad = np.argwhere(Dg != Dr)
    assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()
    rand, forced = inputs.sample_indices(x["M"], x["N"], w.seed)
    idx = np.concatenate([rand, forced])
    Dn, _ = oracle.gemm_ref("fp16", x["A"], x["B"], idx=idx)
    assert np.array_equal(Dg.ravel()[idx], Dn)


@pytest.mark.parametrize("name", ["llm_proj_bf16", "llm_proj_shard8_bf16"])
def test_llm_projection_integer(name):
    """The projection shapes with integer inputs in [-4, 4] (|partial sums| <=
    65536 < 2^24, so the exact result is an fp32 value): the fp32-output call
    is exact on every element (integer block-Freivalds, exact in float64) and
    on the samples; the bf16-output call equals the nearest-even rounding of
    that exact result on every element, and on the samples the rounding of
    the naive loop's value."""
    w = inputs.WORKLOADS[name]
    x = inputs.generate(w, integer=True)
    say("%s %dx%dx%d integer, bf16 and fp32 out" % (name, w.M, w.N, w.K))
    A, B = dev16(x["A"], "bf16"), dev16(x["B"], "bf16")
    D16 = run16("bf16", A, B, None, out="bf16")
    D32 = run16("bf16", A, B, None, out="f32")
    torch.cuda.synchronize()
    d32 = D32.cpu().numpy()
    del D32
    d16 = bf16_bits(D16)
    del D16
    a, b = oracle.operands_f64("bf16", x["A"], x["B"])
    ok, worst = check.freivalds_blocks(d32, a, b, None, block=64, integer=True)
    say("  integer freivalds ok=%s worst %.3g" % (ok, worst))
    assert ok
    assert np.array_equal(d16, oracle.rne_bf16_f32(d32))
    rand, forced = inputs.sample_indices(x["M"], x["N"], w.seed)
    idx = np.concatenate([rand, forced])
    Dn, _ = oracle.gemm_ref("bf16", x["A"], x["B"], idx=idx)
    assert np.array_equal(d32.ravel()[idx].astype(np.float64), Dn)
    assert np.array_equal(d16.ravel()[idx], oracle.rne_bf16(Dn))


@pytest.mark.parametrize("name", ["llm_proj_bf16", "llm_proj_shard8_bf16"])
def test_llm_projection_bf16_out(name):
    w = inputs.WORKLOADS[name]
    x = inputs.generate(w)
    say("%s %dx%dx%d bf16 out" % (name, w.M, w.N, w.K))
    A, B = dev16(x["A"], "bf16"), dev16(x["B"], "bf16")
    D16 = run16("bf16", A, B, None, out="bf16")
    D32 = run16("bf16", A, B, None, out="f32")
    torch.cuda.synchronize()
    d32 = D32.cpu().numpy()
    del D32
    # (ii) bf16 result is the nearest-even rounding of the same kernel's fp32 result, every element
    assert np.array_equal(bf16_bits(D16), oracle.rne_bf16_f32(d32))
    # (i) the fp32 result meets the tolerance on the samples and the block-Freivalds check
    _sampled(w, x, d32.ravel().astype(np.float64))
    # (iii) the bf16 result against the oracle with the bf16 half-ulp added
    _sampled(w, x, to_f64(D16).ravel(), extra_rel=2.0 ** -8)
    a, b = oracle.operands_f64("bf16", x["A"], x["B"])
    ok, ratio = check.freivalds_blocks(d32, a, b, None, block=64)
    say("  freivalds worst ratio %.3g" % ratio)
    assert ok


# ---- every kernel configuration ------------------------------------------------------------

# Kernel configurations (csrc/f16_launch.hpp): 0 takes rows only 4- or
# 8-byte aligned; 1 .. 4 the direct-to-LDS kernels; 5 the four-wave kernel
# (256 x 256 tiles), 6 its shifted-row variant (which takes 16-byte rows
# too); 7 and 8 the same two with 192 x 256 tiles.
LANE16_CFGS = [1, 2, 3, 4, 5, 6, 7, 8]
LANE4_CFGS = [0, 1, 2]
FOUR_WAVE, FOUR_WAVE_SHIFTED, FOUR_WAVE_192, FOUR_WAVE_SHIFTED_192 = 5, 6, 7, 8
FOUR_WAVE_ALL = (FOUR_WAVE, FOUR_WAVE_SHIFTED, FOUR_WAVE_192, FOUR_WAVE_SHIFTED_192)


@pytest.mark.parametrize("cfg", LANE16_CFGS)
def test_every_config(cfg, monkeypatch):
    """Each configuration the kernel choice uses, forced through the test
    override on 16-byte rows: bit-exact on integers over ragged shapes,
    within tolerance on random data."""
    monkeypatch.setenv("TILEGEMM_F16_CONFIG", str(cfg))
    for (M, N, K) in [(300, 520, 200), (777, 513, 1000), (64, 64, 64)]:
        for integer in (True, False):
            x, C = _case("bf16", M, N, K, seed=cfg * 31 + M, integer=integer)
            say("cfg %d %dx%dx%d integer=%s" % (cfg, M, N, K, integer))
            D = run16("bf16", dev16(x["A"], "bf16"), dev16(x["B"], "bf16"), torch.from_numpy(C).to(DEV))
            torch.cuda.synchronize()
            _full_check("bf16", x, to_f64(D), integer, C)
    x, _ = _case("fp16", 513, 300, 4160, seed=cfg, integer=True, with_c=False)
    D16 = run16("fp16", dev16(x["A"], "fp16"), dev16(x["B"], "fp16"), None, out="bf16")
    D32 = run16("fp16", dev16(x["A"], "fp16"), dev16(x["B"], "fp16"), None, out="f32")
    torch.cuda.synchronize()
    _full_check("fp16", x, to_f64(D32), True)
    assert np.array_equal(bf16_bits(D16), oracle.rne_bf16_f32(D32.cpu().numpy()))


@pytest.mark.parametrize("cfg", LANE4_CFGS)
@pytest.mark.parametrize("pad", [2, 4])
def test_lane4_configs(cfg, pad, monkeypatch):
    """Rows only 4- or 8-byte aligned (leading dimension K + pad) take the
    4-byte-lane direct-to-LDS kernels; every such configuration, forced."""
    monkeypatch.setenv("TILEGEMM_F16_CONFIG", str(cfg))
    for in_type in ("bf16", "fp16"):
        for integer in (True, False):
            M, N, K = 520, 300, 4100
            x, C = _case(in_type, M, N, K, seed=cfg + pad, integer=integer)
            lda = K + pad
            Ab = np.zeros((M, lda), np.uint16); Ab[:, :K] = x["A"]
            Bb = np.zeros((N, lda), np.uint16); Bb[:, :K] = x["B"]
            say("lane4 cfg %d pad %d %s integer=%s" % (cfg, pad, in_type, integer))
            D = run16(in_type, dev16(Ab, in_type)[:, :K], dev16(Bb, in_type)[:, :K], torch.from_numpy(C).to(DEV))
            torch.cuda.synchronize()
            _full_check(in_type, x, to_f64(D), integer, C)


@pytest.mark.parametrize("cfg", LANE16_CFGS)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_c_streamed_in_k_loop(cfg, out, monkeypatch):
    """K long enough (>= 34 tiles of 64) that C is added during the K loop
    instead of in the epilogue: ragged M/N, both output types, and C == D."""
    monkeypatch.setenv("TILEGEMM_F16_CONFIG", str(cfg))
    M = 300
    cases = [(520, 2304)]
    if cfg in FOUR_WAVE_ALL:
        # the stream's threshold (20 K tiles for 256 x 256 tiles, 16 for
        # 192 x 256), a ragged K with the stream, and N % 4 != 0 (C added in
        # the epilogue)
        cases += [(520, 1344), (520, 1280), (520, 1216), (520, 1300), (518, 2304)]
    for N, K, integer in [(n, k, i) for (n, k) in cases for i in (True, False)]:
        x, C = _case("bf16", M, N, K, seed=cfg * 7 + (out == "bf16"), integer=integer)
        A, B = dev16(x["A"], "bf16"), dev16(x["B"], "bf16")
        if out == "bf16":
            Cb = torch.from_numpy(C).to(DEV).to(torch.bfloat16)
            Cref = Cb.float().cpu().numpy()
            say("c-loop cfg %d N %d K %d bf16 out integer=%s" % (cfg, N, K, integer))
            D16 = run16("bf16", A, B, Cb, out="bf16")
            D32 = run16("bf16", A, B, torch.from_numpy(Cref).to(DEV), out="f32")
            torch.cuda.synchronize()
            _full_check("bf16", x, to_f64(D32), integer, Cref)
            assert np.array_equal(bf16_bits(D16), oracle.rne_bf16_f32(D32.cpu().numpy()))
        else:
            Cd = torch.from_numpy(C).to(DEV)
            say("c-loop cfg %d N %d K %d f32 out integer=%s" % (cfg, N, K, integer))
            D = run16("bf16", A, B, Cd)
            inplace = Cd.clone()
            run16("bf16", A, B, inplace, D=inplace)
            torch.cuda.synchronize()
            _full_check("bf16", x, to_f64(D), integer, C)
            assert torch.equal(D, inplace)


@pytest.mark.parametrize("cfg", [None, FOUR_WAVE, FOUR_WAVE_SHIFTED, FOUR_WAVE_192, FOUR_WAVE_SHIFTED_192, 1, 3])
@pytest.mark.parametrize("K,pad", [(100, 4), (200, 8), (72, 16), (4100, 4), (36, 60)])
def test_nan_past_k_never_reaches_d(cfg, K, pad, monkeypatch):
    """Rows padded past K with NaN codes: the kernels load whole chunks and
    clear what lies past K in LDS, so no padding value may reach D (a NaN
    times a zero would).  Integer inputs, every element exact."""
    if cfg is not None:
        monkeypatch.setenv("TILEGEMM_F16_CONFIG", str(cfg))
    M, N = 300, 520
    ld = K + pad
    if cfg in (FOUR_WAVE, FOUR_WAVE_192, 1, 3) and ld % 8:
        pytest.skip("16-byte rows only")
    x, C = _case("bf16", M, N, K, seed=K + pad, integer=True)
    Ab = np.full((M, ld), 0x7FC0, np.uint16); Ab[:, :K] = x["A"]
    Bb = np.full((N, ld), 0x7FC0, np.uint16); Bb[:, :K] = x["B"]
    say("NaN past K cfg %s K %d ld %d" % (cfg, K, ld))
    D = run16("bf16", dev16(Ab, "bf16")[:, :K], dev16(Bb, "bf16")[:, :K], torch.from_numpy(C).to(DEV))
    torch.cuda.synchronize()
    _full_check("bf16", x, to_f64(D), True, C)


# ---- rows only 8-byte aligned: the shifted-row four-wave kernel ---------------------------

@pytest.mark.parametrize("cfg", [FOUR_WAVE_SHIFTED, FOUR_WAVE_SHIFTED_192])
@pytest.mark.parametrize("case", [
    # M, N, K, pad (lda = ldb = K + pad), element offset of A and B, C, output
    (520, 300, 4100, 0, 0, True, "f32"),     # packed 8-byte rows, ragged last K tile (past K cleared)
    (300, 520, 4100, 0, 4, True, "f32"),     # operands start 8 bytes past a 16-byte boundary
    (257, 260, 36, 0, 0, True, "f32"),       # one ragged K tile (cleared in the prologue)
    (257, 260, 100, 4, 0, False, "f32"),     # two K tiles, padded rows
    (256, 256, 320, 4, 4, True, "f32"),      # K a multiple of 64, 8-byte rows
    (300, 520, 2308, 0, 0, True, "f32"),     # C streamed in the K loop
    (300, 520, 2308, 0, 0, True, "bf16"),
])
def test_shifted_rows(case, cfg, monkeypatch):
    monkeypatch.setenv("TILEGEMM_F16_CONFIG", str(cfg))
    M, N, K, pad, off, with_c, out = case
    for in_type in ("fp16", "bf16"):
        for integer in (True, False):
            x, C = _case(in_type, M, N, K, seed=M + K + pad + off, integer=integer, with_c=with_c)
            ld = K + pad
            Ab = np.zeros(off + M * ld, np.uint16); Ab[off:].reshape(M, ld)[:, :K] = x["A"]
            Bb = np.zeros(off + N * ld, np.uint16); Bb[off:].reshape(N, ld)[:, :K] = x["B"]
            A = dev16(Ab, in_type)[off:].view(M, ld)[:, :K]
            B = dev16(Bb, in_type)[off:].view(N, ld)[:, :K]
            say("shifted rows %dx%dx%d pad %d off %d C %s %s out %s integer=%s" % (M, N, K, pad, off, with_c, in_type, out, integer))
            if out == "bf16":
                Cb = torch.from_numpy(C).to(DEV).to(torch.bfloat16) if with_c else None
                Cref = Cb.float().cpu().numpy() if with_c else None
                D16 = run16(in_type, A, B, Cb, out="bf16")
                D32 = run16(in_type, A, B, torch.from_numpy(Cref).to(DEV) if with_c else None, out="f32")
                torch.cuda.synchronize()
                _full_check(in_type, x, to_f64(D32), integer, Cref)
                assert np.array_equal(bf16_bits(D16), oracle.rne_bf16_f32(D32.cpu().numpy()))
            else:
                D = run16(in_type, A, B, torch.from_numpy(C).to(DEV) if with_c else None)
                torch.cuda.synchronize()
                _full_check(in_type, x, to_f64(D), integer, C if with_c else None)
