"""fp6 operands as tile images (gemm_mxfp6_pack, gemm_mxfp6_packed).

The image layout is restated here from its definition in the header (image
(b, t) of row block b and K tile t at (b * K/128 + t) * 24576; its 16-byte
chunk c holds bytes 96 t + 16 h .. + 15 of row 256 b + c / 6, h = (c % 6) ^
((c / 6 >> 3) & 1); zeros past the last row) and the packing kernel's output
is compared with it byte for byte, on aligned rows (one 16-byte load per
chunk) and on rows that start at any byte.  The packed GEMM: bit-exact
against the oracle on integer-valued inputs, within |D - D_ref| <= 2^-12 *
sum|a*b| + 1e-6 on random ones, and equal bit for bit to gemm_mxfp6 on the
same operands (the same kernel and MFMA order), over ragged M and N, a
single tile, K not a multiple of the 512-wide scale group, C and no C, both
output types and a grid large enough for the persistent kernel.  (Scale rows
are padded to whole 16-byte words, which the packed call requires.)
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


def images_ref(X, K):
    """The tile images of the (rows, >= 3K/4) byte array X, from the layout's
    definition."""
    rows = X.shape[0]
    nb, nk = (rows + 255) // 256, K // 128
    out = np.zeros((nb, nk, 1536, 16), np.uint8)
    c = np.arange(1536)
    r = c // 6
    h = (c % 6) ^ ((r >> 3) & 1)
    for b in range(nb):
        for t in range(nk):
            for cc in range(1536):
                row = 256 * b + r[cc]
                if row < rows:
                    s = 96 * t + 16 * h[cc]
                    out[b, t, cc] = X[row, s:s + 16]
    return out.reshape(-1)


# (rows, K, extra bytes per row, byte offset of the first row)
PACK_CASES = [(256, 128, 0, 0), (300, 512, 0, 0), (1, 256, 0, 0), (513, 384, 48, 0), (70, 256, 3, 0),
              (40, 128, 0, 5), (257, 640, 9, 7)]


@pytest.mark.parametrize("case", PACK_CASES, ids=["%dx%d+%d@%d" % c for c in PACK_CASES])
def test_pack_layout(case):
    rows, K, pad, off = case
    rng = np.random.default_rng(rows + K + pad + off)
    w = K // 4 * 3 + pad
    store = rng.integers(0, 256, size=off + rows * w, dtype=np.uint8)
    X = store[off:].reshape(rows, w)
    dX = dev8(store)[off:].view(rows, w)[:, :K // 4 * 3]
    say("mxfp6 pack rows %d K %d pad %d off %d" % (rows, K, pad, off))
    P = tg.mxfp6_pack(dX)
    torch.cuda.synchronize()
    assert P.numel() == tg.mxfp6_packed_bytes(rows, K) == images_ref(X, K).size
    assert np.array_equal(P.cpu().numpy(), images_ref(X, K))


def test_pack_leaves_bytes_past_the_images():
    rows, K = 100, 256
    rng = np.random.default_rng(3)
    X = rng.integers(0, 256, size=(rows, K // 4 * 3), dtype=np.uint8)
    need = tg.mxfp6_packed_bytes(rows, K)
    big = torch.full((need + 4096,), 0xA5, dtype=torch.uint8, device=DEV)
    tg.mxfp6_pack(dev8(X), out=big)
    torch.cuda.synchronize()
    got = big.cpu().numpy()
    assert np.array_equal(got[:need], images_ref(X, K))
    assert (got[need:] == 0xA5).all()


def dev_scales(S):
    """Device scales with rows padded to whole 16-byte words (what the
    packed call requires of ldsfa / ldsfb)."""
    rows, n = S.shape
    ld = -(-max(n, 1) // 16) * 16
    buf = np.zeros((rows, ld), np.uint8)
    buf[:, :n] = S
    return dev8(buf)[:, :n]


def _case(fmt, M, N, K, seed, integer, with_c):
    rng = np.random.default_rng(seed)
    A = inputs.random_codes(rng, fmt, (M, K), integer=integer)
    B = inputs.random_codes(rng, fmt, (N, K), integer=integer)
    if integer:
        e = inputs.fp6_integer_scale(fmt)
        SFA = (127 + e + rng.integers(0, 2, size=(M, K // 32))).astype(np.uint8)
        SFB = np.full((N, K // 32), 127 + e, np.uint8)
    else:
        SFA = (127 + rng.integers(-4, 5, size=(M, K // 32))).astype(np.uint8)
        SFB = (127 + rng.integers(-4, 5, size=(N, K // 32))).astype(np.uint8)
    C = None
    if with_c:
        C = (rng.integers(-4, 5, size=(M, N)) if integer else rng.uniform(-1, 1, size=(M, N))).astype(np.float32)
    return A, B, SFA, SFB, C


# (M, N, K, C given): ragged tiles, one tile, K % 512 != 0 (the last scale
# group short), one K tile, a persistent grid (no C, more tiles than CUs)
GEMM_CASES = [(300, 200, 256, True), (256, 256, 128, True), (513, 260, 640, False), (100, 36, 1152, True),
              (64, 520, 128, False), (4200, 4300, 512, False)]


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
@pytest.mark.parametrize("case", GEMM_CASES, ids=["%dx%dx%d%s" % (c[0], c[1], c[2], "+C" if c[3] else "")
                                                  for c in GEMM_CASES])
def test_packed_gemm(fmt, case):
    M, N, K, with_c = case
    big = M * N > 4 * 10 ** 6
    for integer in ((True,) if big else (True, False)):
        A, B, SFA, SFB, C = _case(fmt, M, N, K, M + 3 * N + K + len(fmt) + integer, integer, with_c)
        dA, dB, dSA, dSB = dev8(A), dev8(B), dev_scales(SFA), dev_scales(SFB)
        AP, BP = tg.mxfp6_pack(dA), tg.mxfp6_pack(dB)
        for out in (torch.float32, torch.bfloat16):
            Cd = torch.from_numpy(C).to(DEV).to(out) if C is not None else None
            say("mxfp6 packed %s %dx%dx%d C=%s integer=%s out=%s" % (fmt, M, N, K, with_c, integer, out))
            D = tg.gemm_mxfp6_packed(AP, dSA, BP, dSB, M, N, K, Cd, out_dtype=out, fmt=fmt)
            Ds = tg.gemm_mxfp6(dA, dSA, dB, dSB, Cd, out_dtype=out, fmt=fmt)
            torch.cuda.synchronize()
            assert torch.equal(D, Ds)
            if out == torch.bfloat16:
                continue
            if big:
                rand, forced = inputs.sample_indices(M, N, K)
                idx = np.concatenate([rand, forced])
                Dr, _ = oracle.gemm_ref(fmt, A, B, idx=idx, SFA=SFA, SFB=SFB)
                assert np.array_equal(to_f64(D).ravel()[idx], Dr)
                continue
            Dr, S = oracle.gemm_ref_full(fmt, A, B, C=C, SFA=SFA, SFB=SFB)
            Dg = to_f64(D)
            if integer:
                bad = np.argwhere(Dg != Dr)
                assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()
            else:
                rep = check.report(Dg, Dr, S)
                assert rep["fail"] == 0, rep


def test_packed_bf16_output_is_rne_of_f32():
    M, N, K = 260, 300, 384
    A, B, SFA, SFB, C = _case("e2m3", M, N, K, 17, False, True)
    AP, BP = tg.mxfp6_pack(dev8(A)), tg.mxfp6_pack(dev8(B))
    Cf = torch.from_numpy(C).to(DEV)
    say("mxfp6 packed bf16 out")
    dSA, dSB = dev_scales(SFA), dev_scales(SFB)
    D32 = tg.gemm_mxfp6_packed(AP, dSA, BP, dSB, M, N, K, Cf.bfloat16().float())
    D16 = tg.gemm_mxfp6_packed(AP, dSA, BP, dSB, M, N, K, Cf.bfloat16(), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(D16), oracle.rne_bf16_f32(D32.cpu().numpy()))


def test_packed_k_zero_gives_c():
    M, N = 70, 90
    C = torch.randn((M, N), device=DEV)
    e = torch.empty(0, dtype=torch.uint8, device=DEV)
    s = torch.empty((M, 0), dtype=torch.uint8, device=DEV)
    t = torch.empty((N, 0), dtype=torch.uint8, device=DEV)
    D = tg.gemm_mxfp6_packed(e, s, e, t, M, N, 0, C)
    torch.cuda.synchronize()
    assert torch.equal(D, C)


@pytest.mark.parametrize("integer", [False, True])
def test_packed_workload_8192(integer):
    """The timed packed workload (8192^3, operands packed once, the
    persistent kernel): sampled outputs against the oracle, exact on integer
    inputs, and the block-Freivalds check over all of D."""
    w = inputs.WORKLOADS["mxfp6_8192_packed"]
    x = inputs.generate(w, integer=integer)
    say("mxfp6 packed 8192^3 integer=%s" % integer)
    SA, SB = dev8(x["SFA"]), dev8(x["SFB"])
    AP, BP = tg.mxfp6_pack(dev8(x["A"])), tg.mxfp6_pack(dev8(x["B"]))
    D = tg.gemm_mxfp6_packed(AP, SA, BP, SB, w.M, w.N, w.K, fmt=w.in_type)
    torch.cuda.synchronize()
    Dg = D.cpu().numpy()
    del D, AP, BP
    rand, forced = inputs.sample_indices(w.M, w.N, w.seed)
    a, b = oracle.operands_f64(w.in_type, x["A"], x["B"], SFA=x["SFA"], SFB=x["SFB"])
    for name, idx in (("random", rand), ("forced", forced)):
        Dr, S = oracle.gemm_ref(w.in_type, x["A"], x["B"], SFA=x["SFA"], SFB=x["SFB"], idx=idx)
        got = Dg.ravel()[idx].astype(np.float64)
        if integer:
            assert np.array_equal(got, Dr), name
        else:
            rep = check.report(got, Dr, S)
            assert rep["fail"] == 0, (name, rep)
    ok, ratio = check.freivalds_blocks(Dg, a, b, None, block=64, integer=integer)
    say("  freivalds ok=%s worst %.3g" % (ok, ratio))
    assert ok


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
@pytest.mark.parametrize("case", [(300, 200, 640, True), (4200, 4300, 512, False)], ids=["300x200x640+C", "4200x4300x512"])
def test_ex_ws_k_contiguous_uses_images(fmt, case):
    """gemm_mxfp6 with a workspace and K-contiguous operands (gemm_mxfp6_ex_ws):
    the operands' tile images in the workspace, then the packed kernel --
    equal bit for bit to the plain call; a workspace one byte short gives
    the plain call."""
    M, N, K, with_c = case
    A, B, SFA, SFB, C = _case(fmt, M, N, K, M + N + K + len(fmt), True, with_c)
    dA, dB, dSA, dSB = dev8(A), dev8(B), dev_scales(SFA), dev_scales(SFB)
    need = tg.ex_workspace_bytes(6, M, N, K)
    assert need == -(-tg.mxfp6_packed_bytes(M, K) // 256) * 256 + -(-tg.mxfp6_packed_bytes(N, K) // 256) * 256
    for out in (torch.float32, torch.bfloat16):
        Cd = torch.from_numpy(C).to(DEV).to(out) if C is not None else None
        say("mxfp6 ex_ws images %s %dx%dx%d C=%s out=%s" % (fmt, M, N, K, with_c, out))
        ws = torch.empty(need + 256, dtype=torch.uint8, device=DEV)
        ws = ws[(-ws.data_ptr()) % 256:]
        D = tg.gemm_mxfp6(dA, dSA, dB, dSB, Cd, out_dtype=out, fmt=fmt, workspace=ws[:need])
        Dshort = tg.gemm_mxfp6(dA, dSA, dB, dSB, Cd, out_dtype=out, fmt=fmt, workspace=ws[:need - 1])
        Ds = tg.gemm_mxfp6(dA, dSA, dB, dSB, Cd, out_dtype=out, fmt=fmt)
        torch.cuda.synchronize()
        assert torch.equal(D, Ds)
        assert torch.equal(Dshort, Ds)
    if not (M * N > 4 * 10 ** 6):
        Dr, _ = oracle.gemm_ref_full(fmt, A, B, C=C, SFA=SFA, SFB=SFB)
        D = tg.gemm_mxfp6(dA, dSA, dB, dSB, torch.from_numpy(C).to(DEV) if C is not None else None, fmt=fmt,
                          workspace=ws[:need])
        torch.cuda.synchronize()
        assert np.array_equal(to_f64(D), Dr)


@pytest.mark.parametrize("shape", [(1, 1, 128), (1, 300, 256), (257, 1, 384), (16, 16, 8192)],
                         ids=["1x1x128", "1x300x256", "257x1x384", "16x16x8192"])
def test_packed_edge_shapes(shape):
    """Single rows and columns (image blocks almost all padding), one K tile,
    a long K with a short grid: exact on integer inputs, equal to the plain
    call."""
    M, N, K = shape
    A, B, SFA, SFB, C = _case("e3m2", M, N, K, M * 7 + N * 3 + K, True, True)
    dSA, dSB = dev_scales(SFA), dev_scales(SFB)
    AP, BP = tg.mxfp6_pack(dev8(A)), tg.mxfp6_pack(dev8(B))
    Cd = torch.from_numpy(C).to(DEV)
    say("mxfp6 packed edge %dx%dx%d" % (M, N, K))
    D = tg.gemm_mxfp6_packed(AP, dSA, BP, dSB, M, N, K, Cd, fmt="e3m2")
    Ds = tg.gemm_mxfp6(dev8(A), dSA, dev8(B), dSB, Cd, fmt="e3m2")
    torch.cuda.synchronize()
    assert torch.equal(D, Ds)
    Dr, _ = oracle.gemm_ref_full("e3m2", A, B, C=C, SFA=SFA, SFB=SFB)
    assert np.array_equal(to_f64(D), Dr)


def test_packed_in_place_c_equals_d():
    """C == D (ldc == ldd): each element read before it is written."""
    M, N, K = 300, 260, 512
    A, B, SFA, SFB, C = _case("e2m3", M, N, K, 21, True, True)
    dSA, dSB = dev_scales(SFA), dev_scales(SFB)
    AP, BP = tg.mxfp6_pack(dev8(A)), tg.mxfp6_pack(dev8(B))
    CD = torch.from_numpy(C).to(DEV)
    say("mxfp6 packed C == D")
    tg.gemm_mxfp6_packed(AP, dSA, BP, dSB, M, N, K, CD, D=CD)
    torch.cuda.synchronize()
    Dr, _ = oracle.gemm_ref_full("e2m3", A, B, C=C, SFA=SFA, SFB=SFB)
    assert np.array_equal(to_f64(CD), Dr)
