"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments before touching the GPU (CPU only: no compute call is made)."""
import os
import re
import subprocess

import pytest

import tiled_dense_gemm_tile_amd as tg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tilegemm.h")

OK, INVALID_SIZE, NULL_POINTER, BAD_LD, MISALIGNED, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3, 4, 5, 7
F32, BF16 = 0, 1
P = 0x10000000  # a fake, aligned device address: never dereferenced by these calls


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["gemm_bf16", "gemm_bf16_ex", "gemm_bf16_ex_ws", "gemm_bf16_splitk",
                                    "gemm_bf16_splitk_noalloc", "gemm_ex_workspace_bytes",
                                    "gemm_fp16", "gemm_fp16_ex", "gemm_fp16_ex_ws", "gemm_fp16_splitk",
                                    "gemm_last_hip_error",
                                    "gemm_mx_kblock", "gemm_mx_kblock_workspace_bytes", "gemm_mx_kblock_ws",
                                    "gemm_mxfp4", "gemm_mxfp4_ex", "gemm_mxfp4_ex_ws", "gemm_mxfp4_splitk",
                                    "gemm_mxfp6", "gemm_mxfp6_ex", "gemm_mxfp6_ex_ws", "gemm_mxfp6_pack",
                                    "gemm_mxfp6_packed", "gemm_mxfp6_packed_bytes", "gemm_mxfp6_splitk",
                                    "gemm_mxfp8", "gemm_mxfp8_ex", "gemm_mxfp8_ex_ws", "gemm_mxfp8_splitk",
                                    "gemm_splitk_scratch_limit", "gemm_splitk_workspace_bytes",
                                    "gemm_status_string"]


def test_library_exports_every_declared_symbol():
    path = tg.library_path()
    assert os.path.exists(path), "build the library first"
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(tg.raw, name) is not None


def test_status_strings():
    for s in range(9):
        assert tg.raw.status_string(s).startswith(tg.STATUS[s])
    assert "unknown" in tg.raw.status_string(99)
    assert tg.raw.gemm_last_hip_error() == 0


def call16(fn="gemm_bf16", M=64, N=64, K=64, A=P, lda=64, B=P, ldb=64, C=None, ldc=0, D=P + (1 << 24),
           ldd=64, out=F32):
    return getattr(tg.raw, fn)(M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out, None)


@pytest.mark.parametrize("fn", ["gemm_bf16", "gemm_fp16"])
def test_validation_16bit(fn):
    assert call16(fn, M=-1) == INVALID_SIZE
    assert call16(fn, N=-5) == INVALID_SIZE
    assert call16(fn, K=-1) == INVALID_SIZE
    assert call16(fn, M=0) == OK                       # nothing to do, nothing launched
    assert call16(fn, N=0, D=None, A=None) == OK
    assert call16(fn, M=1 << 31) == UNSUPPORTED
    assert call16(fn, out=7) == UNSUPPORTED
    assert call16(fn, lda=63) == BAD_LD
    assert call16(fn, ldb=10) == BAD_LD
    assert call16(fn, ldd=63) == BAD_LD
    assert call16(fn, C=P + (1 << 26), ldc=32) == BAD_LD
    assert call16(fn, D=None) == NULL_POINTER
    assert call16(fn, A=None) == NULL_POINTER
    assert call16(fn, B=None) == NULL_POINTER
    assert call16(fn, A=P + 1) == MISALIGNED
    assert call16(fn, D=P + (1 << 24) + 2) == MISALIGNED
    assert call16(fn, D=P + (1 << 24) + 2, out=BF16, C=P + 3, ldc=64) == MISALIGNED
    assert call16(fn, lda=4 << 20, K=64) == UNSUPPORTED     # 8 MiB rows
    D = P + (1 << 24)
    assert call16(fn, C=D + 4, ldc=64, D=D) == UNSUPPORTED  # partial overlap of C and D
    assert call16(fn, C=D, ldc=128, D=D, ldd=64) == UNSUPPORTED


def call8(M=64, N=64, K=64, A=P, lda=64, SFA=P + 4096, ldsfa=2, B=P, ldb=64, SFB=P + 8192, ldsfb=2,
          C=None, ldc=0, D=P + (1 << 24), ldd=64, out=F32):
    return tg.raw.gemm_mxfp8(M, N, K, A, lda, SFA, ldsfa, B, ldb, SFB, ldsfb, C, ldc, D, ldd, out, None)


def test_validation_mxfp8():
    assert call8(M=-1) == INVALID_SIZE
    assert call8(M=0) == OK
    assert call8(K=48, lda=64, ldb=64) == UNSUPPORTED       # K not a multiple of 32
    assert call8(ldsfa=1) == BAD_LD
    assert call8(ldsfb=1) == BAD_LD
    assert call8(SFA=None) == NULL_POINTER
    assert call8(SFB=None) == NULL_POINTER
    assert call8(lda=32) == BAD_LD
    assert call8(D=None) == NULL_POINTER


def call4(M=64, N=64, K=512, A=P, lda=512, SFA=P + 4096, ldsfa=16, B=P, ldb=512, SFB=P + 8192, ldsfb=16,
          C=None, ldc=0, D=P + (1 << 24), ldd=64, out=F32):
    return tg.raw.gemm_mxfp4(M, N, K, A, lda, SFA, ldsfa, B, ldb, SFB, ldsfb, C, ldc, D, ldd, out, None)


def test_validation_mxfp4():
    """Every case is refused before anything is launched (lda, ldb, K in
    elements, two per byte)."""
    assert call4(M=-1) == INVALID_SIZE
    assert call4(K=-2) == INVALID_SIZE
    assert call4(M=0) == OK
    assert call4(out=3) == UNSUPPORTED
    assert call4(lda=510) == BAD_LD
    assert call4(ldb=2) == BAD_LD
    assert call4(ldd=32) == BAD_LD
    assert call4(lda=513) == UNSUPPORTED                   # rows must start on a byte
    assert call4(ldb=515) == UNSUPPORTED
    assert call4(K=48, lda=64, ldb=64) == UNSUPPORTED       # K not a multiple of 32
    assert call4(ldsfa=15) == BAD_LD
    assert call4(ldsfb=8) == BAD_LD
    assert call4(SFA=None) == NULL_POINTER
    assert call4(SFB=None) == NULL_POINTER
    assert call4(A=None) == NULL_POINTER
    assert call4(D=None) == NULL_POINTER
    assert call4(lda=16 << 20) == UNSUPPORTED               # 8 MiB rows
    assert call4(K=1 << 31, lda=1 << 31, ldb=1 << 31) == UNSUPPORTED


def call6(M=64, N=64, K=512, A=P, lda=512, SFA=P + 4096, ldsfa=16, B=P, ldb=512, SFB=P + 8192, ldsfb=16,
          C=None, ldc=0, D=P + (1 << 24), ldd=64, fmt=0, out=F32):
    return tg.raw.gemm_mxfp6(M, N, K, A, lda, SFA, ldsfa, B, ldb, SFB, ldsfb, C, ldc, D, ldd, fmt, out, None)


def test_validation_mxfp6():
    """Every case is refused before anything is launched (lda, ldb, K in
    elements, four per three bytes)."""
    assert call6(M=-1) == INVALID_SIZE
    assert call6(K=-4) == INVALID_SIZE
    assert call6(M=0) == OK
    assert call6(out=3) == UNSUPPORTED
    assert call6(fmt=2) == UNSUPPORTED
    assert call6(fmt=-1) == UNSUPPORTED
    assert call6(lda=508) == BAD_LD
    assert call6(ldb=4) == BAD_LD
    assert call6(ldd=32) == BAD_LD
    assert call6(lda=514) == UNSUPPORTED                   # rows must start on a byte
    assert call6(ldb=513) == UNSUPPORTED
    assert call6(K=48, lda=64, ldb=64) == UNSUPPORTED       # K not a multiple of 32
    assert call6(ldsfa=15) == BAD_LD
    assert call6(ldsfb=8) == BAD_LD
    assert call6(SFA=None) == NULL_POINTER
    assert call6(SFB=None) == NULL_POINTER
    assert call6(A=None) == NULL_POINTER
    assert call6(D=None) == NULL_POINTER
    assert call6(lda=16 << 20) == UNSUPPORTED               # 12 MiB rows
    assert call6(K=1 << 31, lda=1 << 31, ldb=1 << 31) == UNSUPPORTED


def splitk_bytes(M, N, K, splits):
    return tg.raw.gemm_splitk_workspace_bytes(M, N, K, splits)


def test_splitk_workspace_bytes():
    # splits_used * M * round_up(N, 4) * 4
    assert splitk_bytes(256, 256, 4096, 4) == 4 * 256 * 256 * 4
    assert splitk_bytes(300, 201, 5000, 3) == 3 * 300 * 204 * 4
    assert splitk_bytes(64, 64, 8192, 1) == 0                 # no split
    assert splitk_bytes(64, 64, 64, 4) == 0                   # one K tile: nothing to split
    assert splitk_bytes(64, 64, 192, 8) == 3 * 64 * 64 * 4    # at most one split per 64-wide K tile
    assert splitk_bytes(64, 64, 640, 4) == 4 * 64 * 64 * 4    # 10 K tiles: ranges of 3, 3, 3, 1
    assert splitk_bytes(64, 64, 576, 4) == 3 * 64 * 64 * 4    # 9 K tiles: ranges of 3 -> 3 splits
    assert splitk_bytes(1024, 1024, 65536, 0) == 16 * 1024 * 1024 * 4   # 16 tiles, 1024 K tiles: 16 splits
    assert splitk_bytes(4096, 4096, 4096, 0) == 0             # 256 tiles: the library does not split
    assert splitk_bytes(512, 512, 8192, 0) == 2 * 512 * 512 * 4   # 4 tiles, 128 K tiles: 2 splits of 4096
    assert splitk_bytes(1024, 1024, 8192, 0) == 0             # 16 tiles x 6 ranges < 200 workgroups: unsplit
    assert splitk_bytes(2304, 2304, 4096, 0) == 3 * 2304 * 2304 * 4   # 81 tiles: 3 ranges of >= 20 K tiles
    assert splitk_bytes(2048, 2048, 8192, 0) == 4 * 2048 * 2048 * 4   # 64 tiles: 4 ranges
    assert splitk_bytes(2048, 2048, 4096, 0) == 0             # 64 tiles x 3 ranges < 200: unsplit
    assert splitk_bytes(64, 64, 4096, 65) == 0 and splitk_bytes(-1, 64, 4096, 2) == 0


def call16s(fn="gemm_bf16_splitk", M=256, N=256, K=4096, A=P, lda=4096, B=P, ldb=4096, C=None, ldc=0,
            D=P + (1 << 24), ldd=256, out=F32, splits=4, ws=P + (1 << 26), wsb=None):
    if wsb is None:
        wsb = splitk_bytes(M, N, K, splits)
    return getattr(tg.raw, fn)(M, N, K, A, lda, B, ldb, C, ldc, D, ldd, out, splits, ws, wsb, None)


@pytest.mark.parametrize("fn", ["gemm_bf16_splitk", "gemm_fp16_splitk"])
def test_validation_splitk(fn):
    """Every case is refused before anything is launched."""
    assert call16s(fn, M=-1) == INVALID_SIZE
    assert call16s(fn, M=0) == OK
    assert call16s(fn, lda=100) == BAD_LD
    assert call16s(fn, D=None) == NULL_POINTER
    assert call16s(fn, out=9) == UNSUPPORTED
    assert call16s(fn, splits=-1) == UNSUPPORTED
    assert call16s(fn, splits=65) == UNSUPPORTED
    assert call16s(fn, ws=None) == WORKSPACE
    assert call16s(fn, wsb=4 * 256 * 256 * 4 - 1) == WORKSPACE
    assert call16s(fn, ws=P + (1 << 26) + 128) == MISALIGNED


def callms(fn, M=256, N=256, K=4096, A=P, lda=4096, SFA=P + 4096, ldsfa=128, B=P, ldb=4096, SFB=P + 8192,
           ldsfb=128, C=None, ldc=0, D=P + (1 << 24), ldd=256, out=F32, splits=4, ws=P + (1 << 26), wsb=None,
           fmt=0):
    if wsb is None:
        wsb = splitk_bytes(M, N, K, splits)
    args = [M, N, K, A, lda, SFA, ldsfa, B, ldb, SFB, ldsfb, C, ldc, D, ldd]
    if fn == "gemm_mxfp6_splitk":
        args.append(fmt)
    return getattr(tg.raw, fn)(*args, out, splits, ws, wsb, None)


@pytest.mark.parametrize("fn", ["gemm_mxfp8_splitk", "gemm_mxfp4_splitk", "gemm_mxfp6_splitk"])
def test_validation_mx_splitk(fn):
    """Every case is refused before anything is launched (the arguments are a
    valid fast-path call apart from the one changed)."""
    assert callms(fn, M=-1) == INVALID_SIZE
    assert callms(fn, M=0) == OK
    assert callms(fn, lda=100) == BAD_LD
    assert callms(fn, ldsfa=100) == BAD_LD
    assert callms(fn, SFB=None) == NULL_POINTER
    assert callms(fn, D=None) == NULL_POINTER
    assert callms(fn, out=9) == UNSUPPORTED
    assert callms(fn, splits=-1) == UNSUPPORTED
    assert callms(fn, splits=65) == UNSUPPORTED
    assert callms(fn, ws=None) == WORKSPACE
    assert callms(fn, wsb=4 * 256 * 256 * 4 - 1) == WORKSPACE
    assert callms(fn, ws=P + (1 << 26) + 128) == MISALIGNED
    if fn == "gemm_mxfp6_splitk":
        assert callms(fn, fmt=2) == UNSUPPORTED


def callmx(fn, M=256, N=192, K=512, A=P, lda=256, ao=1, SFA=P + 4096, ldsfa=16, B=P, ldb=512, bo=0,
           SFB=P + 8192, ldsfb=16, C=None, ldc=0, D=P + (1 << 24), ldd=192, out=F32, fmt=0):
    args = [M, N, K, A, lda, ao, SFA, ldsfa, B, ldb, bo, SFB, ldsfb, C, ldc, D, ldd]
    if fn == "gemm_mxfp6_ex":
        args.append(fmt)
    return getattr(tg.raw, fn)(*args, out, None)


@pytest.mark.parametrize("fn", ["gemm_mxfp8_ex", "gemm_mxfp4_ex", "gemm_mxfp6_ex"])
def test_validation_mx_orders(fn):
    """MN-contiguous block-scaled operands: leading dimension against M (N);
    every case is refused before anything is launched."""
    assert callmx(fn, M=-1) == INVALID_SIZE
    assert callmx(fn, M=0) == OK
    assert callmx(fn, ao=2) == UNSUPPORTED
    assert callmx(fn, bo=-1) == UNSUPPORTED
    assert callmx(fn, lda=252) == BAD_LD                  # A stored K x M: lda >= M
    assert callmx(fn, ao=0, bo=1, lda=512, ldb=188) == BAD_LD
    assert callmx(fn, ldb=508) == BAD_LD                  # B K-contiguous: ldb >= K
    assert callmx(fn, SFA=None) == NULL_POINTER
    assert callmx(fn, ldsfa=15) == BAD_LD
    assert callmx(fn, K=48) == UNSUPPORTED                # K % 32
    if fn != "gemm_mxfp8_ex":
        assert callmx(fn, lda=257 if fn == "gemm_mxfp4_ex" else 258) == UNSUPPORTED   # whole-byte rows
    if fn == "gemm_mxfp6_ex":
        assert callmx(fn, fmt=7) == UNSUPPORTED


def callx(fn="gemm_bf16_ex", M=256, N=256, K=512, A=P, lda=256, ao=1, B=P, ldb=512, bo=0, C=None, ldc=0,
          D=P + (1 << 24), ldd=256, out=F32):
    return getattr(tg.raw, fn)(M, N, K, A, lda, ao, B, ldb, bo, C, ldc, D, ldd, out, None)


@pytest.mark.parametrize("fn", ["gemm_bf16_ex", "gemm_fp16_ex"])
def test_validation_orders(fn):
    """MN-contiguous operands: leading dimension against M (N); every case is
    refused before anything is launched."""
    assert callx(fn, M=-1) == INVALID_SIZE
    assert callx(fn, M=0) == OK
    assert callx(fn, ao=2) == UNSUPPORTED
    assert callx(fn, bo=-1) == UNSUPPORTED
    assert callx(fn, lda=255) == BAD_LD                        # A stored K x M: lda >= M
    assert callx(fn, ao=0, lda=511, bo=1, ldb=256) == BAD_LD   # A K-contiguous: lda >= K
    assert callx(fn, bo=1, ldb=255) == BAD_LD                  # B stored K x N: ldb >= N
    assert callx(fn, lda=260) == UNSUPPORTED                   # rows not 16-byte multiples
    assert callx(fn, K=500, ldb=504) == UNSUPPORTED            # K-contiguous B with K % 8 != 0
    assert callx(fn, A=P + 8) == UNSUPPORTED                   # A not 16-byte aligned
    assert callx(fn, A=P + 1) == MISALIGNED
    assert callx(fn, D=None) == NULL_POINTER
    assert callx(fn, lda=8 << 20) == UNSUPPORTED               # 16 MiB rows


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(tg, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(tg, "_lib", None)
    with pytest.raises(tg.LibraryMissing):
        tg.raw.gemm_bf16


class _FakeDevice:
    """A host tensor that reports itself as living on cuda:0, so the
    binding's argument checks can be driven without a GPU.  The checks under
    test must raise before any pointer reaches the library."""

    def __init__(self, t):
        import torch
        self._t, self.is_cuda, self.device = t, True, torch.device("cuda", 0)

    def __getattr__(self, name):
        return getattr(self._t, name)


@pytest.mark.parametrize("which", ["C", "D"])
def test_binding_rejects_host_c_and_d(which):
    import torch
    A = _FakeDevice(torch.zeros(8, 16, dtype=torch.bfloat16))
    B = _FakeDevice(torch.zeros(4, 16, dtype=torch.bfloat16))
    host = torch.zeros(8, 4)
    dev = _FakeDevice(torch.zeros(8, 4))
    kw = {"C": host, "D": dev} if which == "C" else {"C": None, "D": host}
    for fn in (tg.gemm_bf16, tg.gemm_bf16_splitk):
        with pytest.raises(ValueError, match=which):
            fn(A, B, **kw)
    A8 = _FakeDevice(torch.zeros(8, 64, dtype=torch.uint8))
    B8 = _FakeDevice(torch.zeros(4, 64, dtype=torch.uint8))
    SFA = _FakeDevice(torch.full((8, 2), 127, dtype=torch.uint8))
    SFB = _FakeDevice(torch.full((4, 2), 127, dtype=torch.uint8))
    for order in ("k", "mn"):
        Ao = A8 if order == "k" else _FakeDevice(torch.zeros(64, 8, dtype=torch.uint8))
        with pytest.raises(ValueError, match=which):
            tg.gemm_mxfp8(Ao, SFA, B8, SFB, a_order=order, **kw)


def test_binding_rejects_host_workspace_and_scales():
    import torch
    A = _FakeDevice(torch.zeros(256, 8192, dtype=torch.bfloat16))
    B = _FakeDevice(torch.zeros(256, 8192, dtype=torch.bfloat16))
    D = _FakeDevice(torch.zeros(256, 256))
    with pytest.raises(ValueError, match="workspace"):
        tg.gemm_bf16_splitk(A, B, D=D, splits=4, workspace=torch.zeros(1 << 24, dtype=torch.uint8))
    A8 = _FakeDevice(torch.zeros(8, 64, dtype=torch.uint8))
    B8 = _FakeDevice(torch.zeros(4, 64, dtype=torch.uint8))
    D8 = _FakeDevice(torch.zeros(8, 4))
    with pytest.raises(ValueError):
        tg.gemm_mxfp8(A8, torch.full((8, 2), 127, dtype=torch.uint8), B8,
                      _FakeDevice(torch.full((4, 2), 127, dtype=torch.uint8)), D=D8)


def test_noalloc_splitk_validation_and_limit():
    """The allocation-free split-K entry point validates like gemm_bf16_splitk
    and refuses partials beyond its static scratch area before any GPU call."""
    f = tg.raw.gemm_bf16_splitk_noalloc
    D = P + (1 << 24)
    call = lambda M=1024, N=1024, K=65536, lda=65536, ldb=65536, splits=16, out=F32, A=P, B=P: \
        f(M, N, K, A, lda, B, ldb, None, 0, D, N, out, splits, None)
    assert tg.raw.gemm_splitk_scratch_limit() == 64 << 20
    assert call(M=-1) == INVALID_SIZE
    assert call(lda=100) == BAD_LD
    assert call(A=None) == NULL_POINTER
    assert call(A=P + 1) == MISALIGNED
    assert call(splits=65) == UNSUPPORTED
    assert call(out=3) == UNSUPPORTED
    assert call(M=0) == OK
    # 4096 x 4096 in 64 ranges: 4 GiB of partials
    assert call(M=4096, N=4096, splits=64) == 8
    assert tg.raw.status_string(8).startswith("GEMM_ERR_SCRATCH_LIMIT")
    # 1024 x 1024 in 17 ranges: 68 MiB, one range past the 64 MiB area
    assert call(splits=17) == 8


def test_validation_mx_kblock():
    """Wide scale blocks: block width, scale leading dimensions and element
    packing are checked before any GPU call."""
    f = tg.raw.gemm_mx_kblock
    D = P + (1 << 24)

    def call(fmt=0, M=64, N=64, K=256, kb=64, lda=256, ldsfa=4, ldb=256, ldsfb=4, SFA=P + 4096, out=F32):
        return f(fmt, M, N, K, kb, P, lda, SFA, ldsfa, P, ldb, P + 8192, ldsfb, None, 0, D, N, out, None)
    for bad_kb in (0, 16, 48, -32):
        assert call(kb=bad_kb) == UNSUPPORTED
    assert call(fmt=4) == UNSUPPORTED
    assert call(ldsfa=3) == BAD_LD                     # ceil(256 / 64) = 4 scales per row
    assert call(kb=96, ldsfa=3, ldsfb=3) == UNSUPPORTED  # not 32 times a power of two, below K
    assert call(kb=288, ldsfa=0, ldsfb=1) == BAD_LD   # >= K: one scale per row
    assert call(kb=512, ldsfa=1, ldsfb=1, SFA=None) == NULL_POINTER
    assert call(K=48) == UNSUPPORTED                   # K % 32
    assert call(fmt=1, lda=255) == UNSUPPORTED         # fp4 rows of whole bytes
    assert call(fmt=2, lda=254) == UNSUPPORTED         # fp6 rows of whole byte groups
    assert call(lda=100) == BAD_LD
    assert call(M=0) == OK
    assert call(M=-1) == INVALID_SIZE


def test_validation_mx_kblock_ws():
    """The replicated-scale path checks everything, its workspace included,
    before launching anything (no GPU call: every case below fails a check
    or has nothing to do)."""
    f = tg.raw.gemm_mx_kblock_ws
    D = P + (1 << 24)
    WS = P + (1 << 26)

    def call(fmt=0, M=64, N=64, K=256, kb=64, lda=256, ldsfa=4, ldb=256, ldsfb=4, out=F32, ws=WS, wsb=1 << 20,
             ldd=64):
        return f(fmt, M, N, K, kb, P, lda, P + 4096, ldsfa, P, ldb, P + 8192, ldsfb, None, 0, D, ldd, out, ws, wsb,
                 None)
    need = tg.raw.gemm_mx_kblock_workspace_bytes(64, 64, 256)
    assert need == 128 * 16                            # 8 scale bytes per row rounded up to 16
    assert tg.raw.gemm_mx_kblock_workspace_bytes(3, 5, 1024) == 8 * 32
    assert tg.raw.gemm_mx_kblock_workspace_bytes(-1, 5, 1024) == 0
    assert call(wsb=need - 1) == WORKSPACE
    assert call(ws=WS + 64) == MISALIGNED
    # the operand and scale checks come first, as in gemm_mx_kblock
    assert call(kb=96, ldsfa=3, ldsfb=3) == UNSUPPORTED
    assert call(ldsfa=3) == BAD_LD
    assert call(lda=100) == BAD_LD
    assert call(ldd=32) == BAD_LD
    assert call(fmt=1, lda=255) == UNSUPPORTED
    assert call(M=0, wsb=0) == OK
    assert call(M=-1) == INVALID_SIZE


def test_validation_ex_ws():
    """*_ex_ws: the _ex call's checks, then the workspace's, before any GPU
    call (every case below fails a check or has nothing to do)."""
    D = P + (1 << 24)
    WS = P + (1 << 26)
    MN, KC = 1, 0
    f16 = tg.raw.gemm_bf16_ex_ws
    mx8 = tg.raw.gemm_mxfp8_ex_ws

    def c16(M=300, N=200, K=130, lda=300, ao=MN, ldb=130, bo=KC, ws=WS, wsb=1 << 24, ldd=200):
        return f16(M, N, K, P, lda, ao, P, ldb, bo, None, 0, D, ldd, F32, ws, wsb, None)

    def c8(M=300, N=200, K=256, lda=300, ao=MN, ldb=256, bo=KC, ws=WS, wsb=1 << 24, ldsfa=8):
        return mx8(M, N, K, P, lda, ao, P + 4096, ldsfa, P, ldb, bo, P + 8192, 8, None, 0, D, N, F32, ws, wsb, None)
    # sizes: rows of K rounded up to 1024 / bits elements (fp6 192), each
    # copy rounded to 256 bytes
    assert tg.raw.gemm_ex_workspace_bytes(16, 300, 200, 130, MN, KC) == (300 * 192 * 2 + 255) // 256 * 256
    assert tg.raw.gemm_ex_workspace_bytes(8, 300, 200, 256, MN, MN) == 300 * 256 + 200 * 256
    assert tg.raw.gemm_ex_workspace_bytes(6, 64, 64, 128, KC, MN) == 64 * 144
    assert tg.raw.gemm_ex_workspace_bytes(4, 64, 64, 128, MN, KC) == 64 * 128
    assert tg.raw.gemm_ex_workspace_bytes(4, 64, 64, 128, KC, KC) == 0
    # fp6, both K-contiguous: the tile images of A and of B (2 x 2 and 1 x 2
    # images of 24576 bytes), none when K % 128 != 0
    assert tg.raw.gemm_ex_workspace_bytes(6, 300, 200, 256, KC, KC) == (4 + 2) * 24576
    assert tg.raw.gemm_ex_workspace_bytes(6, 300, 200, 96, KC, KC) == 0
    assert tg.raw.gemm_ex_workspace_bytes(5, 64, 64, 128, MN, MN) == 0
    need16 = tg.raw.gemm_ex_workspace_bytes(16, 300, 200, 130, MN, KC)
    assert c16(wsb=need16 - 1) == WORKSPACE
    assert c16(ws=WS + 16) == MISALIGNED
    assert c16(lda=299) == BAD_LD                      # MN-contiguous A: lda >= M
    assert c16(ldd=100) == BAD_LD
    assert c16(ao=2) == UNSUPPORTED
    assert c16(M=0, wsb=0) == OK
    need8 = tg.raw.gemm_ex_workspace_bytes(8, 300, 200, 256, MN, KC)
    assert c8(wsb=need8 - 1) == WORKSPACE
    assert c8(ws=WS + 128) == MISALIGNED
    assert c8(ldsfa=7) == BAD_LD                       # scale rows as the plain call
    assert c8(K=48) == UNSUPPORTED
    assert c8(M=-1) == INVALID_SIZE


def test_validation_mxfp6_packed():
    """fp6 tile images: the size rule, and every refused pack or GEMM case
    checked before anything is launched (no GPU call: each case below fails
    a check or has nothing to do)."""
    nbytes = tg.raw.gemm_mxfp6_packed_bytes
    # ceil(rows / 256) row blocks x K / 128 tiles x 24576 bytes
    assert nbytes(256, 128) == 24576
    assert nbytes(257, 512) == 2 * 4 * 24576
    assert nbytes(1, 8192) == 64 * 24576
    assert nbytes(0, 128) == 0 and nbytes(300, 0) == 0
    assert nbytes(300, 96) == 0 and nbytes(-1, 128) == 0 and nbytes(4, 1 << 23) == 0

    def pack(rows=300, K=256, X=P, ldx=256, dst=P + (1 << 26), nb=None):
        if nb is None:
            nb = nbytes(rows, K)
        return tg.raw.gemm_mxfp6_pack(rows, K, X, ldx, dst, nb, None)
    assert pack(rows=-1) == INVALID_SIZE
    assert pack(K=-128) == INVALID_SIZE
    assert pack(K=96, ldx=96) == UNSUPPORTED               # K % 128 != 0
    assert pack(K=1 << 23, ldx=1 << 23, nb=1 << 40) == UNSUPPORTED
    assert pack(ldx=258) == UNSUPPORTED                    # rows must start on a byte
    assert pack(ldx=252) == BAD_LD
    assert pack(X=None) == NULL_POINTER
    assert pack(dst=None) == NULL_POINTER
    assert pack(dst=P + 8) == MISALIGNED
    assert pack(nb=nbytes(300, 256) - 1) == WORKSPACE
    assert pack(rows=0) == OK and pack(K=0, ldx=0) == OK

    D = P + (1 << 24)

    def gemm(M=300, N=200, K=256, AP=P, BP=P + (1 << 22), SFA=P + 4096, ldsfa=16, SFB=P + 8192, ldsfb=16,
             ldd=200, fmt=0, out=F32, C=None, ldc=0):
        return tg.raw.gemm_mxfp6_packed(M, N, K, AP, SFA, ldsfa, BP, SFB, ldsfb, C, ldc, D, ldd, fmt, out, None)
    assert gemm(M=-1) == INVALID_SIZE
    assert gemm(M=0) == OK
    assert gemm(fmt=2) == UNSUPPORTED
    assert gemm(out=3) == UNSUPPORTED
    assert gemm(K=96) == UNSUPPORTED                       # K % 128 != 0
    assert gemm(K=1 << 23, ldsfa=1 << 18, ldsfb=1 << 18) == UNSUPPORTED
    assert gemm(AP=P + 4) == MISALIGNED
    assert gemm(BP=P + 8) == MISALIGNED
    assert gemm(ldsfa=4) == BAD_LD                         # K / 32 = 8 scales per row
    assert gemm(SFB=None) == NULL_POINTER
    assert gemm(AP=None) == NULL_POINTER
    assert gemm(ldsfa=24) == UNSUPPORTED                   # scale rows of whole 16-byte words
    assert gemm(SFA=P + 4100) == UNSUPPORTED
    assert gemm(ldd=100) == BAD_LD
    assert gemm(C=D, ldc=100) == BAD_LD


def test_validation_mxfp6_ex_ws_images():
    """gemm_mxfp6_ex_ws with K-contiguous operands and a workspace for their
    tile images: the plain call's checks come first (nothing launched)."""
    D = P + (1 << 24)
    WS = P + (1 << 26)
    KC = 0

    def call(M=300, N=200, K=256, lda=256, ldb=256, ldsfa=16, ldsfb=16, ldd=200, fmt=0):
        return tg.raw.gemm_mxfp6_ex_ws(M, N, K, P, lda, KC, P + 4096, ldsfa, P, ldb, KC, P + 8192, ldsfb, None, 0,
                                       D, ldd, fmt, F32, WS, 1 << 24, None)
    assert call(ldsfa=4) == BAD_LD
    assert call(lda=252) == BAD_LD
    assert call(ldd=100) == BAD_LD
    assert call(fmt=2) == UNSUPPORTED
    assert call(M=-1) == INVALID_SIZE
    assert call(M=0) == OK
