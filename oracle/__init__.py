"""Oracle for the tiled matrix multiply-accumulate D = A.B + C.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and never imports it.

What the operation is (the pages' definition, restated):

* "Tensor Core 数据布局的演进" (Evolution of Tensor Core data layouts),
  section 概览: D = AB + C, where A and B are multiplied and C is the incoming
  accumulator.
* same page, section 一个具体的 fragment 映射: A row-major, B column-major,
  fp16/bf16 inputs, fp32 C and D.  B column-major is stored here as N rows of
  K (``b(k, n) = B[n, k]``).
* same page, section Block-Scaled MMA 的 Scale Factors: ``SFA[m, sfk]`` scales
  K block ``sfk`` of row m of A, ``SFB[n, sfk]`` scales column n of B; every K
  element of a block shares its scale.  Block width 32, e8m0 scales.

Contents:

* :func:`gemm_ref` -- the naive fp64 triple loop in plain C (``oracle.c``),
  one element at a time, k ascending.  Pinned by the ``not gpu`` tests against
  exact rational arithmetic, closed forms and exhaustive decoder tables.
* :func:`gemm_ref_full` -- the same definition over whole matrices with a
  numpy float64 matmul as the one library step (used to check every element
  of mid-sized outputs quickly).  Pinned against :func:`gemm_ref`.
* :func:`rne_bf16` -- binary64 -> bf16 round-to-nearest-even (``oracle.c``).
* the checker, tiling, prefetch-ring and LDS-bank models in the submodules.

Parity status: every function here has at least one pin in
``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# element type codes, mirrored from oracle.c
BF16, FP16, E4M3, F32, E2M1, E2M3, E3M2 = 0, 1, 2, 3, 4, 5, 6
TYPE_CODES = {"bf16": BF16, "fp16": FP16, "e4m3": E4M3, "f32": F32, "e2m1": E2M1, "e2m3": E2M3, "e3m2": E3M2}
FP6 = ("e2m3", "e3m2")

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain -O2, OpenMP, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
           "-shared", "-fPIC", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    """Load liboracle.so (building it first only if it is missing or stale)."""
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            L = ctypes.CDLL(_LIB_PATH)
            i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
            L.oracle_gemm.restype = ctypes.c_int
            L.oracle_gemm.argtypes = [ctypes.c_int, i64, i64, i64,
                                      vp, i64, vp, i64,
                                      vp, i64, vp, i64,
                                      ctypes.c_int, vp, i64,
                                      i64, vp, dp, dp, ctypes.c_int, i64]
            for name, arg in (("orc_dec_bf16", ctypes.c_uint16), ("orc_dec_fp16", ctypes.c_uint16),
                              ("orc_dec_e4m3", ctypes.c_uint8), ("orc_dec_e8m0", ctypes.c_uint8),
                              ("orc_dec_e2m1", ctypes.c_uint8),
                              ("orc_dec_e2m3", ctypes.c_uint8),
                              ("orc_dec_e3m2", ctypes.c_uint8),
                              ("orc_dec_f32", ctypes.c_uint32)):
                f = getattr(L, name)
                f.restype = ctypes.c_double
                f.argtypes = [arg]
            L.orc_rne_bf16.restype = ctypes.c_uint16
            L.orc_rne_bf16.argtypes = [ctypes.c_double]
            L.orc_rne_bf16_f32_array.restype = None
            L.orc_rne_bf16_f32_array.argtypes = [vp, vp, i64]
            L.oracle_num_threads.restype = ctypes.c_int
            L.oracle_num_threads.argtypes = []
            _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


_ERRS = {-1: "bad argument", -2: "NaN e8m0 scale code (0xFF)",
         -3: "scaled form needs K % 32 == 0 and a scale block width that is a multiple of 32"}


def _ptr(a):
    return None if a is None else a.ctypes.data


def gemm_ref(in_type: str, A, B, K: int | None = None, C=None, c_type: str = "f32",
             SFA=None, SFB=None, idx=None, nthreads: int = 0, kblock: int = 32):
    """D_ref and S = sum_k |a*b| at the requested elements, in float64.

    ``A``: (M, lda) raw element bits (uint16 for bf16/fp16, uint8 for e4m3),
    row-major; for e2m1 (M, lda / 2) bytes, two elements per byte (element
    2i in the low nibble of byte i); ``B``: (N, ldb) raw bits, row n holds
    column n of the K x N operand; ``K`` (elements) defaults to the row
    length.  ``C``: (M, ldc) float32 array
    (``c_type='f32'``) or uint16 bf16 bits (``c_type='bf16'``), or None.
    ``SFA``/``SFB``: (M, ldsfa) / (N, ldsfb) uint8 e8m0 codes, both or neither;
    ``kblock``: the scale block's width in K elements (a multiple of 32;
    the standard form is 32), scale j of a row covering K elements
    [j kblock, (j + 1) kblock).
    ``idx``: flat indices ``m*N + n`` (None: every element, row-major).

    Returns ``(D, S)`` float64 arrays of shape ``idx.shape`` (or (M, N)).
    """
    L = lib()
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    M, lda = A.shape
    N, ldb = B.shape
    if in_type == "e2m1":                       # leading dimensions in elements
        lda, ldb = 2 * lda, 2 * ldb
    elif in_type in FP6:
        if lda % 3 or ldb % 3:
            raise ValueError("fp6 rows are whole groups of three bytes")
        lda, ldb = lda // 3 * 4, ldb // 3 * 4
    if K is None:
        K = lda
    if K > lda or K > ldb:
        raise ValueError("K exceeds a leading dimension")
    if C is not None:
        C = np.ascontiguousarray(C)
        if c_type == "f32":
            C = C.astype(np.float32, copy=False)
        ldc = C.shape[1]
    else:
        ldc = 0
    ldsfa = ldsfb = 0
    if SFA is not None:
        SFA = np.ascontiguousarray(SFA, dtype=np.uint8)
        SFB = np.ascontiguousarray(SFB, dtype=np.uint8)
        ldsfa, ldsfb = SFA.shape[1], SFB.shape[1]
    if idx is None:
        n_out = M * N
        idx_arr = None
        out_shape = (M, N)
    else:
        idx_arr = np.ascontiguousarray(idx, dtype=np.int64)
        n_out = idx_arr.size
        out_shape = idx_arr.shape
    D = np.empty(n_out, dtype=np.float64)
    S = np.empty(n_out, dtype=np.float64)
    rc = L.oracle_gemm(TYPE_CODES[in_type], M, N, K,
                       _ptr(A), lda, _ptr(SFA), ldsfa,
                       _ptr(B), ldb, _ptr(SFB), ldsfb,
                       TYPE_CODES[c_type], _ptr(C), ldc,
                       n_out, _ptr(idx_arr), _ptr(D), _ptr(S), int(nthreads), int(kblock))
    if rc != 0:
        raise OracleError(_ERRS.get(rc, "error %d" % rc))
    return D.reshape(out_shape), S.reshape(out_shape)


# ---- decoders (each a thin call of the C definition) -----------------------

def dec_bf16(bits: int) -> float:
    return lib().orc_dec_bf16(int(bits))


def dec_fp16(bits: int) -> float:
    return lib().orc_dec_fp16(int(bits))


def dec_e4m3(bits: int) -> float:
    return lib().orc_dec_e4m3(int(bits))


def dec_e2m1(bits: int) -> float:
    return lib().orc_dec_e2m1(int(bits))


def dec_e2m3(bits: int) -> float:
    return lib().orc_dec_e2m3(int(bits))


def dec_e3m2(bits: int) -> float:
    return lib().orc_dec_e3m2(int(bits))


def unpack_fp6(packed) -> np.ndarray:
    """(R, 3n) bytes of packed fp6 -> (R, 4n) six-bit codes, element k at
    bits 6k .. 6k+5 of the row read as a little-endian bit string."""
    p = np.asarray(packed, dtype=np.uint8)
    g = p.reshape(p.shape[:-1] + (-1, 3)).astype(np.uint32)
    w = g[..., 0] | (g[..., 1] << 8) | (g[..., 2] << 16)      # 24 bits: four elements
    out = np.empty(p.shape[:-1] + (g.shape[-2], 4), dtype=np.uint8)
    for j in range(4):
        out[..., j] = (w >> (6 * j)) & 0x3F
    return out.reshape(p.shape[:-1] + (-1,))


def unpack_e2m1(packed) -> np.ndarray:
    """(R, n) bytes of packed e2m1 -> (R, 2n) codes, element 2i from the low nibble of byte i."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def dec_e8m0(bits: int) -> float:
    return lib().orc_dec_e8m0(int(bits))


def dec_f32(bits: int) -> float:
    return lib().orc_dec_f32(int(bits))


_TABLES: dict = {}


def decode_table(in_type: str) -> np.ndarray:
    """Full lookup table code -> float64 built from the C decoders."""
    if in_type not in _TABLES:
        f = {"bf16": dec_bf16, "fp16": dec_fp16, "e4m3": dec_e4m3, "e8m0": dec_e8m0, "e2m1": dec_e2m1,
             "e2m3": dec_e2m3, "e3m2": dec_e3m2}[in_type]
        n = {"e4m3": 256, "e8m0": 256, "e2m1": 16, "e2m3": 64, "e3m2": 64}.get(in_type, 65536)
        _TABLES[in_type] = np.array([f(i) for i in range(n)], dtype=np.float64)
    return _TABLES[in_type]


def decode(in_type: str, bits) -> np.ndarray:
    """Decode an array of raw codes to float64 with the C decoders' tables."""
    return decode_table(in_type)[np.asarray(bits)]


def rne_bf16(x) -> np.ndarray:
    """Round float64 values to bf16 bits, nearest-even (vectorised over the C routine)."""
    f = lib().orc_rne_bf16
    x = np.asarray(x, dtype=np.float64)
    out = np.fromiter((f(float(v)) for v in x.ravel()), dtype=np.uint16, count=x.size)
    return out.reshape(x.shape)


def rne_bf16_f32(x) -> np.ndarray:
    """Round a float32 array to bf16 bits, nearest-even (C loop, OpenMP)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_rne_bf16_f32_array(x.ctypes.data, out.ctypes.data, x.size)
    return out


def num_threads() -> int:
    """Threads one oracle call runs on."""
    return lib().oracle_num_threads()


# ---- whole-matrix form with a library matmul as its one step --------------

def operands_f64(in_type: str, A, B, K=None, SFA=None, SFB=None, kblock=32):
    """Decoded, scaled operands a(m,k) (M x K) and b(k,n) stored as (N x K), float64."""
    A = np.asarray(A)
    B = np.asarray(B)
    if in_type == "e2m1":
        A, B = unpack_e2m1(A), unpack_e2m1(B)
    elif in_type in FP6:
        A, B = unpack_fp6(A), unpack_fp6(B)
    if K is None:
        K = A.shape[1]
    a = decode(in_type, A[:, :K])
    b = decode(in_type, B[:, :K])
    if SFA is not None:
        blk = np.arange(K) // kblock
        a = a * decode("e8m0", np.asarray(SFA)[:, blk])
        b = b * decode("e8m0", np.asarray(SFB)[:, blk])
    return a, b


def c_f64(C, c_type="f32"):
    if C is None:
        return None
    if c_type == "f32":
        return np.asarray(C, dtype=np.float32).astype(np.float64)
    return decode("bf16", C)


def gemm_ref_full(in_type: str, A, B, K=None, C=None, c_type="f32", SFA=None, SFB=None,
                  rows=None, kblock=32):
    """(D_ref, S) for every element (or for the given rows) via numpy float64 matmul.

    Same definition as :func:`gemm_ref`; the sum over k is a BLAS float64
    product, whose rounding (at most about K * 2^-53 * S) is far below every
    tolerance used here.
    """
    a, b = operands_f64(in_type, A, B, K, SFA, SFB, kblock)
    if rows is not None:
        a = a[rows]
    D = a @ b.T
    S = np.abs(a) @ np.abs(b).T
    c = c_f64(C, c_type)
    if c is not None:
        c = c[:, : b.shape[0]]
        D = D + (c[rows] if rows is not None else c)
    return D, S
