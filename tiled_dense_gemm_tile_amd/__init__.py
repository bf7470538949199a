"""tiled_dense_gemm_tile_amd -- D = A.B + C on MI355X (gfx950).

Thin Python binding of ``libtilegemm.so`` (the C ABI in ``include/tilegemm.h``).
It only marshals arguments: every step of the operation runs in the HIP
kernels.  PyTorch supplies device memory and the stream.  When the library is
not built the calls raise :class:`LibraryMissing`; there is no fallback.

Tensor conventions (same as the C ABI):
  A: (M, K);  B: (N, K), i.e. the K x N operand indexed [n, k];  C, D: (M, N)
  row-major.  C and D need a last stride of 1 (the first stride is the
  leading dimension).  For the 16-bit calls A and B may each be K-contiguous
  (last stride 1) or MN-contiguous (first stride 1, e.g. ``X.t()`` of a
  contiguous K x M or K x N tensor); the binding passes the storage order to
  ``gemm_bf16_ex`` / ``gemm_fp16_ex`` when one is MN-contiguous.
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = ["gemm_bf16", "gemm_fp16", "gemm_bf16_splitk", "gemm_fp16_splitk", "splitk_workspace_bytes",
           "gemm_mxfp8", "gemm_mxfp4", "gemm_mxfp6", "gemm_mxfp8_splitk", "gemm_mxfp4_splitk", "gemm_mxfp6_splitk", "raw", "GemmError", "LibraryMissing",
           "library_path", "STATUS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libtilegemm.so")

STATUS = {0: "GEMM_OK", 1: "GEMM_ERR_INVALID_SIZE", 2: "GEMM_ERR_NULL_POINTER", 3: "GEMM_ERR_BAD_LD",
          4: "GEMM_ERR_MISALIGNED", 5: "GEMM_ERR_UNSUPPORTED", 6: "GEMM_ERR_HIP", 7: "GEMM_ERR_WORKSPACE",
          8: "GEMM_ERR_SCRATCH_LIMIT"}
OUT_F32, OUT_BF16 = 0, 1


class LibraryMissing(RuntimeError):
    pass


class GemmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lock = threading.Lock()
_lib = None


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise LibraryMissing("libtilegemm.so is not built (run __graft_entry__.build()); "
                                     "there is no fallback path")
            L = ctypes.CDLL(_LIB_PATH)
            i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
            sig16 = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, ci, vp]
            for name in ("gemm_bf16", "gemm_fp16"):
                f = getattr(L, name)
                f.restype, f.argtypes = ci, sig16
            for name in ("gemm_bf16_ex", "gemm_fp16_ex"):
                f = getattr(L, name)
                f.restype, f.argtypes = ci, [i64, i64, i64, vp, i64, ci, vp, i64, ci, vp, i64, vp, i64, ci, vp]
            sz = ctypes.c_size_t
            for name in ("gemm_bf16_splitk", "gemm_fp16_splitk"):
                f = getattr(L, name)
                f.restype, f.argtypes = ci, sig16[:-1] + [ci, vp, sz, vp]
            L.gemm_bf16_splitk_noalloc.restype = ci
            L.gemm_bf16_splitk_noalloc.argtypes = sig16[:-1] + [ci, vp]
            L.gemm_splitk_scratch_limit.restype = sz
            L.gemm_splitk_scratch_limit.argtypes = []
            L.gemm_splitk_workspace_bytes.restype = sz
            L.gemm_splitk_workspace_bytes.argtypes = [i64, i64, i64, ci]
            for name in ("gemm_mxfp8", "gemm_mxfp4"):
                f = getattr(L, name)
                f.restype = ci
                f.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, ci, vp]
            L.gemm_mxfp6.restype = ci
            L.gemm_mxfp6.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, ci, ci, vp]
            smx = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64]
            for name in ("gemm_mxfp8_splitk", "gemm_mxfp4_splitk"):
                f = getattr(L, name)
                f.restype, f.argtypes = ci, smx + [ci, ci, vp, sz, vp]
            L.gemm_mxfp6_splitk.restype = ci
            L.gemm_mxfp6_splitk.argtypes = smx + [ci, ci, ci, vp, sz, vp]
            sex = [i64, i64, i64, vp, i64, ci, vp, i64, vp, i64, ci, vp, i64, vp, i64, vp, i64]
            for name in ("gemm_mxfp8_ex", "gemm_mxfp4_ex"):
                f = getattr(L, name)
                f.restype, f.argtypes = ci, sex + [ci, vp]
            L.gemm_mxfp6_ex.restype = ci
            L.gemm_mxfp6_ex.argtypes = sex + [ci, ci, vp]
            for name in ("gemm_bf16_ex_ws", "gemm_fp16_ex_ws"):
                f = getattr(L, name)
                f.restype, f.argtypes = ci, [i64, i64, i64, vp, i64, ci, vp, i64, ci, vp, i64, vp, i64, ci, vp, sz, vp]
            for name in ("gemm_mxfp8_ex_ws", "gemm_mxfp4_ex_ws"):
                f = getattr(L, name)
                f.restype, f.argtypes = ci, sex + [ci, vp, sz, vp]
            L.gemm_mxfp6_ex_ws.restype = ci
            L.gemm_mxfp6_ex_ws.argtypes = sex + [ci, ci, vp, sz, vp]
            L.gemm_ex_workspace_bytes.restype = sz
            L.gemm_ex_workspace_bytes.argtypes = [ci, i64, i64, i64, ci, ci]
            L.gemm_mx_kblock.restype = ci
            L.gemm_mx_kblock.argtypes = [ci, i64, i64, i64, i64] + smx[3:] + [ci, vp]
            L.gemm_mx_kblock_ws.restype = ci
            L.gemm_mx_kblock_ws.argtypes = [ci, i64, i64, i64, i64] + smx[3:] + [ci, vp, sz, vp]
            L.gemm_mx_kblock_workspace_bytes.restype = sz
            L.gemm_mx_kblock_workspace_bytes.argtypes = [i64, i64, i64]
            L.gemm_mxfp6_packed_bytes.restype = sz
            L.gemm_mxfp6_packed_bytes.argtypes = [i64, i64]
            L.gemm_mxfp6_pack.restype = ci
            L.gemm_mxfp6_pack.argtypes = [i64, i64, vp, i64, vp, sz, vp]
            L.gemm_mxfp6_packed.restype = ci
            L.gemm_mxfp6_packed.argtypes = [i64, i64, i64, vp, vp, i64, vp, vp, i64, vp, i64, vp, i64, ci, ci, vp]
            L.gemm_status_string.restype = ctypes.c_char_p
            L.gemm_status_string.argtypes = [ci]
            L.gemm_last_hip_error.restype = ci
            L.gemm_last_hip_error.argtypes = []
            _lib = L
    return _lib


class _Raw:
    """Direct C-ABI calls with integer pointers; each returns the gemm_status."""

    def __getattr__(self, name):
        return getattr(_load(), name)

    def status_string(self, s: int) -> str:
        return _load().gemm_status_string(int(s)).decode()


raw = _Raw()


def _check(status: int):
    if status != 0:
        L = _load()
        msg = L.gemm_status_string(status).decode()
        if status == 6:
            msg += " (hipError_t %d)" % L.gemm_last_hip_error()
        raise GemmError(status, msg)


def _ld(t, cols):
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("the last stride must be 1")
    if t.shape[0] <= 1:
        return max(cols, t.stride(0) if t.shape[0] == 1 else 0)
    return t.stride(0)


def _on_device(ref, **tensors):
    """Raise unless every given tensor lives on ``ref``'s GPU: a host tensor's
    data_ptr() handed to a kernel would be an address the GPU cannot map."""
    for name, t in tensors.items():
        if t is not None and (not t.is_cuda or t.device != ref.device):
            raise ValueError("%s must be a device tensor on %s" % (name, ref.device))


def _prep(A, B, C, D, out_dtype, in_dtypes):
    import torch
    if A.dtype not in in_dtypes or B.dtype not in in_dtypes:
        raise TypeError("A and B must be %s" % (in_dtypes,))
    if not (A.is_cuda and B.is_cuda):
        raise ValueError("A and B must be device tensors")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("B must be (N, K) with K = A.shape[1]")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    if D is None:
        D = torch.empty((M, N), dtype=out_dtype, device=A.device)
    if D.dtype != out_dtype or tuple(D.shape) != (M, N):
        raise ValueError("D must be (M, N) of out_dtype")
    if C is not None and (C.dtype != out_dtype or tuple(C.shape) != (M, N)):
        raise ValueError("C must be (M, N) of out_dtype")
    _on_device(A, B=B, C=C, D=D)
    out = OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32
    return M, N, K, D, _Stream(A), out


class _Stream:
    """torch's current stream on A's device, looked up when the call is
    marshalled (after every argument check), as a ctypes argument."""

    def __init__(self, A):
        self._dev = A.device

    @property
    def _as_parameter_(self):
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream(self._dev).cuda_stream)


K_CONTIGUOUS, MN_CONTIGUOUS = 0, 1


def _order(t):
    """(storage order, leading dimension) of a 2-D operand viewed (rows, K)."""
    rows, cols = t.shape
    if cols <= 1 or t.stride(1) == 1:
        return K_CONTIGUOUS, _ld(t, cols)
    if rows <= 1 or t.stride(0) == 1:
        return MN_CONTIGUOUS, max(t.stride(1), rows)
    raise ValueError("each operand needs a unit stride along K or along M/N")


def _call16(name, A, B, C, out_dtype, D, dtype, workspace=None):
    _on_device(A, workspace=workspace)
    M, N, K, D, stream, out = _prep(A, B, C, D, out_dtype, (dtype,))
    (ao, lda), (bo, ldb) = _order(A), _order(B)
    if not K:
        ao, lda, bo, ldb = K_CONTIGUOUS, 0, K_CONTIGUOUS, 0
    cptr, ldc = (C.data_ptr(), _ld(C, N)) if C is not None else (None, 0)
    L = _load()
    if ao == K_CONTIGUOUS and bo == K_CONTIGUOUS:
        st = getattr(L, name)(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, cptr, ldc, D.data_ptr(), _ld(D, N),
                              out, stream)
    elif workspace is None:
        st = getattr(L, name + "_ex")(M, N, K, A.data_ptr(), lda, ao, B.data_ptr(), ldb, bo, cptr, ldc,
                                      D.data_ptr(), _ld(D, N), out, stream)
    else:
        st = getattr(L, name + "_ex_ws")(M, N, K, A.data_ptr(), lda, ao, B.data_ptr(), ldb, bo, cptr, ldc,
                                         D.data_ptr(), _ld(D, N), out, workspace.data_ptr(),
                                         workspace.numel() * workspace.element_size(), stream)
    _check(st)
    return D


def gemm_bf16(A, B, C=None, out_dtype=None, D=None, workspace=None):
    """D = A @ B.T + C for bf16 A (M, K) and B (N, K); fp32 accumulation.

    ``out_dtype`` float32 (default) or bfloat16; C (optional) has out_dtype;
    D is allocated unless given.  Enqueued on torch's current stream.
    ``workspace``: for operands given MN-contiguous (a transposed view), a
    device byte tensor of :func:`ex_workspace_bytes` bytes, 256-byte aligned:
    they are copied there K-contiguous first (gemm_bf16_ex_ws).
    """
    import torch
    return _call16("gemm_bf16", A, B, C, torch.float32 if out_dtype is None else out_dtype, D, torch.bfloat16,
                   workspace)


def gemm_fp16(A, B, C=None, out_dtype=None, D=None, workspace=None):
    """As :func:`gemm_bf16` with float16 A and B."""
    import torch
    return _call16("gemm_fp16", A, B, C, torch.float32 if out_dtype is None else out_dtype, D, torch.float16,
                   workspace)


def ex_workspace_bytes(element_bits: int, M: int, N: int, K: int, a_order: str = "k", b_order: str = "k") -> int:
    """Workspace bytes of the *_ex_ws calls (element_bits 16, 8, 6 or 4)."""
    return int(_load().gemm_ex_workspace_bytes(element_bits, M, N, K, _ORDERS[a_order], _ORDERS[b_order]))


def splitk_workspace_bytes(M: int, N: int, K: int, splits: int = 0) -> int:
    """Workspace bytes the split-K calls need (0: no split would be used)."""
    return int(_load().gemm_splitk_workspace_bytes(M, N, K, splits))


def _call16_split(name, A, B, C, out_dtype, D, dtype, splits, workspace):
    import torch
    _on_device(A, workspace=workspace)
    M, N, K, D, stream, out = _prep(A, B, C, D, out_dtype, (dtype,))
    need = splitk_workspace_bytes(M, N, K, splits) if M and N and K else 0
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=A.device)
    _on_device(A, workspace=workspace)
    wp = workspace.data_ptr() if workspace is not None else None
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = getattr(_load(), name)(M, N, K, A.data_ptr(), _ld(A, K) if K else 0, B.data_ptr(), _ld(B, K) if K else 0,
                                C.data_ptr() if C is not None else None, _ld(C, N) if C is not None else 0,
                                D.data_ptr(), _ld(D, N), out, splits, wp, wb, stream)
    _check(st)
    return D


def gemm_bf16_splitk(A, B, C=None, out_dtype=None, D=None, splits=0, workspace=None):
    """:func:`gemm_bf16` with K split over ``splits`` ranges (0: the library's
    choice).  ``workspace``: a device tensor of at least
    :func:`splitk_workspace_bytes` bytes, 256-byte aligned; allocated per
    call when not given."""
    import torch
    return _call16_split("gemm_bf16_splitk", A, B, C, torch.float32 if out_dtype is None else out_dtype, D,
                         torch.bfloat16, splits, workspace)


def gemm_fp16_splitk(A, B, C=None, out_dtype=None, D=None, splits=0, workspace=None):
    """As :func:`gemm_bf16_splitk` with float16 A and B."""
    import torch
    return _call16_split("gemm_fp16_splitk", A, B, C, torch.float32 if out_dtype is None else out_dtype, D,
                         torch.float16, splits, workspace)


def gemm_bf16_splitk_noalloc(A, B, C=None, out_dtype=None, D=None, splits=0):
    """:func:`gemm_bf16_splitk` with the partials in the library's static
    scratch area instead of a workspace: the C call allocates nothing (give
    ``D`` to keep the whole call allocation-free).  Raises GemmError
    (GEMM_ERR_SCRATCH_LIMIT) when the partials exceed
    :func:`splitk_scratch_limit` bytes.  Calls that may overlap on one GPU
    race on the shared area."""
    import torch
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    M, N, K, D, stream, out = _prep(A, B, C, D, out_dtype, (torch.bfloat16,))
    st = _load().gemm_bf16_splitk_noalloc(M, N, K, A.data_ptr(), _ld(A, K) if K else 0, B.data_ptr(),
                                          _ld(B, K) if K else 0, C.data_ptr() if C is not None else None,
                                          _ld(C, N) if C is not None else 0, D.data_ptr(), _ld(D, N), out, splits,
                                          stream)
    _check(st)
    return D


def splitk_scratch_limit() -> int:
    """Bytes of the static scratch area behind :func:`gemm_bf16_splitk_noalloc`."""
    return int(_load().gemm_splitk_scratch_limit())


def _scales(SFA, SFB, M, N, A):
    import torch
    for s, rows in ((SFA, M), (SFB, N)):
        if s.dtype not in (torch.uint8, torch.float8_e8m0fnu) or not s.is_cuda or s.shape[0] != rows:
            raise ValueError("scale arrays must be uint8/e8m0 device tensors of shape (rows, K/32)")
    _on_device(A, SFA=SFA, SFB=SFB)


def _split_tail(M, N, K, A, splits, workspace):
    """(splits, workspace pointer, workspace bytes, kept tensor) of a split-K call."""
    import torch
    need = splitk_workspace_bytes(M, N, K, splits) if M and N and K else 0
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=A.device)
    _on_device(A, workspace=workspace)
    wp = workspace.data_ptr() if workspace is not None else None
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return [splits, wp, wb], workspace


# elements per byte of the block-scaled formats, as (numerator, denominator)
_EPB = {"e4m3": (1, 1), "e2m1": (2, 1), "e2m3": (4, 3), "e3m2": (4, 3)}
_ORDERS = {"k": K_CONTIGUOUS, "mn": MN_CONTIGUOUS}


def _mx_operand(t, X, order):
    """(rows, K, leading dimension in elements) of a block-scaled operand
    given as its byte storage: (rows, K bytes) K-contiguous or (K, rows
    bytes) MN-contiguous."""
    num, den = _EPB[t]
    r, c = X.shape
    if c > 1 and X.stride(1) != 1:
        raise ValueError("the byte storage needs a unit last stride")
    sb = X.stride(0) if r > 1 else c
    if (c * num) % den or (sb * num) % den:
        raise ValueError("rows must hold whole groups of elements (fp6: multiples of 3 bytes)")
    elems, ld = c * num // den, sb * num // den
    return (r, elems, ld) if order == "k" else (elems, r, ld)


def _mx_ex(t, A, SFA, B, SFB, C, out_dtype, D, a_order, b_order, fmt=None, workspace=None):
    """A block-scaled call with explicit storage orders (the *_ex entry
    points; *_ex_ws with a workspace)."""
    import torch
    _on_device(A, workspace=workspace)
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if a_order not in _ORDERS or b_order not in _ORDERS:
        raise ValueError("orders are 'k' or 'mn'")
    ok = (torch.uint8, torch.float8_e4m3fn) if t == "e4m3" else (torch.uint8,)
    if A.dtype not in ok or B.dtype not in ok or not (A.is_cuda and B.is_cuda):
        raise TypeError("A and B must be device byte tensors")
    M, K, lda = _mx_operand(t, A, a_order)
    N, KB, ldb = _mx_operand(t, B, b_order)
    if K != KB:
        raise ValueError("A and B disagree on K")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    if D is None:
        D = torch.empty((M, N), dtype=out_dtype, device=A.device)
    if D.dtype != out_dtype or tuple(D.shape) != (M, N):
        raise ValueError("D must be (M, N) of out_dtype")
    if C is not None and (C.dtype != out_dtype or tuple(C.shape) != (M, N)):
        raise ValueError("C must be (M, N) of out_dtype")
    _on_device(A, B=B, C=C, D=D)
    _scales(SFA, SFB, M, N, A)
    nkb = K // 32
    stream = _Stream(A)
    out = OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32
    args = [M, N, K, A.data_ptr(), lda if K else 0, _ORDERS[a_order], SFA.data_ptr(), _ld(SFA, nkb) if K else 0,
            B.data_ptr(), ldb if K else 0, _ORDERS[b_order], SFB.data_ptr(), _ld(SFB, nkb) if K else 0,
            C.data_ptr() if C is not None else None, _ld(C, N) if C is not None else 0, D.data_ptr(), _ld(D, N)]
    name = {"e4m3": "gemm_mxfp8_ex", "e2m1": "gemm_mxfp4_ex"}.get(t, "gemm_mxfp6_ex")
    if fmt is not None:
        args.append(FP6_FORMATS[fmt])
    if workspace is None:
        _check(getattr(_load(), name)(*args, out, stream))
    else:
        _check(getattr(_load(), name + "_ws")(*args, out, workspace.data_ptr(),
                                               workspace.numel() * workspace.element_size(), stream))
    return D


def _mx8(name, A, SFA, B, SFB, C, out_dtype, D, split):
    import torch
    if split is not None:
        _on_device(A, workspace=split[1])
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    M, N, K, D, stream, out = _prep(A, B, C, D, out_dtype, (torch.float8_e4m3fn, torch.uint8))
    _scales(SFA, SFB, M, N, A)
    nkb = K // 32
    args = [M, N, K, A.data_ptr(), _ld(A, K) if K else 0, SFA.data_ptr(), _ld(SFA, nkb) if K else 0,
            B.data_ptr(), _ld(B, K) if K else 0, SFB.data_ptr(), _ld(SFB, nkb) if K else 0,
            C.data_ptr() if C is not None else None, _ld(C, N) if C is not None else 0, D.data_ptr(), _ld(D, N), out]
    keep = None
    if split is not None:
        tail, keep = _split_tail(M, N, K, A, *split)
        args += tail
    _check(getattr(_load(), name)(*args, stream))
    return D


def gemm_mxfp8(A, SFA, B, SFB, C=None, out_dtype=None, D=None, a_order="k", b_order="k", workspace=None):
    """Block-scaled fp8: A (M, K), B (N, K) e4m3 (float8_e4m3fn or uint8 codes);
    SFA (M, K/32), SFB (N, K/32) e8m0 codes (uint8 or float8_e8m0fnu).
    ``a_order="mn"``: A given as its K x M storage (element (m, k) at [k, m]);
    ``b_order="mn"``: B as K x N (gemm_mxfp8_ex; with ``workspace``, of
    :func:`ex_workspace_bytes` bytes, gemm_mxfp8_ex_ws)."""
    if a_order != "k" or b_order != "k":
        return _mx_ex("e4m3", A, SFA, B, SFB, C, out_dtype, D, a_order, b_order, workspace=workspace)
    return _mx8("gemm_mxfp8", A, SFA, B, SFB, C, out_dtype, D, None)


def gemm_mxfp8_splitk(A, SFA, B, SFB, C=None, out_dtype=None, D=None, splits=0, workspace=None):
    """:func:`gemm_mxfp8` with K split over ``splits`` ranges of whole 512-K
    groups (0: the library's choice); ``workspace`` as
    :func:`gemm_bf16_splitk`."""
    return _mx8("gemm_mxfp8_splitk", A, SFA, B, SFB, C, out_dtype, D, (splits, workspace))


def _mx4(name, A, SFA, B, SFB, C, out_dtype, D, split):
    import torch
    if split is not None:
        _on_device(A, workspace=split[1])
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    fp4x2 = getattr(torch, "float4_e2m1fn_x2", torch.uint8)
    M, N, KB, D, stream, out = _prep(A, B, C, D, out_dtype, (torch.uint8, fp4x2))
    K = 2 * KB
    _scales(SFA, SFB, M, N, A)
    nkb = K // 32
    args = [M, N, K, A.data_ptr(), 2 * _ld(A, KB) if K else 0, SFA.data_ptr(), _ld(SFA, nkb) if K else 0,
            B.data_ptr(), 2 * _ld(B, KB) if K else 0, SFB.data_ptr(), _ld(SFB, nkb) if K else 0,
            C.data_ptr() if C is not None else None, _ld(C, N) if C is not None else 0, D.data_ptr(), _ld(D, N), out]
    keep = None
    if split is not None:
        tail, keep = _split_tail(M, N, K, A, *split)
        args += tail
    _check(getattr(_load(), name)(*args, stream))
    return D


def gemm_mxfp4(A, SFA, B, SFB, C=None, out_dtype=None, D=None, a_order="k", b_order="k", workspace=None):
    """Block-scaled fp4: A (M, K/2), B (N, K/2) uint8 bytes each holding two
    e2m1 codes (element 2i in the low nibble of byte i; float4_e2m1fn_x2 is
    accepted too); SFA (M, K/32), SFB (N, K/32) e8m0 codes.  K is twice the
    byte width of A.  ``a_order="mn"``: A given as its K x M storage, (K,
    M/2) bytes packed along M; ``b_order="mn"`` likewise (gemm_mxfp4_ex;
    with ``workspace`` gemm_mxfp4_ex_ws)."""
    if a_order != "k" or b_order != "k":
        return _mx_ex("e2m1", A, SFA, B, SFB, C, out_dtype, D, a_order, b_order, workspace=workspace)
    return _mx4("gemm_mxfp4", A, SFA, B, SFB, C, out_dtype, D, None)


def gemm_mxfp4_splitk(A, SFA, B, SFB, C=None, out_dtype=None, D=None, splits=0, workspace=None):
    """:func:`gemm_mxfp4` with K split over ``splits`` ranges of whole 512-K
    groups (0: the library's choice); ``workspace`` as
    :func:`gemm_bf16_splitk`."""
    return _mx4("gemm_mxfp4_splitk", A, SFA, B, SFB, C, out_dtype, D, (splits, workspace))


FP6_FORMATS = {"e2m3": 0, "e3m2": 1}


def _mx6(name, A, SFA, B, SFB, C, out_dtype, D, fmt, split):
    import torch
    if split is not None:
        _on_device(A, workspace=split[1])
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if fmt not in FP6_FORMATS:
        raise ValueError("fmt must be 'e2m3' or 'e3m2'")
    M, N, KB, D, stream, out = _prep(A, B, C, D, out_dtype, (torch.uint8,))
    if KB % 3:
        raise ValueError("the byte width of A and B must be a multiple of 3 (four elements per three bytes)")
    K = KB // 3 * 4
    _scales(SFA, SFB, M, N, A)
    lds = []
    for X in (A, B):
        ldb_ = _ld(X, KB) if K else 0
        if ldb_ % 3:
            raise ValueError("row strides of A and B must be multiples of 3 bytes")
        lds.append(ldb_ // 3 * 4)
    nkb = K // 32
    args = [M, N, K, A.data_ptr(), lds[0], SFA.data_ptr(), _ld(SFA, nkb) if K else 0,
            B.data_ptr(), lds[1], SFB.data_ptr(), _ld(SFB, nkb) if K else 0,
            C.data_ptr() if C is not None else None, _ld(C, N) if C is not None else 0,
            D.data_ptr(), _ld(D, N), FP6_FORMATS[fmt], out]
    keep = None
    if split is not None:
        tail, keep = _split_tail(M, N, K, A, *split)
        args += tail
    _check(getattr(_load(), name)(*args, stream))
    return D


def gemm_mxfp6(A, SFA, B, SFB, C=None, out_dtype=None, D=None, fmt="e2m3", a_order="k", b_order="k",
               workspace=None):
    """Block-scaled fp6: A (M, 3K/4), B (N, 3K/4) uint8 bytes holding six-bit
    codes (element k at bits 6k .. 6k+5 of a row read as a little-endian bit
    string) in format ``fmt`` ("e2m3" or "e3m2"); SFA (M, K/32), SFB (N, K/32)
    e8m0 codes.  K is four thirds of the byte width of A.  ``a_order="mn"``:
    A given as its K x M storage, (K, 3M/4) bytes packed along M;
    ``b_order="mn"`` likewise (gemm_mxfp6_ex; with ``workspace``
    gemm_mxfp6_ex_ws, which for K-contiguous operands and a workspace of
    :func:`ex_workspace_bytes` (6, M, N, K) bytes runs on their tile
    images)."""
    if a_order != "k" or b_order != "k" or workspace is not None:
        if fmt not in FP6_FORMATS:
            raise ValueError("fmt must be 'e2m3' or 'e3m2'")
        return _mx_ex(fmt, A, SFA, B, SFB, C, out_dtype, D, a_order, b_order, fmt, workspace=workspace)
    return _mx6("gemm_mxfp6", A, SFA, B, SFB, C, out_dtype, D, fmt, None)


MX_FORMATS = {"e4m3": 0, "e2m1": 1, "e2m3": 2, "e3m2": 3}


def mx_kblock_workspace_bytes(M: int, N: int, K: int) -> int:
    """Workspace bytes :func:`gemm_mx_kblock` needs with ``workspace``."""
    return int(_load().gemm_mx_kblock_workspace_bytes(M, N, K))


def gemm_mx_kblock(fmt, A, SFA, B, SFB, kblock, C=None, out_dtype=None, D=None, workspace=None):
    """Block-scaled D = A @ B.T + C with scale blocks ``kblock`` K elements
    wide (a multiple of 32; >= K: one scale per row).  ``fmt``: "e4m3",
    "e2m1", "e2m3" or "e3m2"; A (M, K bytes-of-format) and B (N, ...) as the
    format's standard call takes them; SFA (M, ceil(K / kblock)), SFB (N,
    ceil(K / kblock)) e8m0 codes.  ``workspace``: a device byte tensor of at
    least :func:`mx_kblock_workspace_bytes` bytes, 256-byte aligned: the
    scales are replicated to 32-wide blocks there and the call runs on the
    format's tiled kernels (gemm_mx_kblock_ws); None: the general kernel."""
    import torch
    if fmt not in MX_FORMATS:
        raise ValueError("fmt must be one of %s" % sorted(MX_FORMATS))
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    ok = (torch.uint8, torch.float8_e4m3fn) if fmt == "e4m3" else (torch.uint8,)
    if A.dtype not in ok or B.dtype not in ok or not (A.is_cuda and B.is_cuda):
        raise TypeError("A and B must be device byte tensors")
    M, K, lda = _mx_operand(fmt, A, "k")
    N, KB, ldb = _mx_operand(fmt, B, "k")
    if K != KB:
        raise ValueError("A and B disagree on K")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    if D is None:
        D = torch.empty((M, N), dtype=out_dtype, device=A.device)
    if D.dtype != out_dtype or tuple(D.shape) != (M, N):
        raise ValueError("D must be (M, N) of out_dtype")
    if C is not None and (C.dtype != out_dtype or tuple(C.shape) != (M, N)):
        raise ValueError("C must be (M, N) of out_dtype")
    _on_device(A, B=B, C=C, D=D, workspace=workspace)
    _scales(SFA, SFB, M, N, A)
    nsc = -(-K // kblock) if kblock > 0 else 0
    out = OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32
    args = [MX_FORMATS[fmt], M, N, K, int(kblock), A.data_ptr(), lda if K else 0,
            SFA.data_ptr(), _ld(SFA, nsc) if K else 0, B.data_ptr(), ldb if K else 0,
            SFB.data_ptr(), _ld(SFB, nsc) if K else 0,
            C.data_ptr() if C is not None else None, _ld(C, N) if C is not None else 0,
            D.data_ptr(), _ld(D, N), out]
    if workspace is None:
        _check(_load().gemm_mx_kblock(*args, _Stream(A)))
    else:
        nbytes = workspace.numel() * workspace.element_size()
        _check(_load().gemm_mx_kblock_ws(*args, workspace.data_ptr(), nbytes, _Stream(A)))
    return D


def mxfp6_packed_bytes(rows: int, K: int) -> int:
    """Bytes of the tile images of an fp6 operand of ``rows`` rows and K
    elements (gemm_mxfp6_packed_bytes; 0 when K % 128 != 0)."""
    return int(_load().gemm_mxfp6_packed_bytes(rows, K))


def mxfp6_pack(X, out=None):
    """Tile images of the fp6 operand X -- (rows, 3K/4) uint8 bytes, as
    :func:`gemm_mxfp6` takes A or B -- for :func:`gemm_mxfp6_packed`
    (gemm_mxfp6_pack).  ``out``: a device uint8 tensor of at least
    :func:`mxfp6_packed_bytes` bytes, 16-byte aligned (None: allocated).
    Returns the images as a flat uint8 tensor."""
    import torch
    if X.dtype != torch.uint8 or X.dim() != 2 or not X.is_cuda:
        raise TypeError("X must be a 2-D uint8 device tensor")
    rows, KB = X.shape
    if KB % 3:
        raise ValueError("the byte width of X must be a multiple of 3 (four elements per three bytes)")
    K = KB // 3 * 4
    ldb_ = _ld(X, KB) if K else 0
    if ldb_ % 3:
        raise ValueError("the row stride of X must be a multiple of 3 bytes")
    need = mxfp6_packed_bytes(rows, K)
    if out is None:
        out = torch.empty(need, dtype=torch.uint8, device=X.device)
    _on_device(X, out=out)
    nb = out.numel() * out.element_size()
    _check(_load().gemm_mxfp6_pack(rows, K, X.data_ptr(), ldb_ // 3 * 4, out.data_ptr(), nb, _Stream(X)))
    return out


def gemm_mxfp6_packed(AP, SFA, BP, SFB, M, N, K, C=None, out_dtype=None, D=None, fmt="e2m3"):
    """:func:`gemm_mxfp6` with A and B given as their tile images
    (:func:`mxfp6_pack` of the (M, 3K/4) and (N, 3K/4) operands; flat
    device uint8 tensors); the same D bit for bit (gemm_mxfp6_packed)."""
    import torch
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if fmt not in FP6_FORMATS:
        raise ValueError("fmt must be 'e2m3' or 'e3m2'")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    for name, X, rows in (("AP", AP, M), ("BP", BP, N)):
        if X.dtype != torch.uint8 or not X.is_cuda or not X.is_contiguous():
            raise TypeError("%s must be a contiguous uint8 device tensor" % name)
        if X.numel() < mxfp6_packed_bytes(rows, K):
            raise ValueError("%s holds fewer bytes than the images of %d rows" % (name, rows))
    if D is None:
        D = torch.empty((M, N), dtype=out_dtype, device=AP.device)
    if D.dtype != out_dtype or tuple(D.shape) != (M, N):
        raise ValueError("D must be (M, N) of out_dtype")
    if C is not None and (C.dtype != out_dtype or tuple(C.shape) != (M, N)):
        raise ValueError("C must be (M, N) of out_dtype")
    _on_device(AP, BP=BP, C=C, D=D)
    _scales(SFA, SFB, M, N, AP)
    nkb = K // 32
    out = OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32
    _check(_load().gemm_mxfp6_packed(M, N, K, AP.data_ptr(), SFA.data_ptr(), _ld(SFA, nkb) if K else 0,
                                     BP.data_ptr(), SFB.data_ptr(), _ld(SFB, nkb) if K else 0,
                                     C.data_ptr() if C is not None else None, _ld(C, N) if C is not None else 0,
                                     D.data_ptr(), _ld(D, N), FP6_FORMATS[fmt], out, _Stream(AP)))
    return D


def gemm_mxfp6_splitk(A, SFA, B, SFB, C=None, out_dtype=None, D=None, fmt="e2m3", splits=0, workspace=None):
    """:func:`gemm_mxfp6` with K split over ``splits`` ranges of whole 512-K
    groups (0: the library's choice); ``workspace`` as
    :func:`gemm_bf16_splitk`."""
    return _mx6("gemm_mxfp6_splitk", A, SFA, B, SFB, C, out_dtype, D, fmt, (splits, workspace))
