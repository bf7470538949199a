"""Seeded synthetic workloads for D = A.B + C.

This module only draws numbers: it holds none of the operation's arithmetic and
imports neither the HIP binding nor the oracle.  Both sides take their inputs
from here.

Draw recipe (the same for every workload):

* ``numpy.random.default_rng(seed)`` (PCG64); draw order A (M x K, row-major),
  B (its N x K storage order), C (M x N), then SFA, SFB.
* Floating values are drawn in float32 and rounded to the element type with
  torch's CPU casts (round to nearest even): bf16, fp16, float8_e4m3fn.
* "N(0, s)": s is the standard deviation.
* Integer variants: A, B, C uniform integers in [-4, 4]; for the block-scaled
  form the e4m3 elements are integers in [-4, 4] and the scale exponents lie
  in {0, 1, 2}, so every partial sum stays an integer below 2^24.
* e8m0 scales: exponent e uniform in {-4..4}, stored code 127 + e.
* e2m1 (fp4) elements: codes drawn uniformly from all 16 (each value of
  {0, 0.5, 1, 1.5, 2, 3, 4, 6} and its negative equally likely), packed two
  per byte with element 2i in the low nibble of byte i; the integer variant
  draws the same codes with scale exponents in {1, 2}, so every product is
  an integer and partial sums stay below 2^24 for K up to 16384.
* e2m3 / e3m2 (fp6) elements: codes drawn uniformly from all 64, packed six
  bits each (element k at bits 6k .. 6k+5 of the row as a little-endian bit
  string, four per three bytes); the integer variant draws codes of
  magnitude at most 1 with scale exponent 3 (e2m3) or 4 (e3m2), so every
  product is an integer of magnitude at most 64 (256) and partial sums stay
  below 2^24 for K up to 65536.

Each workload keeps its operands as raw element codes (uint16 for bf16/fp16,
uint8 for e4m3/e8m0, packed uint8 pairs for e2m1) plus float32 C, laid out
packed (lda = ldb = K elements, ldc = N).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    in_type: str            # "bf16" | "fp16" | "e4m3" | "e2m1"
    out_type: str           # "f32" | "bf16"
    dist_a: tuple
    dist_b: tuple
    dist_c: tuple | None    # None: C absent (C = 0, passed as NULL)
    seed: int
    scaled: bool = False    # block-scaled e4m3 / e2m1 with e8m0 scales per 32 K
    note: str = ""
    packed: bool = False    # fp6: A and B given as tile images (gemm_mxfp6_packed)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


U11 = ("uniform", -1.0, 1.0)
CODES = ("codes",)          # e2m1: every 4-bit code equally likely

WORKLOADS = {
    "square256_bf16": Workload("square256_bf16", 256, 256, 256, "bf16", "f32", U11, U11, U11, 0,
                               note="M=N=K=256 bf16, C and D fp32"),
    "square4096_bf16": Workload("square4096_bf16", 4096, 4096, 4096, "bf16", "f32", U11, U11, U11, 1,
                                note="M=N=K=4096 bf16, C and D fp32"),
    "ragged_fp16": Workload("ragged_fp16", 4000, 3000, 4100, "fp16", "f32",
                            ("normal", 1.0), ("normal", 1.0), None, 2,
                            note="M=4000 N=3000 K=4100 fp16, C=0, fp32 out"),
    "llm_proj_bf16": Workload("llm_proj_bf16", 16384, 14336, 4096, "bf16", "bf16",
                              ("normal", 1.0), ("normal", 0.02), None, 3,
                              note="M=16384 N=14336 K=4096 bf16, C=0, bf16 out"),
    "llm_proj_shard8_bf16": Workload("llm_proj_shard8_bf16", 16384, 1792, 4096, "bf16", "bf16",
                                     ("normal", 1.0), ("normal", 0.02), None, 3,
                                     note="one GPU's share of the projection N-sharded 8 ways: M=16384 N=1792 "
                                          "K=4096 bf16, C=0, bf16 out"),
    "largek_bf16": Workload("largek_bf16", 1024, 1024, 65536, "bf16", "f32", U11, U11, None, 6,
                            note="M=N=1024 K=65536 bf16, C=0, fp32 out (16 output tiles: split-K)"),
    "mxfp8_8192": Workload("mxfp8_8192", 8192, 8192, 8192, "e4m3", "f32", U11, U11, None, 4,
                           scaled=True, note="M=N=K=8192 e4m3 + e8m0 per 32 K, C=0, fp32 out"),
    "largek_mxfp8": Workload("largek_mxfp8", 1024, 1024, 65536, "e4m3", "f32", U11, U11, None, 8, scaled=True,
                             note="M=N=1024 K=65536 e4m3 + e8m0 per 32 K, C=0, fp32 out (16 output tiles: split-K)"),
    "mxfp6_8192": Workload("mxfp6_8192", 8192, 8192, 8192, "e2m3", "f32", CODES, CODES, None, 7,
                           scaled=True, note="M=N=K=8192 fp6 e2m3 + e8m0 per 32 K, C=0, fp32 out"),
    "mxfp6_8192_packed": Workload("mxfp6_8192_packed", 8192, 8192, 8192, "e2m3", "f32", CODES, CODES, None, 7,
                                  scaled=True, packed=True,
                                  note="mxfp6_8192 with A and B as tile images, packed once before the timed "
                                       "steps (operands reused across calls, e.g. weights)"),
    "mxfp4_8192": Workload("mxfp4_8192", 8192, 8192, 8192, "e2m1", "f32", CODES, CODES, None, 5,
                           scaled=True, note="M=N=K=8192 e2m1 + e8m0 per 32 K, C=0, fp32 out"),
}


def _draw(rng, dist, shape):
    kind = dist[0]
    if kind == "uniform":
        lo, hi = dist[1], dist[2]
        return rng.uniform(lo, hi, size=shape).astype(np.float32)
    if kind == "normal":
        x = rng.standard_normal(size=shape, dtype=np.float32)
        return x * np.float32(dist[1])
    raise ValueError(kind)


def to_codes(x_f32: np.ndarray, in_type: str) -> np.ndarray:
    """float32 -> raw element codes by torch's RNE casts (generation only)."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    if in_type == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if in_type == "fp16":
        return t.to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    if in_type == "e4m3":
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    raise ValueError(in_type)


def pack_e2m1(codes: np.ndarray) -> np.ndarray:
    """(R, 2n) 4-bit codes -> (R, n) bytes, element 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def _e2m1(rng, shape):
    return pack_e2m1(rng.integers(0, 16, size=shape).astype(np.uint8))


FP6 = ("e2m3", "e3m2")
# codes of magnitude <= 1 (sign bit 0x20 free): e2m3 0..8 (0 .. 1 in steps of
# 1/8), e3m2 0..12 (0 .. 1: subnormals 1/16 .. 3/16, then 0.25 .. 1)
_FP6_UNIT = {"e2m3": 9, "e3m2": 13}
_FP6_INT_SCALE = {"e2m3": 3, "e3m2": 4}


def pack_fp6(codes: np.ndarray) -> np.ndarray:
    """(R, 4n) six-bit codes -> (R, 3n) bytes, element k at bits 6k .. 6k+5
    of the row read as a little-endian bit string."""
    c = np.asarray(codes, dtype=np.uint32)
    g = c.reshape(c.shape[:-1] + (-1, 4))
    w = g[..., 0] | (g[..., 1] << 6) | (g[..., 2] << 12) | (g[..., 3] << 18)
    out = np.empty(c.shape[:-1] + (g.shape[-2], 3), dtype=np.uint8)
    for j in range(3):
        out[..., j] = (w >> (8 * j)) & 0xFF
    return out.reshape(c.shape[:-1] + (-1,))


def _fp6(rng, in_type, shape, integer=False):
    if integer:
        mag = rng.integers(0, _FP6_UNIT[in_type], size=shape)
        codes = mag | (rng.integers(0, 2, size=shape) << 5)
    else:
        codes = rng.integers(0, 64, size=shape)
    return pack_fp6(codes.astype(np.uint8))


def generate(w: Workload, integer: bool = False, M=None, N=None, K=None, seed=None):
    """Draw a workload's operands.  Sizes and seed may be overridden (for
    reduced-size parity cases of the same recipe).

    Returns a dict with ``A`` (M x K codes), ``B`` (N x K codes), ``C`` (M x N
    float32 or None), ``SFA``/``SFB`` (uint8 e8m0 codes or None) and the sizes.
    """
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    if w.in_type in FP6:
        A, B, C = _fp6(rng, w.in_type, (M, K), integer), _fp6(rng, w.in_type, (N, K), integer), None
        if w.dist_c is not None:
            C = rng.integers(-4, 5, size=(M, N)).astype(np.float32) if integer else _draw(rng, w.dist_c, (M, N))
    elif w.in_type == "e2m1":
        A, B, C = _e2m1(rng, (M, K)), _e2m1(rng, (N, K)), None
        if w.dist_c is not None:
            C = rng.integers(-4, 5, size=(M, N)).astype(np.float32) if integer else _draw(rng, w.dist_c, (M, N))
    elif integer:
        A = to_codes(rng.integers(-4, 5, size=(M, K)).astype(np.float32), w.in_type)
        B = to_codes(rng.integers(-4, 5, size=(N, K)).astype(np.float32), w.in_type)
        C = rng.integers(-4, 5, size=(M, N)).astype(np.float32) if w.dist_c is not None else None
    else:
        A = to_codes(_draw(rng, w.dist_a, (M, K)), w.in_type)
        B = to_codes(_draw(rng, w.dist_b, (N, K)), w.in_type)
        C = _draw(rng, w.dist_c, (M, N)) if w.dist_c is not None else None
    SFA = SFB = None
    if w.scaled:
        nkb = -(-K // 32)
        if integer and w.in_type in FP6:
            lo, hi = _FP6_INT_SCALE[w.in_type], _FP6_INT_SCALE[w.in_type] + 1
            SFA = (127 + rng.integers(lo, hi, size=(M, nkb))).astype(np.uint8)
            SFB = (127 + rng.integers(lo, hi, size=(N, nkb))).astype(np.uint8)
        elif integer:
            lo, hi = (1, 3) if w.in_type == "e2m1" else (0, 3)
            SFA = (127 + rng.integers(lo, hi, size=(M, nkb))).astype(np.uint8)
            SFB = (127 + rng.integers(lo, hi, size=(N, nkb))).astype(np.uint8)
        else:
            SFA = (127 + rng.integers(-4, 5, size=(M, nkb))).astype(np.uint8)
            SFB = (127 + rng.integers(-4, 5, size=(N, nkb))).astype(np.uint8)
    return {"A": A, "B": B, "C": C, "SFA": SFA, "SFB": SFB, "M": M, "N": N, "K": K,
            "in_type": w.in_type, "out_type": w.out_type}


def random_codes(rng, in_type, shape, integer=False, dist=U11):
    """Free-standing operand draw (parity sweeps of odd shapes).  For e2m1 the
    codes are uniform (integer or not: the scales make the values integral)
    and ``shape[-1]`` is the element count, returned packed two per byte;
    for the fp6 types likewise, packed four per three bytes (integer: the
    codes of magnitude at most 1, for use with ``fp6_integer_scale``)."""
    if in_type == "e2m1":
        return _e2m1(rng, shape)
    if in_type in FP6:
        return _fp6(rng, in_type, shape, integer)
    if integer:
        return to_codes(rng.integers(-4, 5, size=shape).astype(np.float32), in_type)
    return to_codes(_draw(rng, dist, shape), in_type)


def fp6_integer_scale(in_type: str) -> int:
    """The e8m0 exponent that makes the integer variant's fp6 values integers."""
    return _FP6_INT_SCALE[in_type]


def sample_indices(M: int, N: int, seed: int, count: int = 4096):
    """Output elements to check on large outputs.

    ``(random, forced)`` flat indices ``m*N + n``: ``count`` distinct elements
    from ``default_rng(seed + 7919)``, and a forced set: the four corners, 64
    elements in the last 256 rows, 64 in the last 256 columns, and the
    crossings of rows and columns on both sides of the 128/256 boundaries.
    """
    total = M * N
    rng = np.random.default_rng(seed + 7919)
    count = min(count, total)
    rand = rng.choice(total, size=count, replace=False).astype(np.int64)
    forced = {(0, 0), (0, N - 1), (M - 1, 0), (M - 1, N - 1)}
    r_lo, c_lo = max(0, M - 256), max(0, N - 256)
    for _ in range(64):
        forced.add((int(rng.integers(r_lo, M)), int(rng.integers(0, N))))
        forced.add((int(rng.integers(0, M)), int(rng.integers(c_lo, N))))
    edges_r = [r for r in (127, 128, 255, 256, M - 2) if 0 <= r < M]
    edges_c = [c for c in (127, 128, 255, 256, N - 2) if 0 <= c < N]
    for r in edges_r:
        for c in edges_c:
            forced.add((r, c))
    forced_idx = np.array(sorted(m * N + n for m, n in forced), dtype=np.int64)
    return rand, forced_idx
