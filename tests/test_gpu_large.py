"""Operands and results past 4 GiB, on an MI355X.

Buffer resources address at most 2^32 bytes, and row offsets such as
m * lda overflow 32 bits long before the sizes the library accepts, so
each case puts an operand (and, where it says so, D) well past 4 GiB and
checks whole rows or columns at the start, around the 2 GiB and 4 GiB byte
offsets and at the ragged end against the oracle, exactly (integer-valued
inputs).

The big operand is built on the device from a block of P = 4099 seeded rows:
row r is block row r mod P (P prime, so a wrong 32-bit wrap-around lands on
a row with other contents); the oracle gets the same block rows.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_dense_gemm_tile_amd as tg
from tiled_dense_gemm_tile_amd import inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpuutil import DEV, dev8, dev16, say

P = 4099
BIG = 1_050_000

# (label, in_type, M, N, K, big operand, out): A (or B) > 4 GiB; the first
# bf16 case also has D > 4 GiB, the last case a bf16 D > 4 GiB
CASES = [
    ("bf16_a_and_d", "bf16", BIG, 1040, 2112, "A", torch.float32),
    ("bf16_b", "bf16", 160, BIG, 2112, "B", torch.float32),
    ("bf16_d_bf16out", "bf16", BIG, 2100, 64, "A", torch.bfloat16),
    ("mxfp8_a", "e4m3", BIG, 520, 4608, "A", torch.float32),
    ("mxfp4_a", "e2m1", BIG, 520, 8704, "A", torch.float32),
    ("mxfp6_a", "e2m3", BIG, 520, 5760, "A", torch.float32),
]

_ROW_BYTES = {"bf16": 2.0, "e4m3": 1.0, "e2m1": 0.5, "e2m3": 0.75}


def _scale_exps(t):
    if t == "e4m3":
        return 0, 2
    if t == "e2m1":
        return 1, 3
    e = inputs.fp6_integer_scale(t)
    return e, e + 1


def _rows_to_check(rows, row_bytes, rng):
    """Rows at the start, either side of the 2 GiB and 4 GiB byte offsets of
    each storage whose row length is in row_bytes, at the end, and a few
    random ones."""
    pick = {0, 1, 255, 256, rows - 257, rows - 256, rows - 1}
    for rb in row_bytes:
        for edge in (1 << 31, 1 << 32):
            r = int(edge // rb)
            pick.update(x for x in (r - 1, r, r + 1) if 0 <= x < rows)
    pick.update(int(x) for x in rng.integers(0, rows, size=24))
    return np.array(sorted(pick), dtype=np.int64)


def _expand(block_dev, rows):
    idx = torch.arange(rows, device=DEV) % P
    return block_dev.index_select(0, idx)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_past_4gib(case):
    label, t, M, N, K, big, out = case
    rng = np.random.default_rng(sum(map(ord, label)))
    scaled = t != "bf16"
    big_rows, small_rows = (M, N) if big == "A" else (N, M)
    blk = inputs.random_codes(rng, t, (P, K), integer=True)
    small = inputs.random_codes(rng, t, (small_rows, K), integer=True)
    if scaled:
        lo, hi = _scale_exps(t)
        sblk = (127 + rng.integers(lo, hi, size=(P, K // 32))).astype(np.uint8)
        ssmall = (127 + rng.integers(lo, hi, size=(small_rows, K // 32))).astype(np.uint8)
    say("large %s: %s M=%d N=%d K=%d, big operand %s (%.2f GB)" %
        (label, t, M, N, K, big, big_rows * K * _ROW_BYTES[t] / 1e9))

    put = (lambda x: dev16(x, "bf16")) if t == "bf16" else dev8
    X_big = _expand(put(blk), big_rows)
    X_small = put(small)
    if scaled:
        S_big = _expand(dev8(sblk), big_rows)
        S_small = dev8(ssmall)
    A, B = (X_big, X_small) if big == "A" else (X_small, X_big)
    if scaled:
        SFA, SFB = (S_big, S_small) if big == "A" else (S_small, S_big)
        if t == "e4m3":
            D = tg.gemm_mxfp8(A, SFA, B, SFB, None, out_dtype=out)
        elif t == "e2m1":
            D = tg.gemm_mxfp4(A, SFA, B, SFB, None, out_dtype=out)
        else:
            D = tg.gemm_mxfp6(A, SFA, B, SFB, None, out_dtype=out, fmt=t)
    else:
        D = tg.gemm_bf16(A, B, None, out_dtype=out)
    torch.cuda.synchronize()
    del X_big, A, B
    if scaled:
        del S_big, SFA, SFB

    d_row_bytes = N * (4 if out == torch.float32 else 2)
    in_row_bytes = K * _ROW_BYTES[t]
    if big == "A":
        rows = _rows_to_check(M, (in_row_bytes, d_row_bytes), rng)
        sel = torch.from_numpy(rows).to(DEV)
        Dg = D.index_select(0, sel).cpu()
        a_rows = blk[rows % P]
        kw = {"SFA": sblk[rows % P], "SFB": ssmall} if scaled else {}
        Dr, _ = oracle.gemm_ref(t, a_rows, small, **kw)
    else:
        cols = _rows_to_check(N, (in_row_bytes,), rng)
        sel = torch.from_numpy(cols).to(DEV)
        Dg = D.index_select(1, sel).contiguous().cpu()
        kw = {"SFA": ssmall, "SFB": sblk[cols % P]} if scaled else {}
        Dr, _ = oracle.gemm_ref(t, small, blk[cols % P], **kw)
    del D
    if out == torch.bfloat16:                     # bf16 D: nearest-even rounding of the exact sum
        Dg = Dg.view(torch.int16).numpy().view(np.uint16)
        Dr = oracle.rne_bf16_f32(Dr.astype(np.float32))
    else:
        Dg = Dg.numpy().astype(np.float64)
    bad = np.argwhere(Dg != Dr)
    assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()
