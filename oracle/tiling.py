"""Row-major CTA tiling of an output and its K-tiled product (test infrastructure only).

Source: "（二）CUTLASS —— 掌握 Tensor Memory Accelerator（TMA）", section 示例任务
(example task): a row-major M x N matrix is split into CTA_M x CTA_N tiles with
a numpy reshape, one tile per CTA, and the grid is (M / CTA_M, N / CTA_N).  The
printed snippet is garbled (it passes M, N to ``uniform`` as bounds, its last
reshape extent reads N, and its loops run over M and N); the reading used
here: tile (i, j) is ``X[i*CTA_M:(i+1)*CTA_M, j*CTA_N:(j+1)*CTA_N]`` for
``i < M / CTA_M``, ``j < N / CTA_N``.  Same page, section on remainder tiles:
M and N need not divide by the tile; a partial last tile reads out-of-range
elements as absent (zero here) and writes none of them.  So the tile counts
are ceil-divisions.
"""
from __future__ import annotations

import numpy as np


def tile_counts(M, N, BM, BN):
    return -(-M // BM), -(-N // BN)


def tile_view_reshape(X, BM, BN, i, j):
    """Tile (i, j) of X by the reshape of the page (M, N divisible by BM, BN)."""
    M, N = X.shape
    assert M % BM == 0 and N % BN == 0
    return X.reshape(M // BM, BM, N // BN, BN)[i, :, j, :]


def tile_padded(X, BM, BN, i, j):
    """Tile (i, j) with remainder handling: a BM x BN block, out-of-range entries 0."""
    M, N = X.shape
    out = np.zeros((BM, BN), dtype=X.dtype)
    r0, c0 = i * BM, j * BN
    blk = X[r0:min(r0 + BM, M), c0:min(c0 + BN, N)]
    out[: blk.shape[0], : blk.shape[1]] = blk
    return out


def tiled_gemm(a, b, c, BM, BN, BK):
    """D = a @ b.T + c computed tile by tile with zero-padded K tiles.

    ``a``: (M, K), ``b``: (N, K) (column-major B stored by columns), ``c``: (M, N)
    or None.  Each output tile accumulates its K tiles in order and only the
    in-range part of each tile is written.  Returns (D, coverage) where
    coverage counts the writes of every output element.
    """
    M, K = a.shape
    N = b.shape[0]
    tm, tn = tile_counts(M, N, BM, BN)
    tk = -(-K // BK)
    D = np.zeros((M, N), dtype=np.result_type(a, b))
    cover = np.zeros((M, N), dtype=np.int64)
    for i in range(tm):
        for j in range(tn):
            acc = np.zeros((BM, BN), dtype=D.dtype)
            for t in range(tk):
                at = tile_padded(a, BM, BK, i, t)
                bt = tile_padded(b, BN, BK, j, t)
                acc += at @ bt.T
            r0, c0 = i * BM, j * BN
            r1, c1 = min(r0 + BM, M), min(c0 + BN, N)
            out = acc[: r1 - r0, : c1 - c0]
            if c is not None:
                out = out + c[r0:r1, c0:c1]
            D[r0:r1, c0:c1] = out
            cover[r0:r1, c0:c1] += 1
    return D, cover
