"""Pins of the oracle-side models: tiling, prefetch ring, bank model, checker (CPU only)."""
import os

import numpy as np
import pytest

import oracle
from oracle import banks, check, pipeline, tiling
from tiled_dense_gemm_tile_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


# ---- tiling ------------------------------------------------------------------

def test_reshape_view_equals_slicing():
    X = np.arange(12 * 20).reshape(12, 20)
    for i in range(3):
        for j in range(4):
            assert np.array_equal(tiling.tile_view_reshape(X, 4, 5, i, j), X[4 * i:4 * i + 4, 5 * j:5 * j + 5])
            assert np.array_equal(tiling.tile_padded(X, 4, 5, i, j), X[4 * i:4 * i + 4, 5 * j:5 * j + 5])


@pytest.mark.parametrize("M,N,K,BM,BN,BK", [
    (16, 16, 16, 4, 4, 4), (17, 13, 11, 4, 8, 4), (5, 3, 7, 8, 8, 8), (33, 65, 70, 16, 32, 64),
    (1, 1, 1, 4, 4, 4), (40, 30, 41, 16, 8, 8)])
def test_tiled_equals_untiled_integers(M, N, K, BM, BN, BK):
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    a = rng.integers(-4, 5, size=(M, K)).astype(np.int64)
    b = rng.integers(-4, 5, size=(N, K)).astype(np.int64)
    c = rng.integers(-4, 5, size=(M, N)).astype(np.int64)
    D, cover = tiling.tiled_gemm(a, b, c, BM, BN, BK)
    assert np.array_equal(D, a @ b.T + c)
    assert np.all(cover == 1)
    assert tiling.tile_counts(M, N, BM, BN) == (-(-M // BM), -(-N // BN))


def test_tile_counts_of_workloads():
    assert tiling.tile_counts(4096, 4096, 256, 256) == (16, 16)
    assert tiling.tile_counts(4000, 3000, 256, 256) == (16, 12)
    assert tiling.tile_counts(16384, 14336, 256, 256) == (64, 56)
    # last tile of the ragged workload: 160 rows x 184 columns
    assert 4000 - 15 * 256 == 160 and 3000 - 11 * 256 == 184


def test_tiled_oracle_values_match_oracle():
    """The tiled float64 product of decoded operands agrees with the naive oracle."""
    rng = np.random.default_rng(8)
    M, N, K = 45, 38, 70
    A = inputs.random_codes(rng, "bf16", (M, K), integer=True)
    B = inputs.random_codes(rng, "bf16", (N, K), integer=True)
    D, _ = oracle.gemm_ref("bf16", A, B)
    a, b = oracle.operands_f64("bf16", A, B)
    Dt, _ = tiling.tiled_gemm(a, b, None, 16, 32, 32)
    assert np.array_equal(D, Dt)


# ---- prefetch ring -------------------------------------------------------------

def test_prefetch_schedule_matches_page():
    rows = _golden("prefetch_two_stages.txt")
    S = int(rows[0][1])
    expect = [(int(c), int(f)) for c, f in rows[1:]]
    prologue, steady = pipeline.prefetch_schedule(10, S)
    assert prologue == [0, 1]
    assert steady[: len(expect)] == expect
    assert all(f == c + S for c, f in steady if f is not None)


@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("nk", list(range(1, 13)))
def test_ring_with_s_plus_one_slots_is_safe(S, nk):
    assert pipeline.check_ring(pipeline.ring_trace(nk, S), nk) == []


@pytest.mark.parametrize("S", [2, 3])
def test_ring_with_s_slots_is_flagged(S):
    nk = 8
    probs = pipeline.check_ring(pipeline.ring_trace(nk, S, n_slots=S), nk)
    assert probs and "refilled" in probs[0]


# ---- bank model ------------------------------------------------------------------

def test_bank_model_reproduces_page_8way():
    kv = {r[0]: int(r[1]) for r in _golden("bank_conflict_8x64_fp16.txt")}
    rows, cols, eb, bb = kv["rows"], kv["cols"], kv["elem_bytes"], kv["bank_bytes"]
    pitch = cols * eb
    for j in (0, 5, 63):
        addrs = [r * pitch + j * eb for r in range(rows)]
        assert banks.conflict_ways(addrs, eb, n_banks=32, bank_bytes=bb) == kv["unswizzled_ways"]
        cpr = pitch // 16
        sw = [r * pitch + banks.xor_swizzle_chunk(r, (j * eb) // 16, cpr) * 16 + (j * eb) % 16
              for r in range(rows)]
        assert banks.conflict_ways(sw, eb, n_banks=32, bank_bytes=bb) == 1
    # row writes stay contiguous and conflict-free under the XOR layout
    for r in range(rows):
        addrs = [r * pitch + banks.xor_swizzle_chunk(r, c, 8) * 16 for c in range(8)]
        assert banks.conflict_ways(addrs, 16, n_banks=32, bank_bytes=4) == 1


# ---- checker and block Freivalds ----------------------------------------------

def _case(seed=0, M=70, N=90, K=130, integer=False):
    rng = np.random.default_rng(seed)
    A = inputs.random_codes(rng, "bf16", (M, K), integer=integer)
    B = inputs.random_codes(rng, "bf16", (N, K), integer=integer)
    C = (rng.integers(-4, 5, size=(M, N)) if integer else rng.uniform(-1, 1, size=(M, N))).astype(np.float32)
    return A, B, C


def test_checker_fault_injection():
    A, B, C = _case()
    D, S = oracle.gemm_ref("bf16", A, B, C=C)
    tol = check.tolerance(S)
    assert check.within_tolerance(D, D, S).all()
    bad = D.copy()
    bad[3, 4] += 2 * tol[3, 4]
    assert not check.within_tolerance(bad, D, S)[3, 4]
    ok = D.copy()
    ok[3, 4] -= 0.5 * tol[3, 4]
    assert check.within_tolerance(ok, D, S).all()
    nan = D.copy()
    nan[0, 0] = np.nan
    assert not check.within_tolerance(nan, D, S)[0, 0]
    inf = D.copy()
    inf[1, 1] = np.inf
    assert check.report(inf, D, S)["fail"] == 1


def test_freivalds_passes_fp32_rounded_result():
    A, B, C = _case(1)
    D, S = oracle.gemm_ref("bf16", A, B, C=C)
    a, b = oracle.operands_f64("bf16", A, B)
    ok, ratio = check.freivalds_blocks(D.astype(np.float32), a, b, C, block=16)
    assert ok and ratio < 0.05


def test_freivalds_catches_wrong_block():
    A, B, C = _case(2, M=128, N=128, K=256)
    D, S = oracle.gemm_ref("bf16", A, B, C=C)
    a, b = oracle.operands_f64("bf16", A, B)
    bad = D.copy()
    bad[32:48, 64:80] = 0.0
    ok, _ = check.freivalds_blocks(bad, a, b, C, block=16)
    assert not ok
    bad = D.copy()
    bad[100, 7] = -bad[100, 7] + 1.0     # one flipped element
    ok, _ = check.freivalds_blocks(bad, a, b, C, block=16)
    assert not ok


def test_freivalds_integer_mode_catches_unit_change():
    A, B, C = _case(3, integer=True)
    D, _ = oracle.gemm_ref("bf16", A, B, C=C)
    a, b = oracle.operands_f64("bf16", A, B)
    assert check.freivalds_blocks(D, a, b, C, integer=True)[0]
    bad = D.copy()
    bad[11, 22] += 1
    assert not check.freivalds_blocks(bad, a, b, C, integer=True)[0]


# ---- sampling ------------------------------------------------------------------

def test_sample_indices():
    r1, f1 = inputs.sample_indices(4000, 3000, 2)
    r2, f2 = inputs.sample_indices(4000, 3000, 2)
    assert np.array_equal(r1, r2) and np.array_equal(f1, f2)
    assert len(np.unique(r1)) == 4096 and r1.min() >= 0 and r1.max() < 4000 * 3000
    assert {0, 2999, 3999 * 3000, 4000 * 3000 - 1} <= set(f1.tolist())
    r3, _ = inputs.sample_indices(4, 5, 0)
    assert sorted(r3.tolist()) == list(range(20))
