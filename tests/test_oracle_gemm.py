"""Pins of the oracle's block-scaled grouped GEMM: numpy float64 matmul of the
fully dequantised operands (a different formulation: dequantise first, one
product per group), an exact small-integer case, power-of-two scaling, the
dense special case G = 1, empty groups, and the row-sampled variant."""

import numpy as np
import pytest

from oracle import (dequant_act, dequant_weight, e4m3_encode, grouped_gemm, grouped_gemm_rows,
                    quant_act_1x128, quant_weight_128x128)

RNG = np.random.default_rng(5)


def _problem(M_per, N, K, rng=RNG):
    G = len(M_per)
    M = int(sum(M_per))
    a = rng.standard_normal((M, K)).astype(np.float32) * np.exp2(rng.integers(-3, 3, (M, 1))).astype(np.float32)
    w = (rng.standard_normal((G, N, K)) * 0.02).astype(np.float32)
    aq, as_ = quant_act_1x128(a)
    bq, bs = quant_weight_128x128(w)
    off = np.concatenate([[0], np.cumsum(M_per)]).astype(np.int32)
    return aq, as_, bq, bs, off


def _dequant_matmul(aq, as_, bq, bs, off):
    A = dequant_act(aq, as_)
    B = dequant_weight(bq, bs)
    C = np.zeros((A.shape[0], B.shape[1]))
    for g in range(B.shape[0]):
        C[off[g]:off[g + 1]] = A[off[g]:off[g + 1]] @ B[g].T
    return C


@pytest.mark.parametrize("M_per,N,K", [([5, 0, 17, 1], 256, 384), ([40], 128, 640), ([3, 9], 384, 128)])
def test_matches_dequantised_matmul(M_per, N, K):
    aq, as_, bq, bs, off = _problem(M_per, N, K)
    C, Mag = grouped_gemm(aq, as_, bq, bs, off)
    ref = _dequant_matmul(aq, as_, bq, bs, off)
    assert np.all(np.abs(C - ref) <= 1e-13 * Mag + 1e-300)
    assert np.all(Mag >= np.abs(C))


def test_transposed_weight_would_fail():
    """B is stored [N, K]; using it as [K, N] must not agree (N != K)."""
    aq, as_, bq, bs, off = _problem([8], 256, 256)
    C, _ = grouped_gemm(aq, as_, bq, bs, off)
    A = dequant_act(aq, as_)
    B = dequant_weight(bq, bs)[0]
    assert np.allclose(C, A @ B.T, rtol=1e-12, atol=1e-12)
    assert not np.allclose(C, A @ B, rtol=1e-3, atol=1e-3)


def test_exact_small_integers():
    """Codes of small integers with unit scales: every partial sum is an
    integer, so the result is the exact integer matmul."""
    M, N, K = 24, 256, 512
    ia = RNG.integers(-8, 9, (M, K))
    ib = RNG.integers(-8, 9, (1, N, K))
    aq = e4m3_encode(ia.astype(np.float32))
    bq = e4m3_encode(ib.astype(np.float32))
    as_ = np.ones((M, K // 128), np.float32)
    bs = np.ones((1, N // 128, K // 128), np.float32)
    C, _ = grouped_gemm(aq, as_, bq, bs, np.array([0, M]))
    assert np.array_equal(C, (ia @ ib[0].T).astype(np.float64))


def test_power_of_two_scaling():
    aq, as_, bq, bs, off = _problem([6, 10], 128, 256)
    C, _ = grouped_gemm(aq, as_, bq, bs, off)
    C2, _ = grouped_gemm(aq, (as_ * np.float32(8)).astype(np.float32), bq, bs, off)
    C3, _ = grouped_gemm(aq, as_, bq, (bs * np.float32(0.25)).astype(np.float32), off)
    assert np.array_equal(C2, 8 * C) and np.array_equal(C3, 0.25 * C)


def test_scale_indexing_per_chunk_and_block():
    """Changing one activation tile scale or one weight block scale changes
    exactly the outputs it must."""
    aq, as_, bq, bs, off = _problem([16], 256, 384)
    C, _ = grouped_gemm(aq, as_, bq, bs, off, with_mag=False)
    as2 = as_.copy()
    as2[3, 1] *= 2
    C2, _ = grouped_gemm(aq, as2, bq, bs, off, with_mag=False)
    changed = np.any(C2 != C, axis=1)
    assert changed[3] and changed.sum() == 1
    bs2 = bs.copy()
    bs2[0, 1, 2] *= 2
    C3, _ = grouped_gemm(aq, as_, bq, bs2, off, with_mag=False)
    cols = np.any(C3 != C, axis=0)
    assert cols[128:256].all() and not cols[:128].any()


def test_rows_variant_and_empty_groups():
    aq, as_, bq, bs, off = _problem([0, 7, 0, 12, 0], 128, 256)
    C, Mag = grouped_gemm(aq, as_, bq, bs, off)
    rows = np.array([0, 6, 7, 18])
    Cr, Mr = grouped_gemm_rows(aq, as_, bq, bs, off, rows)
    assert np.array_equal(Cr, C[rows]) and np.array_equal(Mr, Mag[rows])


def test_gemm_errors():
    aq, as_, bq, bs, off = _problem([4], 128, 256)
    with pytest.raises(ValueError):
        grouped_gemm(aq, as_, bq, bs, np.array([0, 3]))
    with pytest.raises(ValueError):
        grouped_gemm(aq, as_, bq, bs, np.array([1, 4]))
