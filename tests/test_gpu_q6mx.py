"""GPU parity of the batch-1 Q6_K GEMV on the matrix cores (int8 digit-plane
products, 16 weight rows per instruction) against the oracle.

Every row width the kernel takes (multiples of 256 columns up to 2048, of
512 up to 4096: one to eight waves per workgroup, four or eight 64-column
tiles per wave), row counts with a partial last block of 16 rows, weights
at 0 and 2 bytes past 4-byte alignment (rows of 210 bytes put odd rows at
2 mod 4), and the width the kernel does not take.  At batch 2 matrices of
16 MiB or more (the lm_head on sampled rows, three widths on every row)
run the two-row kernel, each row bit-identical to its batch-1 result;
smaller matrices the batched kernels; the lm_head at batch 3 and 4 runs
launches of two rows and one.  Tolerance as for every
GEMV: |y - y_ref| <= 1e-4 * sum|w x| + 1e-6 per output.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from parity import assert_agree

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gguf_quant_dequant_amd as q  # noqa: E402
from gpu_util import run_gemv  # noqa: E402

Q6_K = q.QG_Q6_K


def _check(rows, cols, seed, offset=0, kernel="mfma_i8_q6k"):
    W = synth.matrix(synth.rng(seed), Q6_K, rows, cols)
    X = synth.activations(synth.rng(seed + 1), 1, cols)
    Y = run_gemv(Q6_K, W, rows, cols, X, offset=offset)
    assert q.qg_last_kernel() == kernel
    Yr, A = oracle.gemv(Q6_K, W, rows, cols, X)
    assert_agree(Y, Yr, A, f"q6_k {rows}x{cols} off{offset}")


@pytest.mark.parametrize("cols", [256, 512, 768, 1024, 1280, 1536, 1792, 2048, 3072, 4096])
@pytest.mark.parametrize("offset", [0, 2])
def test_every_row_width(cols, offset):
    _check(53, cols, 7000 + cols // 256 + 50 * offset, offset)


@pytest.mark.parametrize("rows", [1, 15, 16, 17, 33, 1000])
def test_row_counts_around_the_block(rows):
    _check(rows, 2048, 7100 + rows)


def test_widths_it_does_not_take_run_on_the_vector_alus():
    # 2304 columns: 36 tiles, neither eight nor nine waves of a whole number
    # of four- or eight-tile ranges within eight waves
    _check(21, 2304, 7200, kernel="valu_q6k_int")


def test_zero_point_codes_and_outliers():
    # every code of some blocks at q = 32 (an exact zero), and activations
    # spanning several orders of magnitude within a 16-column run
    rows, cols = 40, 2048
    W = synth.matrix(synth.rng(7300), Q6_K, rows, cols)
    rb = q.qg_row_bytes(Q6_K, cols)
    for r in range(0, rows, 3):
        for sb in range(0, cols // 256, 2):
            o = sb * 210
            W[r, o:o + 128] = 0           # low four bits 0
            W[r, o + 128:o + 192] = 0xAA  # top two bits 2: q = 32
    X = synth.activations(synth.rng(7301), 1, cols)
    X[0, ::37] *= 1e4
    X[0, 5::41] *= 1e-4
    Y = run_gemv(Q6_K, W, rows, cols, X)
    assert q.qg_last_kernel() == "mfma_i8_q6k"
    Yr, A = oracle.gemv(Q6_K, W, rows, cols, X)
    assert_agree(Y, Yr, A, "q6_k zero points and outliers")
    assert rb == 1680


def test_lm_head_full_size_sampled_rows():
    case = synth.GEMV_CASES["q6_k_151936x2048"]
    W, X = synth.gemv_inputs(case, 1)
    Y = run_gemv(case.fmt, W, case.rows, case.cols, X)
    assert q.qg_last_kernel() == "mfma_i8_q6k"
    g = np.random.default_rng(91)
    idx = np.unique(np.concatenate([g.integers(0, case.rows, 2000),
                                    np.arange(16), np.arange(case.rows - 16, case.rows)]))
    Yr, A = oracle.gemv(case.fmt, W, case.rows, case.cols, X, row_idx=idx)
    assert_agree(Y[:, idx], Yr, A, "lm_head sampled rows")


def test_run_to_run_bitwise_identical():
    W = synth.matrix(synth.rng(7400), Q6_K, 300, 2048)
    X = synth.activations(synth.rng(7401), 1, 2048)
    a = run_gemv(Q6_K, W, 300, 2048, X)
    b = run_gemv(Q6_K, W, 300, 2048, X)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("rows,cols", [(53, 1024), (1000, 2048), (17, 4096)])
def test_batch_two_on_smaller_matrices_runs_the_batched_kernels(rows, cols):
    seed = 7400 + cols // 256 + rows
    W = synth.matrix(synth.rng(seed), Q6_K, rows, cols)
    X = synth.activations(synth.rng(seed + 1), 2, cols)
    Y = run_gemv(Q6_K, W, rows, cols, X)
    assert q.qg_last_kernel() != "mfma_i8_q6k"
    Yr, A = oracle.gemv(Q6_K, W, rows, cols, X)
    assert_agree(Y, Yr, A, f"q6_k batch 2 {rows}x{cols}")


def test_lm_head_batch_two_sampled_rows():
    # 255 MB of weights: batch 2 runs the two-row kernel, whose every row is
    # its batch-1 result bit for bit (the same sums in the same order)
    case = synth.GEMV_CASES["q6_k_151936x2048"]
    W, X = synth.gemv_inputs(case, 2)
    Y = run_gemv(case.fmt, W, case.rows, case.cols, X)
    assert q.qg_last_kernel() == "mfma_i8_q6k"
    g = np.random.default_rng(92)
    idx = np.unique(np.concatenate([g.integers(0, case.rows, 1000),
                                    np.arange(16), np.arange(case.rows - 16, case.rows)]))
    Yr, A = oracle.gemv(case.fmt, W, case.rows, case.cols, X, row_idx=idx)
    assert_agree(Y[:, idx], Yr, A, "lm_head batch 2 sampled rows")
    Y1 = run_gemv(case.fmt, W, case.rows, case.cols, X[1:2])
    assert np.array_equal(Y[1:2].view(np.uint32), Y1.view(np.uint32))


@pytest.mark.parametrize("rows,cols,offset", [(10240, 2048, 0), (14000, 1536, 2), (5200, 4096, 0)])
def test_two_row_kernel(rows, cols, offset):
    # matrices of 16 MiB or more at batch 2: both rows against each tile's
    # codes (eight, three and eight waves per workgroup), every output row
    seed = 7600 + cols // 256
    W = synth.matrix(synth.rng(seed), Q6_K, rows, cols)
    assert W.nbytes >= 16 << 20
    X = synth.activations(synth.rng(seed + 1), 2, cols)
    Y = run_gemv(Q6_K, W, rows, cols, X, offset=offset)
    assert q.qg_last_kernel() == "mfma_i8_q6k"
    Yr, A = oracle.gemv(Q6_K, W, rows, cols, X)
    assert_agree(Y, Yr, A, f"q6_k two rows {rows}x{cols} off{offset}")
    Y1 = run_gemv(Q6_K, W, rows, cols, X[1:2], offset=offset)
    assert np.array_equal(Y[1:2].view(np.uint32), Y1.view(np.uint32))


@pytest.mark.parametrize("batch", [3, 4])
def test_lm_head_batch_three_and_four(batch):
    # 255 MB of weights at batch 3-4: launches of two rows and one, every
    # row bit-identical to its batch-1 result
    case = synth.GEMV_CASES["q6_k_151936x2048"]
    W, X = synth.gemv_inputs(case, batch)
    Y = run_gemv(case.fmt, W, case.rows, case.cols, X)
    assert q.qg_last_kernel() == "mfma_i8_q6k"
    g = np.random.default_rng(93 + batch)
    idx = np.unique(np.concatenate([g.integers(0, case.rows, 600),
                                    np.arange(16), np.arange(case.rows - 16, case.rows)]))
    Yr, A = oracle.gemv(case.fmt, W, case.rows, case.cols, X, row_idx=idx)
    assert_agree(Y[:, idx], Yr, A, f"lm_head batch {batch} sampled rows")
    b = batch - 1
    Y1 = run_gemv(case.fmt, W, case.rows, case.cols, X[b:b + 1])
    assert np.array_equal(Y[b:b + 1].view(np.uint32), Y1.view(np.uint32))
