"""GPU parity of qgemv's batch 2-32 kernel for tall matrices (activation
operands shared through LDS by a workgroup's 4 row tiles, two column ranges
per workgroup added through LDS, no workspace) against the oracle.

qgemv takes it when the matrix has at least 192 groups of 4 row tiles
(12,241 rows or more) and 4 or more chunks of 256 columns, for every
launch of 2 to 32 batch rows; qgemv_ws up to 16 rows.  Every block
format at batch 2, 3, 5 and 8 (one operand plane), 9, 16 (two), 17, 24 and
32 (four, the second block of 16 rows partial or whole; Q8_0 there on
the other kernel, its LDS need too large), 40 (two launches)
and 33 (a last launch of one row on the other kernel); row counts with a partial last group and a
partial last tile; an odd chunk count (the two ranges of unequal length)
with a partial last chunk; weights 2 bytes past 4-byte alignment; the full
Q5_K 14336 x 4096 workload on sampled rows; zero weights; determinism.
Q6_K at batch 2 runs the batch-1 matrix-core kernel once per row where
that kernel takes the width, so its batch-2 case here has 2304 columns,
a width that kernel refuses.  Tolerance as for every GEMV: |y - y_ref| <= 1e-4 * sum|w x| + 1e-6 per
output.
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

Q4_0, Q8_0, Q4_K, Q5_K, Q6_K = q.QG_Q4_0, q.QG_Q8_0, q.QG_Q4_K, q.QG_Q5_K, q.QG_Q6_K
BLOCK = [Q8_0, Q4_0, Q4_K, Q5_K, Q6_K]
ROWS = 12_290  # 769 tiles, the last of 2 rows; 193 groups, the last of one tile


def _sampled(rows, seed):
    g = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(40), np.arange(rows - 40, rows),
                                     g.integers(0, rows, 400)]))


def _check(fmt, rows, cols, batch, seed, offset=0, sample=True, kernel="gemm_ks2_bf16"):
    W = synth.matrix(synth.rng(seed), fmt, rows, cols)
    X = synth.activations(synth.rng(seed + 1), batch, cols)
    Y = run_gemv(fmt, W, rows, cols, X, offset=offset)
    assert q.qg_last_kernel() == kernel
    idx = _sampled(rows, seed) if sample else None
    Yr, A = oracle.gemv(fmt, W, rows, cols, X, row_idx=idx)
    Yg = Y[:, idx] if sample else Y
    assert_agree(Yg, Yr, A, f"ks2 fmt {fmt} {rows}x{cols} b{batch} off{offset}")
    assert np.isfinite(Y).all()


@pytest.mark.parametrize("fmt", BLOCK)
@pytest.mark.parametrize("batch", [2, 3, 5, 8])
def test_every_format_and_batch(fmt, batch):
    cols = 2304 if fmt == Q6_K and batch <= 2 else 1024
    _check(fmt, ROWS, cols, batch, 9000 + 10 * fmt + batch)


@pytest.mark.parametrize("fmt", BLOCK)
def test_odd_chunk_count_and_partial_last_chunk(fmt):
    # 5 chunks: ranges of 2 and 3 chunks; for the 32-column formats the last
    # chunk holds one block
    cols = 1056 if fmt in (Q8_0, Q4_0) else 1280
    _check(fmt, ROWS, cols, 4, 9100 + fmt)


@pytest.mark.parametrize("fmt", BLOCK)
def test_weights_two_bytes_past_alignment(fmt):
    _check(fmt, ROWS, 1024, 6, 9200 + fmt, offset=2)


def test_every_row_of_one_matrix():
    _check(Q4_K, 12_304, 1024, 8, 9300, sample=False)


def test_below_the_threshold_runs_the_batch8_kernel():
    W = synth.matrix(synth.rng(9400), Q4_K, 12_224, 1024)  # 191 groups of 4 tiles
    X = synth.activations(synth.rng(9401), 8, 1024)
    run_gemv(Q4_K, W, 12_224, 1024, X)
    assert q.qg_last_kernel() == "gemm_bf16"
    W = synth.matrix(synth.rng(9402), Q4_K, ROWS, 768)    # 3 chunks
    X = synth.activations(synth.rng(9403), 8, 768)
    run_gemv(Q4_K, W, ROWS, 768, X)
    assert q.qg_last_kernel() == "gemm_bf16"


@pytest.mark.parametrize("batch", [4, 8])
def test_q5_k_workload_full_size(batch):
    case = synth.GEMV_CASES["q5_k_14336x4096"]
    W, X = synth.gemv_inputs(case, batch)
    Y = run_gemv(case.fmt, W, case.rows, case.cols, X)
    assert q.qg_last_kernel() == "gemm_ks2_bf16"
    idx = _sampled(case.rows, case.seed + batch)
    Yr, A = oracle.gemv(case.fmt, W, case.rows, case.cols, X, row_idx=idx)
    assert_agree(Y[:, idx], Yr, A, f"ks2 q5_k workload b{batch} (sampled rows)")


@pytest.mark.parametrize("fmt", [Q4_K, Q5_K])
def test_rows_of_zero_weights_give_zero(fmt):
    rows, cols = ROWS, 1024
    W = synth.matrix(synth.rng(9500 + fmt), fmt, rows, cols)
    bb = 144 if fmt == Q4_K else 176
    Wr = W.reshape(rows, -1)
    zero_rows = np.arange(0, rows, 97)
    for sb in range(cols // 256):
        o = sb * bb
        Wr[zero_rows, o + 2:o + 4] = 0
        Wr[zero_rows, o + 16:o + bb] = 0
    X = synth.activations(synth.rng(9501), 8, cols)
    Y = run_gemv(fmt, W, rows, cols, X)
    assert q.qg_last_kernel() == "gemm_ks2_bf16"
    assert np.all(np.abs(Y[:, zero_rows]) <= 1e-6), np.abs(Y[:, zero_rows]).max()


def test_run_to_run_bitwise_identical():
    W = synth.matrix(synth.rng(9600), Q5_K, ROWS, 1024)
    X = synth.activations(synth.rng(9601), 8, 1024)
    a = run_gemv(Q5_K, W, ROWS, 1024, X)
    b = run_gemv(Q5_K, W, ROWS, 1024, X, offset=0)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("fmt", BLOCK)
@pytest.mark.parametrize("batch", [9, 16, 17, 24, 32])
def test_every_format_above_eight_rows(fmt, batch):
    # Q8_0's weight slots leave no room for the four-plane images of 17-32
    # rows in LDS: there it runs the other batched kernel
    kernel = "gemm_bf16" if fmt == Q8_0 and batch > 16 else "gemm_ks2_bf16"
    _check(fmt, ROWS, 1024, batch, 9500 + 10 * fmt + batch, kernel=kernel)


@pytest.mark.parametrize("fmt", [Q4_K, Q4_0])
def test_two_launches(fmt):
    # 40 rows: launches of 32 and 8 rows, both on the two-range kernel
    _check(fmt, ROWS, 1280, 40, 9600 + fmt)


def test_a_last_launch_of_one_row_runs_the_other_kernel():
    W = synth.matrix(synth.rng(9700), Q4_K, ROWS, 1024)
    X = synth.activations(synth.rng(9701), 33, 1024)
    Y = run_gemv(Q4_K, W, ROWS, 1024, X)
    assert q.qg_last_kernel() == "gemm_bf16"
    idx = _sampled(ROWS, 9700)
    Yr, A = oracle.gemv(Q4_K, W, ROWS, 1024, X, row_idx=idx)
    assert_agree(Y[:, idx], Yr, A, "ks2 b33 (32 + 1)")


@pytest.mark.parametrize("batch,two_range", [(12, True), (16, True), (17, False), (32, False)])
def test_qgemv_ws_takes_it_up_to_sixteen_rows(batch, two_range):
    from gpu_util import DeviceBytes, dev
    W = synth.matrix(synth.rng(9800 + batch), Q5_K, ROWS, 1024)
    X = synth.activations(synth.rng(9801 + batch), batch, 1024)
    need = q.qgemv_ws_bytes(Q5_K, ROWS, 1024, batch)
    assert (need == 0) == two_range
    Wd = DeviceBytes(W)
    Xd = torch.from_numpy(X).to(dev())
    Yd = torch.full((batch, ROWS), float("nan"), device=dev())
    ws = torch.full((need,), 255, dtype=torch.uint8, device=dev()) if need else None
    q.qgemv_ws(Q5_K, Wd.ptr, ROWS, 1024, Xd, Yd, batch, ws)
    torch.cuda.synchronize()
    Y = Yd.cpu().numpy()
    assert q.qg_last_kernel() == "gemm_ws_bf16"
    idx = _sampled(ROWS, 9800 + batch)
    Yr, A = oracle.gemv(Q5_K, W, ROWS, 1024, X, row_idx=idx)
    assert_agree(Y[:, idx], Yr, A, f"qgemv_ws b{batch}")
    if two_range:
        # the same kernel as qgemv: the same bits
        Y2 = run_gemv(Q5_K, W, ROWS, 1024, X)
        assert np.array_equal(Y.view(np.uint32), Y2.view(np.uint32))
