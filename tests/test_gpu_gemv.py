"""GPU parity of qgemv against the CPU oracle (element by element).

Small shapes span several lane tiles, several row groups and ragged row
tails; the workload shapes run at their full size in the launch
configuration the benchmark times, checked on sampled rows (every row for
the two small ones).  Tolerance: |y - y_ref| <= 1e-4 * sum|w x| + 1e-6 per
output (NaN agrees with NaN).
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

Q4_0, Q8_0, Q4_K, Q5_K, Q6_K, F32 = q.QG_Q4_0, q.QG_Q8_0, q.QG_Q4_K, q.QG_Q5_K, q.QG_Q6_K, q.QG_F32


def _matrix(fmt, rows, cols, seed):
    g = synth.rng(seed)
    if fmt == F32:
        return synth.f32_matrix(g, rows, cols, 1.0)
    return synth.matrix(g, fmt, rows, cols)


def _check(fmt, rows, cols, batch, seed, offset=0, what=""):
    W = _matrix(fmt, rows, cols, seed)
    X = synth.activations(synth.rng(seed + 7), batch, cols)
    Y = run_gemv(fmt, W, rows, cols, X, offset=offset)
    Yr, A = oracle.gemv(fmt, W, rows, cols, X)
    assert_agree(Y, Yr, A, what or f"fmt {fmt} {rows}x{cols} b{batch} off{offset}")


SMALL = {
    Q8_0: [(37, 96), (300, 1056), (5, 32)],
    Q4_0: [(37, 96), (300, 1056), (5, 32)],
    Q4_K: [(37, 256), (300, 2304), (3, 768)],
    Q5_K: [(37, 256), (300, 2304), (3, 768)],
    Q6_K: [(37, 256), (300, 2304), (3, 768)],
    F32: [(37, 100), (300, 1028), (5, 4)],
}


@pytest.mark.parametrize("fmt", list(SMALL))
@pytest.mark.parametrize("batch", [1, 2, 3, 4, 5, 6, 7, 8])
def test_small_shapes_every_batch(fmt, batch):
    for i, (rows, cols) in enumerate(SMALL[fmt]):
        _check(fmt, rows, cols, batch, 1000 + 10 * fmt + i)


@pytest.mark.parametrize("fmt", [Q8_0, Q4_0, Q4_K, Q5_K, Q6_K])
@pytest.mark.parametrize("batch", [1, 4, 8])
def test_weights_at_two_bytes_past_alignment(fmt, batch):
    _check(fmt, 41, 1024 if fmt in (Q8_0, Q4_0) else 768, batch, 2000 + fmt, offset=2)


@pytest.mark.parametrize("fmt,cols", [
    (Q4_K, 32768), (Q5_K, 32768), (Q6_K, 32768), (Q8_0, 16384), (Q4_0, 16384), (F32, 16384),
])
def test_widest_supported_rows(fmt, cols):
    # 512 lane tiles per row: eight waves per row group, reduced through LDS
    _check(fmt, 19, cols, 1, 3000 + fmt)


@pytest.mark.parametrize("fmt", [Q8_0, Q4_0])
def test_rows_past_the_lane_tile_limit_at_batch_1(fmt):
    # 513 blocks of 32: more than 512 lane tiles, within the matrix-core
    # kernel's activation image; the row's last chunk holds one block
    _check(fmt, 45, 16416, 1, 3200 + fmt)


@pytest.mark.parametrize("fmt,cols", [(Q4_K, 16384), (Q4_0, 14336), (Q6_K, 8192)])
def test_wide_rows_large_batch(fmt, cols):
    # batch 8 on wide rows (many chunks per wave)
    _check(fmt, 23, cols, 8, 3100 + fmt)


@pytest.mark.parametrize("fmt", [Q8_0, Q4_0, Q4_K, Q5_K, Q6_K])
@pytest.mark.parametrize("batch", [9, 16, 33, 64])
def test_batch_above_eight(fmt, batch):
    # the batched matrix-core kernel: one or two batch blocks of 16 per
    # launch, launches of up to 32 rows (the last one partial)
    _check(fmt, 45, 512 if fmt in (Q8_0, Q4_0) else 768, batch, 3500 + fmt + batch)


def test_batch_32_full_size_headline_shape():
    case = synth.GEMV_CASES["q4_k_4096x4096"]
    W, X = synth.gemv_inputs(case, 32)
    Y = run_gemv(case.fmt, W, case.rows, case.cols, X)
    idx = _sample_rows(case.rows, 300, 77)
    Yr, A = oracle.gemv(case.fmt, W, case.rows, case.cols, X, row_idx=idx)
    assert_agree(Y[:, idx], Yr, A, "q4_k 4096x4096 b32 (sampled rows)")


@pytest.mark.parametrize("fmt,cols,batch,offset", [
    (Q5_K, 4096, 8, 0), (Q4_0, 14336, 4, 2), (Q8_0, 12320, 8, 2), (Q6_K, 6144, 5, 0),
    (Q4_K, 8448, 3, 2),
])
def test_wide_rows_on_the_matrix_cores(fmt, cols, batch, offset):
    # rows wider than 1024 columns run on the batched kernels at every
    # batch (at batch 2..4 the f16 kernel takes only narrower rows); 8200
    # rows give a partial
    # last tile, the column ranges of the waves of a tile start at any
    # weight alignment
    _check(fmt, 8200, cols, batch, 3400 + fmt + batch, offset=offset)


@pytest.mark.parametrize("fmt,rows,cols,batch", [
    (Q4_K, 10000, 1024, 3), (Q8_0, 9000, 992, 2), (Q6_K, 300, 768, 4), (Q4_0, 37, 96, 2),
])
def test_narrow_rows_at_batch_2_to_4_run_the_f16_kernel(fmt, rows, cols, batch):
    # rows of at most 1024 columns at batch 2..4: the f16 matrix-core kernel
    # with the whole row's activations in LDS; 10000 and 9000 rows are more
    # tiles than two per CU, so the workgroups stream phases of chunks
    # through two buffers
    W = _matrix(fmt, rows, cols, 3600 + fmt + batch)
    X = synth.activations(synth.rng(3601 + fmt + batch), batch, cols)
    Y = run_gemv(fmt, W, rows, cols, X)
    assert q.qg_last_kernel() == "mx_f16"
    Yr, A = oracle.gemv(fmt, W, rows, cols, X)
    assert_agree(Y, Yr, A, f"f16 kernel fmt {fmt} {rows}x{cols} b{batch}")


@pytest.mark.parametrize("fmt,cols,batch", [(Q4_0, 14368, 4), (Q8_0, 12320, 3), (Q4_K, 32768, 1)])
def test_activations_staged_in_several_rounds(fmt, cols, batch):
    # batch * cols floats exceed one round of the LDS stage (32 floats per
    # thread); the last round is partial
    _check(fmt, 9, cols, batch, 3300 + fmt)


@pytest.mark.parametrize("fmt,cols", [(Q4_K, 33024), (Q8_0, 65536), (F32, 16388)])
def test_too_wide_rows_are_refused(fmt, cols):
    # wider than both the matrix-core kernel's LDS activation image and the
    # VALU kernel's 512 lane tiles per row
    W = torch.zeros(q.qg_row_bytes(fmt, cols) * 2 + 64, dtype=torch.uint8, device="cuda")
    X = torch.zeros(cols, device="cuda")
    Y = torch.zeros(2, device="cuda")
    with pytest.raises(q.QGError) as e:
        q.qgemv(fmt, W, 2, cols, X, Y, 1)
    assert e.value.code == q.QG_EUNSUPPORTED


def test_single_row_and_single_block():
    for fmt, cols in [(Q8_0, 32), (Q4_0, 32), (Q4_K, 256), (Q5_K, 256), (Q6_K, 256)]:
        _check(fmt, 1, cols, 1, 4000 + fmt)


def test_nan_and_inf_scales_propagate():
    rows, cols = 6, 512
    W = synth.matrix(synth.rng(5000), Q6_K, rows, cols)
    W[1, 208:210] = np.frombuffer(np.float16(np.nan).tobytes(), np.uint8)
    W[3, 210 + 208:210 + 210] = np.frombuffer(np.float16(np.inf).tobytes(), np.uint8)
    X = synth.activations(synth.rng(5001), 1, cols)
    Y = run_gemv(Q6_K, W, rows, cols, X)
    Yr, A = oracle.gemv(Q6_K, W, rows, cols, X)
    assert np.isnan(Y[0, 1]) and np.isnan(Yr[0, 1])
    assert_agree(Y, Yr, A, "nan/inf scales")


def test_zero_weights_give_zero():
    for fmt, cols in [(Q8_0, 64), (Q4_K, 512), (Q6_K, 512)]:
        W = np.zeros((9, q.qg_row_bytes(fmt, cols)), np.uint8)
        X = synth.activations(synth.rng(6000), 3, cols)
        Y = run_gemv(fmt, W, 9, cols, X)
        assert np.array_equal(Y, np.zeros_like(Y))


def _zero_point_matrix(fmt, rows, cols, seed):
    # nonzero scales with every code at the format's zero point (q = 0,
    # nibble 8, q = 32): every dequantised weight is exactly 0
    W = _matrix(fmt, rows, cols, seed)
    B = W.reshape(-1, q.qg_block_bytes(fmt))
    if fmt == Q8_0:
        B[:, 2:34] = 0
    elif fmt == Q4_0:
        B[:, 2:18] = 0x88
    else:
        B[:, 0:128] = 0
        B[:, 128:192] = 0xAA
    return W


@pytest.mark.parametrize("fmt", [Q8_0, Q4_0, Q6_K])
@pytest.mark.parametrize("batch", [1, 2, 3, 4, 8, 16])
def test_codes_at_the_zero_point_give_exact_zero(fmt, batch):
    # the VALU kernels (batch 1) and the matrix-core kernel (batch >= 2)
    # carry the code offset exactly: a row of zero weights gives +-0
    rows, cols = 45, 512
    W = _zero_point_matrix(fmt, rows, cols, 6200 + fmt)
    X = synth.activations(synth.rng(6201 + batch), batch, cols)
    Y = run_gemv(fmt, W, rows, cols, X)
    assert np.array_equal(Y, np.zeros_like(Y))
    Yr, A = oracle.gemv(fmt, W, rows, cols, X)
    assert np.array_equal(Yr, np.zeros_like(Yr))


@pytest.mark.parametrize("fmt", [Q8_0, Q4_0, Q6_K])
@pytest.mark.parametrize("batch", [2, 4, 8])
def test_zero_point_blocks_inside_random_rows(fmt, batch):
    # every other block of a random matrix at its zero point, large
    # activations: the zero blocks add nothing on the matrix cores either
    rows, cols = 70, 2048
    W = _matrix(fmt, rows, cols, 6300 + fmt)
    Z = _zero_point_matrix(fmt, rows, cols, 6300 + fmt)
    bb = q.qg_block_bytes(fmt)
    Wb, Zb = W.reshape(-1, bb), Z.reshape(-1, bb)
    Wb[::2] = Zb[::2]
    X = 1e3 * synth.activations(synth.rng(6301 + batch), batch, cols)
    Y = run_gemv(fmt, W, rows, cols, X)
    Yr, A = oracle.gemv(fmt, W, rows, cols, X)
    assert_agree(Y, Yr, A, f"fmt {fmt} b{batch} half zero-point blocks")


def test_q8_0_code_minus_128():
    W = synth.matrix(synth.rng(6100), Q8_0, 4, 64)
    W[:, 2] = 0x80
    X = synth.activations(synth.rng(6101), 2, 64)
    Y = run_gemv(Q8_0, W, 4, 64, X)
    Yr, A = oracle.gemv(Q8_0, W, 4, 64, X)
    assert_agree(Y, Yr, A, "q8_0 -128")


def test_run_to_run_bitwise_identical():
    W = synth.matrix(synth.rng(7000), Q4_K, 1000, 4096)
    X = synth.activations(synth.rng(7001), 4, 4096)
    a = run_gemv(Q4_K, W, 1000, 4096, X)
    b = run_gemv(Q4_K, W, 1000, 4096, X)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ------------------------------------------------ workload shapes, full size

def _sample_rows(rows, n, seed):
    g = np.random.default_rng(seed)
    idx = np.unique(np.concatenate([np.arange(min(64, rows)), np.arange(max(0, rows - 64), rows),
                                    g.integers(0, rows, n)]))
    return idx


@pytest.mark.parametrize("name", list(synth.GEMV_CASES))
def test_workload_full_size(name):
    case = synth.GEMV_CASES[name]
    for batch in case.batches:
        W, X = synth.gemv_inputs(case, batch)
        Y = run_gemv(case.fmt, W, case.rows, case.cols, X)
        if case.rows * case.cols <= 4096 * 4096:
            Yr, A = oracle.gemv(case.fmt, W, case.rows, case.cols, X)
            assert_agree(Y, Yr, A, f"{name} b{batch}")
        else:
            idx = _sample_rows(case.rows, 1500, case.seed + batch)
            Yr, A = oracle.gemv(case.fmt, W, case.rows, case.cols, X, row_idx=idx)
            assert_agree(Y[:, idx], Yr, A, f"{name} b{batch} (sampled rows)")
            assert np.isfinite(Y).all()


def _q6_k_set_zero_point(W, rows, cols, col):
    # code q = 32 (weight 0) at column col of every row: the low nibble of
    # ql[64h + 32(t%2) + l] (nibble t/2) and bits 2t..2t+1 of qh[32h + l]
    rb = q.qg_row_bytes(Q6_K, cols)
    Wr = W.reshape(rows, rb)
    sb, e = divmod(int(col), 256)
    h, t, l = e // 128, (e % 128) // 32, e % 32
    o = 210 * sb
    iql = o + 64 * h + 32 * (t % 2) + l
    nib = 4 * (t // 2)
    Wr[:, iql] &= np.uint8(0xFF ^ (0xF << nib))
    iqh = o + 128 + 32 * h + l
    Wr[:, iqh] = (Wr[:, iqh] & np.uint8(0xFF ^ (0x3 << (2 * t)))) | np.uint8(0x2 << (2 * t))


@pytest.mark.parametrize("batch", [1, 4])
def test_q6_k_outlier_activations(batch):
    # outlier columns 64x the typical magnitude in a third of the 16-column
    # runs, with every row's code at the zero point in those columns (the
    # case where a run's error bound 2^-22 * max|x| * sum|w| is largest
    # against sum |w x|): inside the tolerance at this dynamic range
    rows, cols = 96, 4096
    W = _matrix(Q6_K, rows, cols, 6400 + batch)
    X = synth.activations(synth.rng(6401 + batch), batch, cols)
    g = synth.rng(6402 + batch)
    cols_out = g.choice(cols, size=cols // 48, replace=False)
    X[:, cols_out] *= 64.0
    for c in cols_out:
        _q6_k_set_zero_point(W, rows, cols, c)
    Wd = oracle.dequant_matrix(Q6_K, W, rows, cols)
    assert np.all(Wd[:, cols_out] == 0)
    Y = run_gemv(Q6_K, W, rows, cols, X)
    Yr, A = oracle.gemv(Q6_K, W, rows, cols, X)
    assert_agree(Y, Yr, A, f"q6_k outliers b{batch}")
