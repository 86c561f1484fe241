"""GPU parity of qgemv_ws (the batched GEMV with activation operands shared
through LDS and a caller-provided workspace) against the oracle.

Every block format at batch 2..64 (one, two or three launches of up to 32
rows; the packed mode at 8 rows or fewer, one and two blocks of 16 batch
rows above), row counts with a partial last group of 8 tiles and a partial
last tile, rows split over several workgroups (the workspace path) and over
one (no workspace), a partial last chunk of 256 columns, weights 2 bytes
past 4-byte alignment, the workload shapes at full size on sampled rows,
the workspace checks, one workspace reused by calls of other shapes,
run-to-run determinism, and the batch 2..8 calls on rows of 16 or fewer
chunks that would be split over workgroups, which run qgemv (no
workspace, qgemv's bits).  Tolerance as for every
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
from gpu_util import DeviceBytes, dev  # noqa: E402

Q4_0, Q8_0, Q4_K, Q5_K, Q6_K, F32 = q.QG_Q4_0, q.QG_Q8_0, q.QG_Q4_K, q.QG_Q5_K, q.QG_Q6_K, q.QG_F32
BLOCK = [Q8_0, Q4_0, Q4_K, Q5_K, Q6_K]


def run_ws(fmt, W, rows, cols, X, offset=0, ws_pad=0):
    Wd = DeviceBytes(W, offset)
    Xd = torch.from_numpy(np.ascontiguousarray(X, dtype=np.float32)).to(dev())
    Y = torch.full((X.shape[0], rows), float("nan"), dtype=torch.float32, device=dev())
    need = q.qgemv_ws_bytes(fmt, rows, cols, X.shape[0])
    ws = torch.full((need + ws_pad,), 255, dtype=torch.uint8, device=dev()) if need else None
    q.qgemv_ws(fmt, Wd.ptr, rows, cols, Xd, Y, X.shape[0], ws)
    torch.cuda.synchronize()
    return Y.cpu().numpy(), need


def _check(fmt, rows, cols, batch, seed, offset=0, want_ws=None):
    g = synth.rng(seed)
    W = synth.f32_matrix(g, rows, cols, 1.0) if fmt == F32 else synth.matrix(g, fmt, rows, cols)
    X = synth.activations(synth.rng(seed + 7), batch, cols)
    Y, need = run_ws(fmt, W, rows, cols, X, offset)
    if fmt != F32 and batch > 1:
        assert q.qg_last_kernel() == "gemm_ws_bf16"
    if want_ws is not None:
        assert (need > 0) == want_ws, need
    Yr, A = oracle.gemv(fmt, W, rows, cols, X)
    assert_agree(Y, Yr, A, f"ws fmt {fmt} {rows}x{cols} b{batch} off{offset}")


@pytest.mark.parametrize("fmt", BLOCK)
@pytest.mark.parametrize("batch", [2, 3, 5, 8, 9, 16, 17, 32, 33, 64])
def test_every_format_and_batch_with_split_rows(fmt, batch):
    # 300 rows: 19 tiles in 3 groups of 8 (the last partial, its last tile
    # partial); 4352 columns: 17 chunks over several workgroups (at 16 or
    # fewer, batch 2..8 runs qgemv)
    cols = 4352
    _check(fmt, 300, cols, batch, 8000 + 100 * fmt + batch, want_ws=True)


@pytest.mark.parametrize("fmt", BLOCK)
@pytest.mark.parametrize("batch", [4, 8, 24])
def test_rows_on_one_workgroup_and_a_partial_chunk(fmt, batch):
    # 480 / 768 columns: two or three chunks, one column range (no
    # workspace); the last chunk partial for the 32-column formats
    cols = 480 if fmt in (Q8_0, Q4_0) else 768
    _check(fmt, 45, cols, batch, 8100 + 10 * fmt + batch, want_ws=False)


@pytest.mark.parametrize("fmt", BLOCK)
@pytest.mark.parametrize("batch", [3, 8, 20])
def test_weights_two_bytes_past_alignment(fmt, batch):
    cols = 4384 if fmt in (Q8_0, Q4_0) else 4608
    _check(fmt, 130, cols, batch, 8200 + 10 * fmt + batch, offset=2)


def test_batch_one_and_f32_run_qgemv():
    _check(Q4_K, 37, 512, 1, 8300)
    _check(F32, 37, 1028, 5, 8301)
    assert q.qgemv_ws_bytes(Q4_K, 4096, 4096, 1) == 0
    assert q.qgemv_ws_bytes(F32, 4096, 4096, 8) == 0


@pytest.mark.parametrize("name,batch", [("q5_k_14336x4096", 8), ("q4_0_4096x14336", 8),
                                        ("q4_0_4096x14336", 4), ("q4_k_4096x4096", 32),
                                        ("q4_k_4096x4096", 64)])
def test_workload_shapes_full_size(name, batch):
    case = synth.GEMV_CASES[name]
    W, X = synth.gemv_inputs(case, batch)
    Y, need = run_ws(case.fmt, W, case.rows, case.cols, X)
    assert q.qg_last_kernel() == "gemm_ws_bf16"
    g = np.random.default_rng(case.seed + batch)
    idx = np.unique(np.concatenate([np.arange(64), np.arange(case.rows - 64, case.rows),
                                    g.integers(0, case.rows, 300)]))
    Yr, A = oracle.gemv(case.fmt, W, case.rows, case.cols, X, row_idx=idx)
    assert_agree(Y[:, idx], Yr, A, f"ws {name} b{batch} (sampled rows)")
    assert np.isfinite(Y).all()


def test_workspace_checks():
    rows, cols, batch = 300, 4352, 8
    W = synth.matrix(synth.rng(8400), Q4_K, rows, cols)
    Wd = DeviceBytes(W)
    X = torch.zeros((batch, cols), device=dev())
    Y = torch.zeros((batch, rows), device=dev())
    need = q.qgemv_ws_bytes(Q4_K, rows, cols, batch)
    assert need > 0 and need % 16 == 0
    with pytest.raises(q.QGError) as e:
        q.qgemv_ws(Q4_K, Wd.ptr, rows, cols, X, Y, batch, None, 0)
    assert e.value.code == q.QG_EINVAL
    ws = torch.empty(need + 16, dtype=torch.uint8, device=dev())
    with pytest.raises(q.QGError) as e:
        q.qgemv_ws(Q4_K, Wd.ptr, rows, cols, X, Y, batch, ws, need - 4)
    assert e.value.code == q.QG_EINVAL
    with pytest.raises(q.QGError) as e:
        q.qgemv_ws(Q4_K, Wd.ptr, rows, cols, X, Y, batch, ws.data_ptr() + 4, need)
    assert e.value.code == q.QG_EINVAL
    q.qgemv_ws(Q4_K, Wd.ptr, rows, cols, X, Y, batch, ws, need)
    torch.cuda.synchronize()
    assert not torch.any(Y).item()


def test_run_to_run_bitwise_identical():
    rows, cols, batch = 1000, 4352, 8
    W = synth.matrix(synth.rng(8500), Q5_K, rows, cols)
    X = synth.activations(synth.rng(8501), batch, cols)
    a, _ = run_ws(Q5_K, W, rows, cols, X)
    b, _ = run_ws(Q5_K, W, rows, cols, X, ws_pad=64)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("fmt", [Q4_K, Q5_K])
@pytest.mark.parametrize("batch", [2, 4, 8, 16, 32])
def test_k_quant_rows_of_zero_weights_give_zero(fmt, batch):
    # every super-block of every third row: nonzero d and sub-block scales,
    # dmin = 0 and all codes 0, so every weight is 0 and the output must be
    # 0 (the codes enter the matrix core as 128 + q; the 128 offset must
    # cancel exactly), through qgemv and qgemv_ws
    rows, cols = 150, 2048
    W = synth.matrix(synth.rng(8600 + fmt + batch), fmt, rows, cols)
    rb = q.qg_row_bytes(fmt, cols)
    bb = 144 if fmt == Q4_K else 176
    Wr = W.reshape(rows, rb)
    zero_rows = np.arange(0, rows, 3)
    for sb in range(cols // 256):
        o = sb * bb
        Wr[zero_rows, o + 2:o + 4] = 0          # dmin
        Wr[zero_rows, o + 16:o + bb] = 0        # (qh and) qs
    X = synth.activations(synth.rng(8700 + batch), batch, cols)
    Yr, A = oracle.gemv(fmt, W, rows, cols, X)
    assert np.all(Yr[:, zero_rows] == 0)
    Y, _ = run_ws(fmt, W, rows, cols, X)
    assert np.all(np.abs(Y[:, zero_rows]) <= 1e-6), np.abs(Y[:, zero_rows]).max()
    assert_agree(Y, Yr, A, f"ws zero rows fmt {fmt} b{batch}")
    from gpu_util import run_gemv
    Y2 = run_gemv(fmt, W, rows, cols, X)
    assert np.all(np.abs(Y2[:, zero_rows]) <= 1e-6), np.abs(Y2[:, zero_rows]).max()
    assert_agree(Y2, Yr, A, f"qgemv zero rows fmt {fmt} b{batch}")


def test_one_workspace_reused_by_calls_of_other_shapes():
    # no initial contents needed: one workspace of garbage bytes serves calls
    # of other shapes and sizes one after another
    shapes = [(Q4_0, 300, 4352, 8), (Q4_K, 1000, 4352, 4), (Q5_K, 150, 2048, 16),
              (Q4_0, 300, 4352, 8), (Q6_K, 600, 4096, 40), (Q4_K, 1000, 4352, 4)]
    need = max(q.qgemv_ws_bytes(f, r, c, b) for f, r, c, b in shapes)
    ws = torch.full((need,), 255, dtype=torch.uint8, device=dev())
    for i, (fmt, rows, cols, batch) in enumerate(shapes):
        W = synth.matrix(synth.rng(8800 + i), fmt, rows, cols)
        X = synth.activations(synth.rng(8900 + i), batch, cols)
        Wd = DeviceBytes(W)
        Xd = torch.from_numpy(X).to(dev())
        Y = torch.full((batch, rows), float("nan"), device=dev())
        q.qgemv_ws(fmt, Wd.ptr, rows, cols, Xd, Y, batch, ws, need)
        torch.cuda.synchronize()
        Yr, A = oracle.gemv(fmt, W, rows, cols, X)
        assert_agree(Y.cpu().numpy(), Yr, A, f"reused workspace, call {i}")


@pytest.mark.parametrize("fmt", BLOCK)
@pytest.mark.parametrize("batch", [2, 5, 8])
def test_short_rows_split_across_workgroups_run_qgemv(fmt, batch):
    # 300 x 4096 at batch 2..8: 16 chunks that the shared-operand kernel
    # would split over workgroups; qgemv's kernels run instead, with no
    # workspace, and give qgemv's bits
    rows, cols = 300, 4096
    assert q.qgemv_ws_bytes(fmt, rows, cols, batch) == 0
    g = synth.rng(8950 + fmt + batch)
    W = synth.matrix(g, fmt, rows, cols)
    X = synth.activations(synth.rng(8960 + batch), batch, cols)
    Y, _ = run_ws(fmt, W, rows, cols, X)
    assert q.qg_last_kernel() != "gemm_ws_bf16"
    from gpu_util import run_gemv
    Y2 = run_gemv(fmt, W, rows, cols, X)
    assert np.array_equal(Y.view(np.uint32), Y2.view(np.uint32))
    Yr, A = oracle.gemv(fmt, W, rows, cols, X)
    assert_agree(Y, Yr, A, f"ws via qgemv fmt {fmt} b{batch}")
    # at batch 9 the shared-operand kernel takes the same shape
    X9 = synth.activations(synth.rng(8970), 9, cols)
    assert q.qgemv_ws_bytes(fmt, rows, cols, 9) > 0
    run_ws(fmt, W, rows, cols, X9)
    assert q.qg_last_kernel() == "gemm_ws_bf16"
