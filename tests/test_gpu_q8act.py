"""GPU parity of qgemv_q8act (int8-quantised activations, integer dot
products) against the oracle's int8-activation GEMV, which quantises the
activations the same way and accumulates in f64.

Two checks on every result:

* against the oracle's int8-activation GEMV, per row
  1e-4 * sum |w * x_q| + 1e-6 (both sides quantise the activations with the
  same f32 operations; only the order and width of the sums differ);
* against the exact GEMV's oracle, which does not depend on how the
  quantiser is written: per row the departure is at most the quantisation
  bound sum |w| * d / 2 (d the group scale, taken from the exact
  activations as max|x| / 127 in f64) plus the exact path's tolerance.
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

FMTS = [q.QG_Q8_0, q.QG_Q4_0, q.QG_Q4_K, q.QG_Q5_K, q.QG_Q6_K]


def run_q8(fmt, W, rows, cols, x, offset=0):
    Wd = DeviceBytes(W, offset)
    xd = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev())
    Y = torch.full((rows,), float("nan"), device=dev())
    q.qgemv_q8act(fmt, Wd.ptr, rows, cols, xd, Y)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def check_exact_bound(fmt, W, rows, cols, x, y, what, row_idx=None):
    """|y - exact| <= sum_c |w_c| * d(c) / 2 * (1 + 1e-3) + 1e-4 * sum |w x| + 1e-6 per
    row, with d = max |x| / 127 over the 16-column group (f64), exact from
    the exact GEMV's oracle.  row_idx: y holds only these rows of W."""
    x64 = np.asarray(x, np.float64)
    d = np.max(np.abs(x64.reshape(-1, 16)), axis=1) / 127.0
    Wsub = W.reshape(rows, -1) if row_idx is None else W.reshape(rows, -1)[row_idx]
    n = Wsub.shape[0]
    Wd = oracle.dequant_matrix(fmt, Wsub, n, cols)
    bound = np.abs(Wd) @ np.repeat(d, 16) / 2
    Ye, Ae = oracle.gemv(fmt, Wsub, n, cols, x[None].astype(np.float32))
    err = np.abs(np.asarray(y, np.float64) - Ye[0])
    ok = err <= bound * (1 + 1e-3) + 1e-4 * Ae[0] + 1e-6
    assert ok.all(), (what, int((~ok).sum()), float(np.max(err - bound)))
    return float(np.max(err / np.maximum(bound, 1e-30)))


def _check(fmt, rows, cols, seed, offset=0, x=None):
    g = synth.rng(seed)
    W = synth.matrix(g, fmt, rows, cols)
    if x is None:
        x = synth.activations(g, 1, cols)[0]
    y = run_q8(fmt, W, rows, cols, x, offset)
    what = f"q8act fmt {fmt} {rows}x{cols} off{offset}"
    Yr, A = oracle.gemv_q8act(fmt, W, rows, cols, x[None])
    assert_agree(y[None], Yr, A, what)
    if np.isfinite(x).all():
        check_exact_bound(fmt, W, rows, cols, x, y, what)
    return W, x, y


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,cols", [(37, 256), (300, 2304), (5, 4096)])
def test_small_shapes(fmt, rows, cols):
    _check(fmt, rows, cols, 700 + fmt + cols)


@pytest.mark.parametrize("fmt", FMTS)
def test_weights_two_bytes_past_alignment(fmt):
    _check(fmt, 41, 768, 800 + fmt, offset=2)


@pytest.mark.parametrize("fmt", FMTS)
def test_quantisation_error_within_bound(fmt):
    # larger rows; the ratio of the departure to its bound is reported
    rows, cols = 64, 2048
    g = synth.rng(900 + fmt)
    W = synth.matrix(g, fmt, rows, cols)
    x = synth.activations(g, 1, cols)[0]
    y = run_q8(fmt, W, rows, cols, x)
    ratio = check_exact_bound(fmt, W, rows, cols, x, y, f"bound fmt {fmt}")
    print(f"\nfmt {fmt}: largest departure / bound = {ratio:.3f}")


@pytest.mark.parametrize("fmt", FMTS)
def test_representable_activations_give_the_exact_result(fmt):
    # activations that quantise exactly (k * 2^-9, |k| <= 127, 127 in every
    # group): the variant agrees with the exact GEMV's oracle
    rows, cols = 29, 1024
    g = synth.rng(1000 + fmt)
    W = synth.matrix(g, fmt, rows, cols)
    k = g.integers(-127, 128, size=cols)
    k[::16] = 127
    x = (k * 2.0 ** -9).astype(np.float32)
    y = run_q8(fmt, W, rows, cols, x)
    Ye, Ae = oracle.gemv(fmt, W, rows, cols, x[None])
    assert_agree(y[None], Ye, Ae, f"representable fmt {fmt}")
    Yr, A = oracle.gemv_q8act(fmt, W, rows, cols, x[None])
    assert_agree(y[None], Yr, A, f"representable fmt {fmt}, int8 oracle")


def test_zero_and_non_finite_groups():
    fmt, rows, cols = q.QG_Q4_K, 8, 512
    g = synth.rng(1100)
    W = synth.matrix(g, fmt, rows, cols)
    x = synth.activations(g, 1, cols)[0]
    x[:16] = 0.0
    _check(fmt, rows, cols, 1100, x=x)
    x[100] = np.inf
    y = run_q8(fmt, W, rows, cols, x)
    assert np.isnan(y).all()


@pytest.mark.parametrize("name", ["q4_k_4096x4096", "q6_k_151936x2048"])
def test_workload_full_size(name):
    case = synth.GEMV_CASES[name]
    W, X = synth.gemv_inputs(case, 1)
    y = run_q8(case.fmt, W, case.rows, case.cols, X[0])
    g = synth.rng(case.seed + 77)
    idx = np.sort(g.choice(case.rows, size=min(case.rows, 1500), replace=False))
    sub = W.reshape(case.rows, -1)[idx]
    Yr, A = oracle.gemv_q8act(case.fmt, sub, len(idx), case.cols, X)
    assert_agree(y[None, idx], Yr, A, f"{name} q8act (sampled rows)")
    check_exact_bound(case.fmt, W, case.rows, case.cols, X[0], y[idx], f"{name} exact bound",
                      row_idx=idx)
    assert np.isfinite(y).all()


def test_refusals():
    x = torch.zeros(256, device=dev())
    y = torch.zeros(4, device=dev())
    W = torch.zeros(4 * 144, dtype=torch.uint8, device=dev())
    with pytest.raises(q.QGError):
        q.qgemv_q8act(q.QG_F32, W, 4, 64, x, y)
    with pytest.raises(q.QGError):
        q.qgemv_q8act(q.QG_Q4_K, W, 4, 255, x, y)
