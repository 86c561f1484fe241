"""GPU parity of qgemv_q8act (int8-quantised activations, integer dot
products) against the oracle's int8-activation GEMV, which quantises the
activations the same way and accumulates in f64.

Tolerance per row: 1e-4 * sum |w * x_q| + 1e-6 (the quantised activations
are identical on both sides; only the order and width of the sums differ).
The departure from the exact GEMV is checked against the quantisation bound
sum |w| * d / 2 and reported.
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


def _check(fmt, rows, cols, seed, offset=0, x=None):
    g = synth.rng(seed)
    W = synth.matrix(g, fmt, rows, cols)
    if x is None:
        x = synth.activations(g, 1, cols)[0]
    y = run_q8(fmt, W, rows, cols, x, offset)
    Yr, A = oracle.gemv_q8act(fmt, W, rows, cols, x[None])
    assert_agree(y[None], Yr, A, f"q8act fmt {fmt} {rows}x{cols} off{offset}")
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
    # the result departs from the exact GEMV by at most sum |w| * d / 2
    rows, cols = 64, 2048
    W, x, y = _check(fmt, rows, cols, 900 + fmt)
    _, d = oracle.quantize_q8(x)
    Wd = oracle.dequant_matrix(fmt, W, rows, cols)
    bound = np.abs(Wd) @ np.repeat(d.astype(np.float64), 16) / 2
    Ye, Ae = oracle.gemv(fmt, W, rows, cols, x[None])
    assert np.all(np.abs(y - Ye[0]) <= bound * (1 + 1e-3) + 1e-4 * Ae[0] + 1e-6)


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
    assert np.isfinite(y).all()


def test_refusals():
    x = torch.zeros(256, device=dev())
    y = torch.zeros(4, device=dev())
    W = torch.zeros(4 * 144, dtype=torch.uint8, device=dev())
    with pytest.raises(q.QGError):
        q.qgemv_q8act(q.QG_F32, W, 4, 64, x, y)
    with pytest.raises(q.QGError):
        q.qgemv_q8act(q.QG_Q4_K, W, 4, 255, x, y)
