"""Pins of the oracle's int8-activation variant (quantiser and GEMV) against
closed forms and against the exact GEMV oracle (no GPU).

The pages name the variant only in words (gpu.rs page, module notes: the
integer dp4a dot product of llama.cpp's K-quant kernels; weight_matrix.rs
page, cpu_int_dot_enabled: quantise the activation to int8, integer
vec_dot).  Reading: 16-column groups, d = max|x| / 127, id = 1 / d,
q = rint(x * id), all f32.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth

f32 = np.float32


def test_representable_groups_round_trip_exactly():
    # x = k * 2^-7 with max |k| = 127: d = 2^-7 exactly and q = k
    g = synth.rng(3)
    k = g.integers(-127, 128, size=64).astype(np.int64)
    k[::16] = 127 * np.where(g.random(4) < 0.5, -1, 1)
    x = (k * 2.0 ** -7).astype(f32)
    q, d = oracle.quantize_q8(x)
    assert np.array_equal(q.astype(np.int64), k)
    assert np.array_equal(d, np.full(4, 2.0 ** -7, f32))


def test_rounding_is_half_to_even():
    # amax = 127 gives d = 1 and id = 1: x * id is x itself
    x = np.zeros(16, f32)
    x[:6] = [2.5, 3.5, -2.5, -3.5, 0.5, 127.0]
    q, d = oracle.quantize_q8(x)
    assert d[0] == f32(1.0)
    assert list(q[:6]) == [2, 4, -2, -4, 0, 127]


def test_zero_group_and_non_finite_group():
    x = np.zeros(48, f32)
    x[16:32] = np.linspace(-1, 1, 16)
    x[40] = np.inf
    q, d = oracle.quantize_q8(x)
    assert d[0] == 0 and not q[:16].any()
    assert d[1] == f32(1.0 / 127.0) or abs(d[1] - 1 / 127) < 1e-9
    assert np.isnan(d[2]) and not q[32:].any()


def test_error_bound_and_range():
    g = synth.rng(4)
    x = (g.standard_normal(4096) * np.exp(g.standard_normal(4096))).astype(f32)
    q, d = oracle.quantize_q8(x)
    dd = np.repeat(d.astype(np.float64), 16)
    err = np.abs(x.astype(np.float64) - q * dd)
    assert np.all(err <= dd / 2 * (1 + 2 ** -20))
    assert np.abs(q.astype(np.int32)).max() <= 127
    # the largest element of every group maps to +-127
    grp = np.abs(x).reshape(-1, 16).argmax(1)
    assert np.all(np.abs(q.reshape(-1, 16)[np.arange(256), grp]) == 127)


@pytest.mark.parametrize("fmt", [synth.Q8_0, synth.Q4_0, synth.Q4_K, synth.Q5_K, synth.Q6_K])
def test_q8_gemv_equals_exact_gemv_on_representable_activations(fmt):
    # activations that quantise exactly: the variant's result is the exact
    # GEMV's, bit for bit (same products, same order)
    rows, cols = 7, 512
    g = synth.rng(40 + fmt)
    W = synth.matrix(g, fmt, rows, cols)
    k = g.integers(-127, 128, size=(2, cols))
    k[:, ::16] = 127
    X = (k * 2.0 ** -9).astype(f32)
    Y, A = oracle.gemv_q8act(fmt, W, rows, cols, X)
    Ye, Ae = oracle.gemv(fmt, W, rows, cols, X)
    assert np.array_equal(Y, Ye) and np.array_equal(A, Ae)


@pytest.mark.parametrize("fmt", [synth.Q4_K, synth.Q6_K])
def test_q8_gemv_is_the_gemv_of_the_dequantised_activations(fmt):
    rows, cols = 5, 768
    g = synth.rng(50 + fmt)
    W = synth.matrix(g, fmt, rows, cols)
    X = synth.activations(g, 1, cols)
    q, d = oracle.quantize_q8(X[0])
    xq = q.astype(np.float64) * np.repeat(d.astype(np.float64), 16)
    Wd = oracle.dequant_matrix(fmt, W, rows, cols)
    Y, A = oracle.gemv_q8act(fmt, W, rows, cols, X)
    want = Wd @ xq
    assert np.allclose(Y[0], want, rtol=0, atol=1e-12 * (1 + np.abs(Wd) @ np.abs(xq)).max())
    # and it departs from the exact GEMV by at most the quantisation error
    Ye, _ = oracle.gemv(fmt, W, rows, cols, X)
    bound = np.abs(Wd) @ np.repeat(d.astype(np.float64), 16) / 2
    assert np.all(np.abs(Y[0] - Ye[0]) <= bound * (1 + 1e-6))
