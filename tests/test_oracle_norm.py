"""Pins of the oracle's fused residual add + RMSNorm and of the MoE FFN
behind it, against closed forms and invariants (no GPU).

Definition (web page: docs.rs, crate ferrox-cuda 0.14.0, src/gpu.rs,
FUSED_ADD_RMSNORM_KERNEL_SRC): out = (x + r) / sqrt(mean((x + r)^2) + eps)
* weight.  The aprender-serve page's moe_layer applies it (ffn_norm) before
the router and the experts and adds the expert outputs back into hidden.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import synth

f32 = np.float32


def ulp_close(a, b, ulps=1):
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    return bool(np.all(np.abs(a.astype(np.float64) - b.astype(np.float64))
                       <= ulps * np.spacing(np.abs(b)).astype(np.float64)))


@pytest.mark.parametrize("c", [4.0, -0.125, 1.0, -64.0])
def test_constant_vector_normalises_to_the_sign(c):
    # h = c everywhere: mean(h^2) = c^2, so with eps = 0 every h / |c| is +-1
    # exactly and the output is sign(c) * weight, bit for bit (c a power of 2)
    n = 96
    g = synth.rng(5)
    w = g.standard_normal(n).astype(f32)
    x = np.full(n, c / 2, dtype=f32)
    r = np.full(n, c / 2, dtype=f32)
    h, xn = oracle.add_rmsnorm(x, r, w, 0.0)
    assert np.array_equal(h, np.full(n, c, dtype=f32))
    assert np.array_equal(xn, (np.sign(c) * w).astype(f32))


def test_three_four_closed_form():
    # h = (3, 4): mean square 12.5, so xn = (3, 4) / sqrt(12.5) = (3, 4) * sqrt(2) / 5.
    # A sum in place of the mean would give (3, 4) / 5.
    h, xn = oracle.add_rmsnorm(np.array([1, 4], f32), np.array([2, 0], f32),
                               np.ones(2, f32), 0.0)
    assert np.array_equal(h, np.array([3, 4], f32))
    want = [f32(3 * math.sqrt(2) / 5), f32(4 * math.sqrt(2) / 5)]
    assert ulp_close(xn, want)


def test_eps_sits_inside_the_root():
    # h = c everywhere and eps = c^2: xn = c / sqrt(2 c^2) * w = w / sqrt(2) for c > 0;
    # eps added after the root would give c / (|c| + c^2) * w instead
    n = 64
    c = 0.5
    w = np.linspace(-2, 2, n).astype(f32)
    _, xn = oracle.add_rmsnorm(np.full(n, c, f32), np.zeros(n, f32), w, c * c)
    assert ulp_close(xn, (w.astype(np.float64) / math.sqrt(2)).astype(f32))


def test_zero_input_with_eps_is_zero():
    n = 32
    _, xn = oracle.add_rmsnorm(np.zeros(n, f32), np.zeros(n, f32), np.ones(n, f32), 1e-6)
    assert np.array_equal(xn, np.zeros(n, f32))


def test_power_of_two_scale_invariance_is_exact():
    # with eps = 0, scaling h by 2^k scales sum h^2 by 4^k: the root and the
    # quotient scale exactly, so the output is unchanged bit for bit
    n = 2048
    g = synth.rng(11)
    x = g.standard_normal(n).astype(f32)
    r = g.standard_normal(n).astype(f32)
    w = (1 + 0.1 * g.standard_normal(n)).astype(f32)
    _, xn = oracle.add_rmsnorm(x, r, w, 0.0)
    for k in (-3, 1, 5):
        s = f32(2.0 ** k)
        _, xs = oracle.add_rmsnorm(x * s, r * s, w, 0.0)
        assert np.array_equal(xs, xn)


def test_unit_weight_output_has_unit_mean_square():
    n = 2048
    g = synth.rng(12)
    x = g.standard_normal(n).astype(f32)
    r = (3 * g.standard_normal(n)).astype(f32)
    _, xn = oracle.add_rmsnorm(x, r, np.ones(n, f32), 0.0)
    assert abs(np.mean(xn.astype(np.float64) ** 2) - 1.0) < 1e-6


def test_the_add_is_an_f32_addition():
    # 1 + 2^-24 rounds to 1 in f32 (ties to even); 1 + 3*2^-24 rounds up
    x = np.array([1.0, 1.0], f32)
    r = np.array([2.0 ** -24, 3 * 2.0 ** -24], f32)
    h, _ = oracle.add_rmsnorm(x, r, np.ones(2, f32), 0.0)
    assert h[0] == f32(1.0) and h[1] == f32(1.0 + 2.0 ** -22)


def test_matches_a_numpy_composition():
    n = 768
    g = synth.rng(13)
    x = g.standard_normal(n).astype(f32)
    r = g.standard_normal(n).astype(f32)
    w = (1 + 0.2 * g.standard_normal(n)).astype(f32)
    eps = float(f32(1e-6))
    h, xn = oracle.add_rmsnorm(x, r, w, eps)
    hh = (x + r).astype(np.float64)
    want = (hh / np.sqrt(np.mean(hh * hh) + eps) * w).astype(f32)
    assert np.array_equal(h, (x + r))
    assert ulp_close(xn, want)


def _small_moe(seed, E=8, k=2, H=256, F=256):
    g = synth.rng(seed)
    router = synth.f32_matrix(g, E, H, 0.02)
    gate = synth.matrix(g, synth.Q4_K, E * F, H)
    up = synth.matrix(g, synth.Q4_K, E * F, H)
    down = synth.matrix(g, synth.Q6_K, E * H, F)
    return g, router, gate, up, down, (H, E, k, F)


def test_moe_norm_reduces_to_moe_on_a_unit_rms_stream():
    # attn_out = 0, hidden = +-1 (mean square exactly 1), weight = 1, eps = 0:
    # xn = h exactly, so the normed FFN is moe_ffn(x = h, residual = h)
    g, router, gate, up, down, (H, E, k, F) = _small_moe(21)
    hid = np.where(g.standard_normal(H) < 0, -1.0, 1.0).astype(f32)
    r = oracle.moe_ffn_norm(np.zeros(H, f32), hid, np.ones(H, f32), 0.0, router, synth.Q4_K,
                            gate, synth.Q4_K, up, synth.Q6_K, down, H, E, k, F)
    m = oracle.moe_ffn(hid, hid, router, synth.Q4_K, gate, synth.Q4_K, up, synth.Q6_K, down,
                       H, E, k, F)
    assert np.array_equal(r["xn"], hid) and np.array_equal(r["h"], hid)
    for key in ("y", "logits", "sel", "w", "act", "bound"):
        assert np.array_equal(r[key], m[key]), key


def test_moe_norm_output_minus_stream_is_scale_free():
    # with eps = 0, scaling attn_out and hidden by 2 leaves xn, the routing and
    # the expert sum unchanged; only the residual stream doubles
    g, router, gate, up, down, (H, E, k, F) = _small_moe(22)
    a = g.standard_normal(H).astype(f32)
    b = g.standard_normal(H).astype(f32)
    w = (1 + 0.1 * g.standard_normal(H)).astype(f32)
    args = (router, synth.Q4_K, gate, synth.Q4_K, up, synth.Q6_K, down, H, E, k, F)
    r1 = oracle.moe_ffn_norm(a, b, w, 0.0, *args)
    r2 = oracle.moe_ffn_norm(2 * a, 2 * b, w, 0.0, *args)
    assert np.array_equal(r1["xn"], r2["xn"]) and np.array_equal(r1["sel"], r2["sel"])
    d1 = r1["y"] - r1["h"].astype(np.float64)
    d2 = r2["y"] - r2["h"].astype(np.float64)
    assert np.allclose(d1, d2, rtol=0, atol=1e-12 * (1 + r1["bound"].max()))


def test_moe_norm_stream_is_the_f32_sum():
    g, router, gate, up, down, (H, E, k, F) = _small_moe(23)
    a = g.standard_normal(H).astype(f32)
    b = g.standard_normal(H).astype(f32)
    r = oracle.moe_ffn_norm(a, b, np.ones(H, f32), float(f32(1e-6)), router, synth.Q4_K, gate,
                            synth.Q4_K, up, synth.Q6_K, down, H, E, k, F)
    assert np.array_equal(r["h"], a + b)
    # the expert part is the plain MoE on xn with residual h
    m = oracle.moe_ffn(r["xn"], r["h"], router, synth.Q4_K, gate, synth.Q4_K, up, synth.Q6_K,
                       down, H, E, k, F)
    assert np.array_equal(m["y"], r["y"]) and np.array_equal(m["sel"], r["sel"])
