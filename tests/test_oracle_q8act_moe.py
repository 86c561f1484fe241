"""Pins of the oracle's int8-activation MoE FFN and of its bound (no GPU).

The variant quantises x, and each slot's f32 SwiGLU activations, per group
of 16 columns (weight_matrix.rs page, cpu_int_dot_enabled: int8
activations; gpu.rs page, module notes: integer dot products, one float
conversion per block).  oracle.moe_ffn_q8act computes that chain;
oracle.moe_q8act_bound bounds, per output row, how far it may land from
the exact chain (oracle.moe_ffn).  Pinned here:

* the chain against the exact chain through that bound (the bound is
  derived from |q d - v| <= d / 2 and |silu'| <= 1.1, not from the
  variant's code);
* the chain against its own steps done by the already pinned int8 GEMV
  oracle (oracle.gemv_q8act), slot by slot;
* x = 0: nothing is quantised away, y = residual exactly.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth

f32 = np.float32


def _by_steps(x, res, router, gfmt, gate, up, dfmt, down, H, E, K, F):
    """The chain slot by slot through oracle.gemv_q8act: exact routes, the
    gate and up rows of each chosen expert on the quantised x, the f32
    activations w silu(g) u, the down rows on their quantisation."""
    logits = router.astype(np.float64) @ x.astype(np.float64)
    sel, w = oracle.route(logits, K)
    rbg, rbd = oracle.row_bytes(gfmt, H), oracle.row_bytes(dfmt, F)
    y = res.astype(np.float64).copy()
    for s in range(K):
        e = int(sel[s])
        g = oracle.gemv_q8act(gfmt, gate[e * F * rbg:(e + 1) * F * rbg], F, H, x)[0][0]
        u = oracle.gemv_q8act(gfmt, up[e * F * rbg:(e + 1) * F * rbg], F, H, x)[0][0]
        a = (w[s] * oracle_silu(g) * u).astype(f32)
        y += oracle.gemv_q8act(dfmt, down[e * H * rbd:(e + 1) * H * rbd], H, F, a)[0][0]
    return y


def oracle_silu(g):
    return np.array([oracle.silu(float(v)) for v in g])


def _case(seed, gfmt, dfmt, E=6, K=2, H=256, F=256, xscale=1.0):
    g = synth.rng(seed)
    router = synth.f32_matrix(g, E, H, 0.02)
    gate = synth.matrix(g, gfmt, E * F, H).view(np.uint8).reshape(-1)
    up = synth.matrix(g, gfmt, E * F, H).view(np.uint8).reshape(-1)
    down = synth.matrix(g, dfmt, E * H, F).view(np.uint8).reshape(-1)
    x = (synth.activations(g, 1, H)[0] * xscale).astype(f32)
    res = synth.activations(g, 1, H)[0]
    return router, gate, up, down, x, res


@pytest.mark.parametrize("gfmt,dfmt", [(oracle.Q4_K, oracle.Q6_K), (oracle.Q8_0, oracle.Q4_0),
                                       (oracle.Q5_K, oracle.Q8_0), (oracle.Q4_0, oracle.Q5_K)])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_chain_within_the_bound_of_the_exact_chain(gfmt, dfmt, seed):
    E, K, H, F = 6, 2, 256, 256
    router, gate, up, down, x, res = _case(100 * seed + gfmt, gfmt, dfmt)
    ex = oracle.moe_ffn(x, res, router, gfmt, gate, gfmt, up, dfmt, down, H, E, K, F)
    qb = oracle.moe_q8act_bound(x, res, router, gfmt, gate, gfmt, up, dfmt, down, H, E, K, F)
    v = oracle.moe_ffn_q8act(x, res, router, gfmt, gate, gfmt, up, dfmt, down, H, E, K, F)
    assert np.array_equal(v["sel"], ex["sel"]) and np.array_equal(v["w"], ex["w"])
    dep = np.abs(v["y"] - ex["y"])
    assert np.all(np.isfinite(qb)) and np.all(qb >= 0)
    assert np.all(dep <= qb), float(np.max(dep - qb))
    # not vacuous: the departure is a visible part of the bound somewhere
    # (worst-case sums over gate/up and then down make it loose by about
    # two orders of magnitude)
    assert np.max(dep / qb) > 1e-3, float(np.max(dep / qb))


@pytest.mark.parametrize("gfmt,dfmt", [(oracle.Q4_K, oracle.Q6_K), (oracle.Q4_0, oracle.Q5_K)])
def test_chain_equals_its_steps_through_the_int8_gemv(gfmt, dfmt):
    E, K, H, F = 5, 3, 256, 256
    router, gate, up, down, x, res = _case(40 + gfmt, gfmt, dfmt, E=E)
    v = oracle.moe_ffn_q8act(x, res, router, gfmt, gate, gfmt, up, dfmt, down, H, E, K, F)
    y = _by_steps(x, res, router, gfmt, gate, up, dfmt, down, H, E, K, F)
    # same f64 products; only the order of the sums differs
    assert np.all(np.abs(v["y"] - y) <= 1e-12 * v["bound"])


def test_tie_allowance_counts_only_codes_near_a_tie():
    E, K, H, F = 6, 2, 256, 256
    router, gate, up, down, x, res = _case(55, oracle.Q4_K, oracle.Q6_K)
    t0 = oracle.moe_ffn_q8act(x, res, router, oracle.Q4_K, gate, oracle.Q4_K, up, oracle.Q6_K,
                              down, H, E, K, F, tie_window=0.0)["tie"]
    t1 = oracle.moe_ffn_q8act(x, res, router, oracle.Q4_K, gate, oracle.Q4_K, up, oracle.Q6_K,
                              down, H, E, K, F, tie_window=0.5)["tie"]
    qb = oracle.moe_q8act_bound(x, res, router, oracle.Q4_K, gate, oracle.Q4_K, up,
                                oracle.Q6_K, down, H, E, K, F)
    assert np.array_equal(t0, np.zeros(H))
    # window 1/2 takes every code: sum_j |D_rj| d, below the bound's
    # d / 2 share doubled (the bound's steps are at least the variant's)
    assert np.all(t1 > 0) and np.all(t1 <= 2 * qb)


def test_bound_is_zero_when_nothing_is_quantised_away():
    # x = 0 everywhere: every SwiGLU activation is silu(0) * 0 = 0, so the
    # variant quantises nothing away and y = residual exactly
    E, K, H, F = 5, 2, 256, 256
    router, gate, up, down, x, res = _case(7, oracle.Q4_K, oracle.Q6_K, E=E)
    x[:] = 0
    qb = oracle.moe_q8act_bound(x, res, router, oracle.Q4_K, gate, oracle.Q4_K, up,
                                oracle.Q6_K, down, H, E, K, F)
    assert np.array_equal(qb, np.zeros(H))
    v = oracle.moe_ffn_q8act(x, res, router, oracle.Q4_K, gate, oracle.Q4_K, up, oracle.Q6_K,
                             down, H, E, K, F, tie_window=0.5)
    assert np.array_equal(v["y"], res.astype(np.float64))
    assert np.array_equal(v["tie"], np.zeros(H))


def test_bound_grows_linearly_with_the_input_scale_of_the_quantisation_steps():
    # scaling the router-free parts: with x scaled by 2^m the gate/up steps
    # scale by 2^m; the bound of a row must grow, never shrink
    E, K, H, F = 6, 2, 256, 256
    b = []
    for m in (0, 1):
        router, gate, up, down, x, res = _case(11, oracle.Q8_0, oracle.Q4_K, xscale=2.0 ** m)
        b.append(oracle.moe_q8act_bound(x, res, router, oracle.Q8_0, gate, oracle.Q8_0, up,
                                        oracle.Q4_K, down, H, E, K, F))
    assert np.all(b[1] > b[0])


def test_non_finite_x_gives_nan_bounds():
    E, K, H, F = 4, 1, 256, 256
    router, gate, up, down, x, res = _case(13, oracle.Q4_K, oracle.Q6_K, E=E)
    x[3] = np.inf
    qb = oracle.moe_q8act_bound(x, res, router, oracle.Q4_K, gate, oracle.Q4_K, up,
                                oracle.Q6_K, down, H, E, K, F)
    assert np.isnan(qb).all()
