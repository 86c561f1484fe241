"""Pins of the oracle's MoE FFN and of the comparison rule (P7 and checker tests).

The MoE oracle is composed of pieces pinned in test_oracle_pins.py (the
GEMV, the routing, SiLU).  Here the composition is pinned by reductions to
simpler computations done with numpy/scipy library routines on the oracle's
dequantised weights, and by invariants.  The last tests plant mistakes on the
CPU and check that the comparison rule rejects them.
"""
from __future__ import annotations

import numpy as np
import pytest
from scipy.special import expit

import oracle
import synth
from oracle import F32, Q4_0, Q8_0, Q4_K, Q5_K, Q6_K
from parity import agree_mask, assert_agree


def _small_moe(seed, E=6, k=2, H=256, F=256, gate_fmt=Q4_K, down_fmt=Q6_K):
    g = synth.rng(seed)
    router = synth.f32_matrix(g, E, H, 0.02)
    gate = synth.matrix(g, gate_fmt, E * F, H)
    up = synth.matrix(g, gate_fmt, E * F, H)
    down = synth.matrix(g, down_fmt, E * H, F)
    x = synth.activations(g, 1, H)[0]
    res = synth.activations(g, 1, H)[0]
    return dict(router=router, gate=gate, up=up, down=down, x=x, res=res,
                E=E, k=k, H=H, F=F, gate_fmt=gate_fmt, down_fmt=down_fmt)


def _run(m, x=None, res=None, router=None, gate=None, up=None, down=None):
    return oracle.moe_ffn(
        m["x"] if x is None else x, m["res"] if res is None else res,
        m["router"] if router is None else router,
        m["gate_fmt"], m["gate"] if gate is None else gate,
        m["gate_fmt"], m["up"] if up is None else up,
        m["down_fmt"], m["down"] if down is None else down,
        m["H"], m["E"], m["k"], m["F"])


def _numpy_moe(m, sel, w):
    """Same computation with library routines (numpy f64 matmul, scipy
    expit) on the oracle's dequantised weights."""
    H, F = m["H"], m["F"]
    x = m["x"].astype(np.float64)
    y = m["res"].astype(np.float64).copy()
    for s, e in enumerate(sel):
        G = oracle.dequant_matrix(m["gate_fmt"], m["gate"][e * F:(e + 1) * F], F, H)
        U = oracle.dequant_matrix(m["gate_fmt"], m["up"][e * F:(e + 1) * F], F, H)
        D = oracle.dequant_matrix(m["down_fmt"], m["down"][e * H:(e + 1) * H], H, F)
        gg, uu = G @ x, U @ x
        y += w[s] * (D @ (gg * expit(gg) * uu))
    return y


def test_router_logits_are_the_f32_gemv():
    m = _small_moe(1)
    out = _run(m)
    want = m["router"].astype(np.float64) @ m["x"].astype(np.float64)
    assert np.allclose(out["logits"], want, rtol=0, atol=1e-14)
    sel, w = oracle.route(want, m["k"])
    assert np.array_equal(out["sel"], sel)


def test_single_expert_reduces_to_the_dense_swiglu_ffn():
    """E = 1, k = 1: y = residual + D (silu(G x) * (U x)), the dense FFN."""
    m = _small_moe(2, E=1, k=1)
    out = _run(m)
    assert list(out["sel"]) == [0] and out["w"][0] == 1.0
    want = _numpy_moe(m, [0], [1.0])
    assert_agree(out["y"], want, out["bound"], "dense FFN", rel=1e-12, abs_=0)


@pytest.mark.parametrize("gate_fmt,down_fmt", [(Q4_K, Q6_K), (Q8_0, Q4_0), (Q5_K, Q4_K)])
def test_moe_matches_library_composition(gate_fmt, down_fmt):
    m = _small_moe(3, E=5, k=3, gate_fmt=gate_fmt, down_fmt=down_fmt)
    out = _run(m)
    want = _numpy_moe(m, out["sel"], out["w"])
    assert_agree(out["y"], want, out["bound"], "moe", rel=1e-12, abs_=0)


def test_output_minus_residual_does_not_depend_on_residual():
    m = _small_moe(4)
    a = _run(m)
    b = _run(m, res=m["res"] * 3 + 1)
    assert np.array_equal(a["sel"], b["sel"])
    assert np.all(np.abs((a["y"] - m["res"]) - (b["y"] - (m["res"] * 3 + 1)))
                  <= 1e-12 * (a["bound"] + b["bound"]))


def test_relabelling_experts_is_equivariant():
    m = _small_moe(5, E=7, k=3)
    E, F, H = m["E"], m["F"], m["H"]
    perm = np.random.default_rng(5).permutation(E)   # expert e moves to perm[e]
    inv = np.argsort(perm)
    router = m["router"][inv]
    gate = m["gate"].reshape(E, F, -1)[inv].reshape(E * F, -1)
    up = m["up"].reshape(E, F, -1)[inv].reshape(E * F, -1)
    down = m["down"].reshape(E, H, -1)[inv].reshape(E * H, -1)
    a = _run(m)
    b = _run(m, router=router, gate=gate, up=up, down=down)
    assert np.array_equal(b["sel"], perm[a["sel"]])
    assert np.array_equal(a["w"], b["w"])
    assert np.array_equal(a["y"], b["y"])


def test_folding_the_route_weight_equals_scaling_the_down_output():
    m = _small_moe(6)
    out = _run(m)
    H, F = m["H"], m["F"]
    y = m["res"].astype(np.float64).copy()
    for s, e in enumerate(out["sel"]):
        D = oracle.dequant_matrix(m["down_fmt"], m["down"][e * H:(e + 1) * H], H, F)
        unweighted = out["act"][s] / out["w"][s]
        y += out["w"][s] * (D @ unweighted)
    assert_agree(out["y"], y, out["bound"], "fold", rel=1e-12, abs_=0)


def test_act_is_weighted_swiglu_of_the_expert_gemvs():
    m = _small_moe(7)
    out = _run(m)
    H, F = m["H"], m["F"]
    for s, e in enumerate(out["sel"]):
        gg, _ = oracle.gemv(m["gate_fmt"], m["gate"][e * F:(e + 1) * F], F, H, m["x"][None])
        uu, _ = oracle.gemv(m["gate_fmt"], m["up"][e * F:(e + 1) * F], F, H, m["x"][None])
        want = out["w"][s] * gg[0] * expit(gg[0]) * uu[0]
        assert np.allclose(out["act"][s], want, rtol=1e-13, atol=1e-300)


def test_moe_argument_errors():
    m = _small_moe(8)
    with pytest.raises(ValueError):
        oracle.moe_ffn(m["x"], m["res"], m["router"], Q4_K, m["gate"], Q4_K, m["up"],
                       Q6_K, m["down"], m["H"], m["E"], m["E"] + 1, m["F"])
    with pytest.raises(ValueError):
        oracle.moe_ffn(m["x"], m["res"], m["router"], Q4_K, m["gate"], Q4_K, m["up"],
                       Q6_K, m["down"], 100, m["E"], 2, m["F"])


# ------------------------------------------ the checker rejects mistakes

def test_checker_rejects_a_flipped_weight_byte():
    W = synth.matrix(synth.rng(80), Q4_K, 8, 512)
    x = synth.activations(synth.rng(81), 1, 512)
    Y, A = oracle.gemv(Q4_K, W, 8, 512, x)
    W2 = W.copy()
    W2[3, 100] ^= 0x10                      # one quant nibble of row 3
    Y2, _ = oracle.gemv(Q4_K, W2, 8, 512, x)
    ok = agree_mask(Y2[0], Y[0], A[0])
    assert not ok[3] and ok[np.arange(8) != 3].all()


def test_checker_rejects_a_swapped_expert_and_a_perturbed_route_weight():
    m = _small_moe(82, E=6, k=2)
    out = _run(m)
    H, F = m["H"], m["F"]
    sel, w = out["sel"], out["w"]
    # the right experts in the wrong slots: weights attached to the wrong one
    wrong = _numpy_moe(m, sel[::-1], w)
    assert not agree_mask(wrong, out["y"], out["bound"]).all()
    # an expert that was not chosen
    other = [e for e in range(m["E"]) if e not in sel][0]
    wrong = _numpy_moe(m, [sel[0], other], w)
    assert not agree_mask(wrong, out["y"], out["bound"]).all()
    # one route weight off by 1%
    wrong = _numpy_moe(m, sel, w * np.array([1.01, 1.0]))
    assert not agree_mask(wrong, out["y"], out["bound"]).all()


def test_checker_nan_and_inf_rules():
    y = np.array([np.nan, np.inf, -np.inf, 1.0])
    assert agree_mask(y, y, np.ones(4)).all()
    assert not agree_mask(np.array([np.nan]), np.array([1.0]), np.ones(1)).any()
    assert not agree_mask(np.array([np.inf]), np.array([-np.inf]), np.ones(1)).any()
    assert not agree_mask(np.array([1.0]), np.array([np.nan]), np.ones(1)).any()
