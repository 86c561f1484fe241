"""GPU parity of moe_ffn_q8act, the MoE FFN with its expert GEMVs on int8
activations, and the measurement of what it does to the next layer's routes.

Every check compares with the oracle on the same inputs:

* routes: bit for bit with the exact chain (the router reads x itself);
* y against the oracle's int8 chain (oracle.moe_ffn_q8act): per row
  1e-4 * (|residual| + sum |D aq|) + 1e-6, plus one code step for every slot
  activation whose scaled value lies within 5e-3 of a rounding tie (the
  kernel's f32 activations are another rounding of the same values, so such
  a code may differ by one);
* y against the exact chain (oracle.moe_ffn) through the quantisation bound
  oracle.moe_q8act_bound, which does not depend on how the quantiser is
  written.
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

TIE_WINDOW = 5e-3


class Moe:
    def __init__(self, E, k, H, F, gate_fmt, down_fmt, seed=None, weights=None):
        self.E, self.k, self.H, self.F = E, k, H, F
        self.gate_fmt, self.down_fmt = gate_fmt, down_fmt
        if weights is None:
            g = synth.rng(seed)
            weights = (synth.f32_matrix(g, E, H, 0.02), synth.matrix(g, gate_fmt, E * F, H),
                       synth.matrix(g, gate_fmt, E * F, H), synth.matrix(g, down_fmt, E * H, F))
        self.router, self.gate, self.up, self.down = weights
        self.d_router = torch.from_numpy(self.router).to(dev())
        self.d_gate, self.d_up = DeviceBytes(self.gate), DeviceBytes(self.up)
        self.d_down = DeviceBytes(self.down)
        self.ws_bytes = q.moe_ffn_workspace_bytes(E, k, F)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev())

    def args(self):
        return (self.d_router, self.gate_fmt, self.d_gate.ptr, self.gate_fmt, self.d_up.ptr,
                self.down_fmt, self.d_down.ptr, self.H, self.E, self.k, self.F)

    def gpu(self, x, res, q8=True, alias=False):
        xd = torch.from_numpy(x).to(dev())
        rd = torch.from_numpy(res).to(dev())
        y = rd if alias else torch.full_like(rd, float("nan"))
        sel = torch.full((self.k,), -1, dtype=torch.int32, device=dev())
        w = torch.full((self.k,), float("nan"), device=dev())
        fn = q.moe_ffn_q8act if q8 else q.moe_ffn
        fn(xd, rd, y, *self.args(), sel, w, self.ws, self.ws_bytes)
        torch.cuda.synchronize()
        return y.cpu().numpy(), sel.cpu().numpy(), w.cpu().numpy()

    def oracle_args(self):
        return (self.router, self.gate_fmt, self.gate, self.gate_fmt, self.up, self.down_fmt,
                self.down, self.H, self.E, self.k, self.F)


def _check(m, x, res, what, alias=False):
    y, sel, w = m.gpu(x, res, alias=alias)
    ex = oracle.moe_ffn(x, res, *m.oracle_args())
    v = oracle.moe_ffn_q8act(x, res, *m.oracle_args(), tie_window=TIE_WINDOW)
    assert np.array_equal(sel, ex["sel"]), (what, sel, ex["sel"])
    assert np.allclose(w, ex["w"], rtol=1e-6, atol=0), what
    # against the int8 chain
    err = np.abs(y.astype(np.float64) - v["y"])
    tol = 1e-4 * v["bound"] + 1e-6 + v["tie"]
    bad = ~(err <= tol)
    assert not bad.any(), (what, int(bad.sum()), float(np.max(err - tol)))
    # against the exact chain, through the quantisation bound
    qb = oracle.moe_q8act_bound(x, res, *m.oracle_args())
    err_ex = np.abs(y.astype(np.float64) - ex["y"])
    ok = err_ex <= qb + 1e-4 * ex["bound"] + 1e-6
    assert ok.all(), (what, int((~ok).sum()))
    return y, ex, v


@pytest.mark.parametrize("gate_fmt,down_fmt", [
    (q.QG_Q4_K, q.QG_Q6_K), (q.QG_Q5_K, q.QG_Q4_K), (q.QG_Q8_0, q.QG_Q4_0),
    (q.QG_Q4_0, q.QG_Q8_0), (q.QG_Q6_K, q.QG_Q5_K),
])
def test_small_moe_every_format(gate_fmt, down_fmt):
    m = Moe(E=6, k=2, H=512, F=256, gate_fmt=gate_fmt, down_fmt=down_fmt, seed=211 + gate_fmt)
    g = synth.rng(212)
    for t in range(3):
        _check(m, synth.activations(g, 1, 512)[0], synth.activations(g, 1, 512)[0],
               f"q8 small {gate_fmt}/{down_fmt} token {t}")


@pytest.mark.parametrize("E,k", [(1, 1), (64, 8), (257, 8)])
def test_expert_counts(E, k):
    m = Moe(E=E, k=k, H=256, F=256, gate_fmt=q.QG_Q4_K, down_fmt=q.QG_Q6_K, seed=220 + E)
    g = synth.rng(221)
    _check(m, synth.activations(g, 1, 256)[0], synth.activations(g, 1, 256)[0], f"q8 E{E} k{k}")


def test_output_may_alias_residual():
    m = Moe(E=6, k=3, H=256, F=256, gate_fmt=q.QG_Q4_K, down_fmt=q.QG_Q6_K, seed=230)
    g = synth.rng(231)
    _check(m, synth.activations(g, 1, 256)[0], synth.activations(g, 1, 256)[0], "q8 alias",
           alias=True)


def test_zero_input_gives_the_residual():
    m = Moe(E=6, k=2, H=256, F=256, gate_fmt=q.QG_Q4_K, down_fmt=q.QG_Q6_K, seed=240)
    res = synth.activations(synth.rng(241), 1, 256)[0]
    y, _, _ = m.gpu(np.zeros(256, np.float32), res)
    assert np.array_equal(y, res)


def _qwen():
    case = synth.MOE_CASE
    return case, Moe(case.n_experts, case.top_k, case.hidden, case.expert_dim, case.gate_fmt,
                     case.down_fmt, weights=synth.moe_weights(case))


def test_qwen3_moe_shape_tokens():
    case, m = _qwen()
    xs, rs = synth.moe_tokens(case)
    for t in (0, 17, 40, 63):
        _check(m, xs[t], rs[t], f"q8 qwen3 token {t}")


def test_next_layer_routes_on_all_64_tokens():
    # The aprender-serve page keeps the float kernels until the int8
    # variant's effect on routing is measured.  Within one layer the routes
    # cannot move (the router reads x itself); they move in the next layer,
    # whose router reads the normed output.  For every benchmark token: the
    # layer's output by both chains (GPU), the next layer's logits from a
    # second router (f64, CPU) on RMSNorm of each, the top-k of each.
    # Measured: how many tokens keep their expert sets, the smallest k / k+1
    # margin of the exact logits and the largest logit change.  A set may
    # only change where the margin is below twice the logit change (the
    # order within a kept set may change wherever two chosen logits lie
    # closer than that).
    case, m = _qwen()
    xs, rs = synth.moe_tokens(case)
    router2 = synth.f32_matrix(synth.rng(case.seed + 901), m.E, m.H, 0.02).astype(np.float64)
    ones = np.ones(m.H, np.float32)
    zeros = np.zeros(m.H, np.float32)
    same, reordered, margins, changes, moved = 0, 0, [], [], []
    for t in range(xs.shape[0]):
        y_ex, _, _ = m.gpu(xs[t], rs[t], q8=False)
        y_q8, _, _ = m.gpu(xs[t], rs[t], q8=True)
        l_ex = router2 @ oracle.add_rmsnorm(y_ex, zeros, ones, 1e-6)[1].astype(np.float64)
        l_q8 = router2 @ oracle.add_rmsnorm(y_q8, zeros, ones, 1e-6)[1].astype(np.float64)
        s_ex, _ = oracle.route(l_ex, m.k)
        s_q8, _ = oracle.route(l_q8, m.k)
        srt = np.sort(l_ex)[::-1]
        margin = srt[m.k - 1] - srt[m.k]
        change = float(np.max(np.abs(l_q8 - l_ex)))
        margins.append(margin)
        changes.append(change)
        if np.array_equal(np.sort(s_ex), np.sort(s_q8)):
            same += 1
            reordered += 0 if np.array_equal(s_ex, s_q8) else 1
        else:
            moved.append(t)
            assert margin <= 2 * change, (t, margin, change)
    print(f"\nnext-layer expert sets kept on {same}/{xs.shape[0]} tokens (changed: {moved}; "
          f"{reordered} kept sets ranked in another order); smallest k/k+1 margin "
          f"{min(margins):.3e}, largest logit change {max(changes):.3e}, median logit change "
          f"{float(np.median(changes)):.3e}")


def test_refusals():
    m = Moe(E=4, k=2, H=256, F=256, gate_fmt=q.QG_Q4_K, down_fmt=q.QG_Q6_K, seed=250)
    x = torch.zeros(256, device=dev())
    y = torch.zeros(256, device=dev())
    with pytest.raises(q.QGError):   # workspace too small
        q.moe_ffn_q8act(x, x, y, *m.args(), None, None, m.ws, m.ws_bytes - 16)
    with pytest.raises(q.QGError):   # y aliases x
        q.moe_ffn_q8act(x, x, x, *m.args(), None, None, m.ws, m.ws_bytes)
