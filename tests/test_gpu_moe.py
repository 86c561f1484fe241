"""GPU parity of the MoE FFN chain and of the routing step against the oracle.

Expert selection is compared bit for bit; route weights to 1e-6 relative;
the output per hidden row to 1e-4 * (|residual| + sum_s sum_j |D a|) + 1e-6
with the oracle's activations (a mismatch in selection fails outright).
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest

import oracle
import synth
from parity import assert_agree

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gguf_quant_dequant_amd as q  # noqa: E402
from gpu_util import DeviceBytes, dev  # noqa: E402


class Moe:
    def __init__(self, E, k, H, F, gate_fmt, down_fmt, seed, offset=0):
        g = synth.rng(seed)
        self.E, self.k, self.H, self.F = E, k, H, F
        self.gate_fmt, self.down_fmt = gate_fmt, down_fmt
        self.router = synth.f32_matrix(g, E, H, 0.02)
        self.gate = synth.matrix(g, gate_fmt, E * F, H)
        self.up = synth.matrix(g, gate_fmt, E * F, H)
        self.down = synth.matrix(g, down_fmt, E * H, F)
        self.d_router = torch.from_numpy(self.router).to(dev())
        self.d_gate = DeviceBytes(self.gate, offset)
        self.d_up = DeviceBytes(self.up, offset)
        self.d_down = DeviceBytes(self.down, offset)
        self.ws_bytes = q.moe_ffn_workspace_bytes(E, k, F)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev())

    def gpu(self, x, res, alias=False):
        xd = torch.from_numpy(x).to(dev())
        rd = torch.from_numpy(res).to(dev())
        y = rd if alias else torch.full_like(rd, float("nan"))
        sel = torch.full((self.k,), -1, dtype=torch.int32, device=dev())
        w = torch.full((self.k,), float("nan"), device=dev())
        q.moe_ffn(xd, rd, y, self.d_router, self.gate_fmt, self.d_gate.ptr, self.gate_fmt,
                  self.d_up.ptr, self.down_fmt, self.d_down.ptr, self.H, self.E, self.k, self.F,
                  sel, w, self.ws, self.ws_bytes)
        torch.cuda.synchronize()
        logits = self.ws[:8 * self.E].view(torch.float64).cpu().numpy()
        return y.cpu().numpy(), sel.cpu().numpy(), w.cpu().numpy(), logits

    def ref(self, x, res):
        return oracle.moe_ffn(x, res, self.router, self.gate_fmt, self.gate, self.gate_fmt,
                              self.up, self.down_fmt, self.down, self.H, self.E, self.k, self.F)


def _compare(m, x, res, what, alias=False):
    y, sel, w, logits = m.gpu(x, res, alias=alias)
    r = m.ref(x, res)
    lb = np.abs(m.router.astype(np.float64)) @ np.abs(x.astype(np.float64))
    assert np.all(np.abs(logits - r["logits"]) <= 1e-12 * lb), what
    assert np.array_equal(sel, r["sel"]), (what, sel, r["sel"])
    assert np.allclose(w, r["w"], rtol=1e-6, atol=0), what
    assert_agree(y, r["y"], r["bound"], what)
    return logits, r


@pytest.mark.parametrize("gate_fmt,down_fmt", [
    (q.QG_Q4_K, q.QG_Q6_K), (q.QG_Q5_K, q.QG_Q4_K), (q.QG_Q8_0, q.QG_Q4_0),
    (q.QG_Q4_0, q.QG_Q8_0), (q.QG_Q6_K, q.QG_Q5_K),
])
def test_small_moe_every_format(gate_fmt, down_fmt):
    m = Moe(E=6, k=2, H=512, F=256, gate_fmt=gate_fmt, down_fmt=down_fmt, seed=11 + gate_fmt)
    g = synth.rng(12)
    for t in range(3):
        _compare(m, synth.activations(g, 1, 512)[0], synth.activations(g, 1, 512)[0],
                 f"small {gate_fmt}/{down_fmt} token {t}")


@pytest.mark.parametrize("E,k", [(1, 1), (8, 8), (64, 1), (130, 5), (256, 32), (257, 8),
                                  (1024, 32)])
def test_moe_expert_counts(E, k):
    m = Moe(E=E, k=k, H=256, F=256, gate_fmt=q.QG_Q4_K, down_fmt=q.QG_Q6_K, seed=20 + E)
    g = synth.rng(21)
    _compare(m, synth.activations(g, 1, 256)[0], synth.activations(g, 1, 256)[0], f"E{E} k{k}")


@pytest.mark.parametrize("E,k", [(24, 7), (300, 9)])
def test_moe_tied_router_logits_pick_the_lower_index(E, k):
    # repeated and all-zero router rows give bit-identical logits: ties
    # across the top-k cut must go to the lower expert index
    m = Moe(E=E, k=k, H=256, F=256, gate_fmt=q.QG_Q4_K, down_fmt=q.QG_Q6_K, seed=25 + E)
    for e in range(E):
        if e % 3 == 1:
            m.router[e] = m.router[e % 5]
        elif e % 7 == 2:
            m.router[e] = 0.0
    m.d_router = torch.from_numpy(m.router).to(dev())
    g = synth.rng(26)
    _compare(m, synth.activations(g, 1, 256)[0], synth.activations(g, 1, 256)[0], f"ties E{E}")


def test_moe_output_may_alias_residual_and_unaligned_stacks():
    m = Moe(E=6, k=3, H=256, F=256, gate_fmt=q.QG_Q4_K, down_fmt=q.QG_Q6_K, seed=30, offset=2)
    g = synth.rng(31)
    _compare(m, synth.activations(g, 1, 256)[0], synth.activations(g, 1, 256)[0], "alias",
             alias=True)


def test_moe_optional_route_outputs():
    m = Moe(E=6, k=2, H=256, F=256, gate_fmt=q.QG_Q4_K, down_fmt=q.QG_Q6_K, seed=40)
    x = synth.activations(synth.rng(41), 1, 256)[0]
    xd = torch.from_numpy(x).to(dev())
    y = torch.empty_like(xd)
    q.moe_ffn(xd, xd, y, m.d_router, m.gate_fmt, m.d_gate.ptr, m.gate_fmt, m.d_up.ptr,
              m.down_fmt, m.d_down.ptr, m.H, m.E, m.k, m.F, None, None, m.ws, m.ws_bytes)
    torch.cuda.synchronize()
    r = m.ref(x, x)
    assert_agree(y.cpu().numpy(), r["y"], r["bound"], "no route outputs")


def test_qwen3_moe_shape_all_64_tokens():
    # every token the benchmark routes: selection bit for bit, weights and
    # outputs to the tolerance.  The oracle's margin between the k-th and
    # (k+1)-th logit and the largest router-logit error are printed: a
    # selection could only differ where the margin is below that error.
    case = synth.MOE_CASE
    router, gate, up, down = synth.moe_weights(case)
    m = Moe.__new__(Moe)
    m.E, m.k, m.H, m.F = case.n_experts, case.top_k, case.hidden, case.expert_dim
    m.gate_fmt, m.down_fmt = case.gate_fmt, case.down_fmt
    m.router, m.gate, m.up, m.down = router, gate, up, down
    m.d_router = torch.from_numpy(router).to(dev())
    m.d_gate, m.d_up, m.d_down = DeviceBytes(gate), DeviceBytes(up), DeviceBytes(down)
    m.ws_bytes = q.moe_ffn_workspace_bytes(m.E, m.k, m.F)
    m.ws = torch.empty(m.ws_bytes, dtype=torch.uint8, device=dev())
    xs, rs = synth.moe_tokens(case)
    assert xs.shape[0] == 64
    margins, errs = [], []
    for t in range(xs.shape[0]):
        logits, r = _compare(m, xs[t], rs[t], f"qwen3 token {t}")
        srt = np.sort(r["logits"])[::-1]
        margins.append(srt[m.k - 1] - srt[m.k])
        errs.append(np.max(np.abs(logits - r["logits"])))
    print(f"\n64 tokens: smallest k/k+1 logit margin {min(margins):.3e}, "
          f"largest router-logit error {max(errs):.3e}")
    assert max(errs) < min(margins)


def test_moe_run_to_run_bitwise_identical():
    m = Moe(E=16, k=4, H=512, F=512, gate_fmt=q.QG_Q4_K, down_fmt=q.QG_Q6_K, seed=50)
    x = synth.activations(synth.rng(51), 1, 512)[0]
    a = m.gpu(x, x)
    b = m.gpu(x, x)
    for u, v in zip(a, b):
        assert np.array_equal(np.asarray(u).view(np.uint8), np.asarray(v).view(np.uint8))


# ------------------------------------------------------- routing in isolation

def _gpu_route(logits, k):
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float64)).to(dev())
    sel = torch.full((k,), -1, dtype=torch.int32, device=dev())
    w = torch.full((k,), float("nan"), device=dev())
    q.qg_route_topk(lg, lg.numel(), k, sel, w)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), w.cpu().numpy()


def test_route_exhaustive_ties_bit_exact():
    for vals in itertools.product([0.0, 1.0, 2.0], repeat=6):
        lg = np.array(vals)
        for k in (1, 2, 3, 6):
            sel, w = _gpu_route(lg, k)
            rs, rw = oracle.route(lg, k)
            assert np.array_equal(sel, rs), (vals, k)
            assert np.allclose(w, rw, rtol=1e-6, atol=0)


def test_route_random_and_constructed_ties():
    g = np.random.default_rng(60)
    for trial in range(60):
        E = int(g.integers(1, 1025))
        k = int(g.integers(1, min(32, E) + 1))
        lg = g.standard_normal(E)
        if trial % 3 == 0 and E > 4:        # duplicate values across the cut
            lg[g.integers(0, E, E // 3)] = lg[int(g.integers(0, E))]
        if trial % 5 == 0:
            lg[g.integers(0, E, 3)] = -np.inf
        sel, w = _gpu_route(lg, k)
        rs, rw = oracle.route(lg, k)
        assert np.array_equal(sel, rs), (trial, E, k)
        assert np.allclose(w, rw, rtol=1e-6, atol=0)


@pytest.mark.parametrize("E", [64, 65, 128, 129, 256, 257, 512, 513, 1024])
def test_route_key_slot_boundaries(E):
    # each lane keeps ceil(E/64) keys rounded up to a power of two; the
    # winners are planted in the last lane and the last slot
    g = np.random.default_rng(70 + E)
    lg = g.standard_normal(E)
    lg[E - 1] = 9.0
    lg[63] = 8.0
    lg[E // 2] = 8.0
    for k in (1, 3, 8):
        sel, w = _gpu_route(lg, k)
        rs, rw = oracle.route(lg, k)
        assert np.array_equal(sel, rs), (E, k)
        assert np.allclose(w, rw, rtol=1e-6, atol=0)


def test_route_nan_logits_rank_last():
    lg = np.array([np.nan, 3.0, np.nan, -1.0, 0.0])
    sel, _ = _gpu_route(lg, 4)
    assert list(sel) == list(oracle.route(lg, 4)[0]) == [1, 4, 3, 0]


@pytest.mark.parametrize("E,k", [(6, 4), (128, 8), (300, 9), (1024, 32)])
def test_route_all_negative_logits(E, k):
    # every chosen logit negative (order keys with the sign flipped) and
    # low key halves with the top bit set: the weights are formed from the
    # chosen keys themselves
    g = np.random.default_rng(80 + E)
    lg = -np.abs(g.standard_normal(E)) - 0.5
    sel, w = _gpu_route(lg, k)
    rs, rw = oracle.route(lg, k)
    assert np.array_equal(sel, rs)
    assert np.allclose(w, rw, rtol=1e-6, atol=0)
    assert abs(float(np.sum(w.astype(np.float64))) - 1.0) < 1e-6
