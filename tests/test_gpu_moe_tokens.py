"""GPU parity of moe_ffn_tokens (several decode tokens, each routed on its
own, expert GEMVs grouped by expert) against the oracle, which runs the
MoE FFN token by token.

Formats, T = 2..8, 64 routes over up to 1024 experts (routed in the
gate/up workgroups and routed ahead), shared and identical tokens, one
token, the Qwen3 shape on all 64 bench tokens, a non-finite token, wide
hidden rows.  Per token: the selection bit for bit, route weights to 1e-6 relative, the
router logits to 1e-12 of sum |R x|, and every output row to
1e-4 * (|residual| + sum_s sum_j |D a|) + 1e-6.
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


class MoeTokens:
    def __init__(self, router, gate, up, down, gate_fmt, down_fmt, E, k, H, F, offset=0):
        self.E, self.k, self.H, self.F = E, k, H, F
        self.gate_fmt, self.down_fmt = gate_fmt, down_fmt
        self.router, self.gate, self.up, self.down = router, gate, up, down
        self.d_router = torch.from_numpy(np.ascontiguousarray(router)).to(dev())
        self.d_gate = DeviceBytes(gate, offset)
        self.d_up = DeviceBytes(up, offset)
        self.d_down = DeviceBytes(down, offset)

    def gpu(self, x, res, alias=False):
        T = x.shape[0]
        xd = torch.from_numpy(np.ascontiguousarray(x)).to(dev())
        rd = torch.from_numpy(np.ascontiguousarray(res)).to(dev())
        y = rd if alias else torch.full_like(rd, float("nan"))
        sel = torch.full((T, self.k), -1, dtype=torch.int32, device=dev())
        w = torch.full((T, self.k), float("nan"), device=dev())
        wsb = q.moe_ffn_tokens_workspace_bytes(T, self.E, self.k, self.F)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev())
        q.moe_ffn_tokens(xd, rd, y, self.d_router, self.gate_fmt, self.d_gate.ptr, self.gate_fmt,
                         self.d_up.ptr, self.down_fmt, self.d_down.ptr, T, self.H, self.E,
                         self.k, self.F, sel, w, ws, wsb)
        torch.cuda.synchronize()
        logits = ws[:8 * T * self.E].view(torch.float64).reshape(T, self.E).cpu().numpy()
        return y.cpu().numpy(), sel.cpu().numpy(), w.cpu().numpy(), logits

    def ref(self, x, res):
        return oracle.moe_ffn_tokens(x, res, self.router, self.gate_fmt, self.gate,
                                     self.gate_fmt, self.up, self.down_fmt, self.down, self.H,
                                     self.E, self.k, self.F)


def _compare(m, x, res, what, alias=False):
    r = m.ref(x, res)
    y, sel, w, logits = m.gpu(x, res, alias=alias)
    for t in range(x.shape[0]):
        lb = np.abs(m.router.astype(np.float64)) @ np.abs(x[t].astype(np.float64))
        assert np.all(np.abs(logits[t] - r["logits"][t]) <= 1e-12 * lb), (what, t)
        assert np.array_equal(sel[t], r["sel"][t]), (what, t, sel[t], r["sel"][t])
        assert np.allclose(w[t], r["w"][t], rtol=1e-6, atol=0), (what, t)
        assert_agree(y[t], r["y"][t], r["bound"][t], f"{what} token {t}")


def _small(gate_fmt, down_fmt, E=6, k=2, H=512, F=256, seed=51, offset=0):
    g = synth.rng(seed)
    router = synth.f32_matrix(g, E, H, 0.02)
    gate = synth.matrix(g, gate_fmt, E * F, H)
    up = synth.matrix(g, gate_fmt, E * F, H)
    down = synth.matrix(g, down_fmt, E * H, F)
    return MoeTokens(router, gate, up, down, gate_fmt, down_fmt, E, k, H, F, offset), g


@pytest.mark.parametrize("gate_fmt,down_fmt", [
    (q.QG_Q4_K, q.QG_Q6_K), (q.QG_Q5_K, q.QG_Q4_K), (q.QG_Q8_0, q.QG_Q4_0),
    (q.QG_Q4_0, q.QG_Q8_0), (q.QG_Q6_K, q.QG_Q5_K),
])
@pytest.mark.parametrize("T", [2, 5, 8])
def test_small_tokens_every_format(gate_fmt, down_fmt, T):
    m, g = _small(gate_fmt, down_fmt, seed=51 + gate_fmt)
    x = synth.activations(g, T, m.H)
    res = synth.activations(g, T, m.H)
    _compare(m, x, res, f"tokens {T} {gate_fmt}/{down_fmt}")


@pytest.mark.parametrize("E,k,T", [(1024, 8, 8), (1000, 32, 2), (130, 16, 4)])
def test_sixty_four_routes_over_many_experts(E, k, T):
    # the most routes a call takes (T * k = 64): 1024 experts routed ahead
    # (the distinct-expert search over 1024 words of LDS), 1000 experts (not
    # a multiple of 64) and 130 routed in the gate/up workgroups
    m, g = _small(q.QG_Q4_K, q.QG_Q8_0, E=E, k=k, H=256, F=64, seed=71 + E + k)
    x = synth.activations(g, T, m.H)
    res = synth.activations(g, T, m.H)
    _compare(m, x, res, f"E {E} k {k} T {T}")


def test_tokens_sharing_every_expert_and_alias():
    # E = k: every token selects every expert, so each expert serves all T
    # tokens in a different slot; the output overwrites the residual
    m, g = _small(q.QG_Q4_K, q.QG_Q6_K, E=4, k=4, seed=61, offset=2)
    x = synth.activations(g, 8, m.H)
    res = synth.activations(g, 8, m.H)
    _compare(m, x, res, "E = k", alias=True)


def test_identical_tokens_match_single_token_moe():
    # T copies of one token: every copy equals moe_ffn on it (the routing and
    # the down GEMVs bit for bit; the grouped gate/up to the tolerance)
    m, g = _small(q.QG_Q4_K, q.QG_Q6_K, E=8, k=2, seed=62)
    x1 = synth.activations(g, 1, m.H)
    r1 = synth.activations(g, 1, m.H)
    y, sel, w, _ = m.gpu(np.repeat(x1, 4, 0), np.repeat(r1, 4, 0))
    assert all(np.array_equal(sel[t], sel[0]) for t in range(4))
    assert all(np.array_equal(y[t], y[0]) for t in range(4))
    _compare(m, np.repeat(x1, 4, 0), np.repeat(r1, 4, 0), "repeated token")


def test_one_token_is_moe_ffn():
    m, g = _small(q.QG_Q4_K, q.QG_Q6_K, E=8, k=2, seed=63)
    x = synth.activations(g, 1, m.H)
    res = synth.activations(g, 1, m.H)
    y, sel, w, _ = m.gpu(x, res)
    xd = torch.from_numpy(x[0]).to(dev())
    rd = torch.from_numpy(res[0]).to(dev())
    y2 = torch.empty_like(rd)
    sel2 = torch.empty(m.k, dtype=torch.int32, device=dev())
    w2 = torch.empty(m.k, device=dev())
    ws = torch.empty(q.moe_ffn_workspace_bytes(m.E, m.k, m.F), dtype=torch.uint8, device=dev())
    q.moe_ffn(xd, rd, y2, m.d_router, m.gate_fmt, m.d_gate.ptr, m.gate_fmt, m.d_up.ptr,
              m.down_fmt, m.d_down.ptr, m.H, m.E, m.k, m.F, sel2, w2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(y[0], y2.cpu().numpy())
    assert np.array_equal(sel[0], sel2.cpu().numpy()) and np.array_equal(w[0], w2.cpu().numpy())


@pytest.mark.parametrize("T", [2, 4, 8])
def test_qwen3_moe_shape_tokens(T):
    case = synth.MOE_CASE
    router, gate, up, down = synth.moe_weights(case)
    m = MoeTokens(router, gate, up, down, case.gate_fmt, case.down_fmt, case.n_experts,
                  case.top_k, case.hidden, case.expert_dim)
    xs, rs = synth.moe_tokens(case)
    _compare(m, xs[:T], rs[:T], f"qwen3 {T} tokens")


def test_qwen3_moe_shape_all_64_tokens_in_calls_of_8():
    # every token the benchmark routes, eight calls of eight tokens
    case = synth.MOE_CASE
    router, gate, up, down = synth.moe_weights(case)
    m = MoeTokens(router, gate, up, down, case.gate_fmt, case.down_fmt, case.n_experts,
                  case.top_k, case.hidden, case.expert_dim)
    xs, rs = synth.moe_tokens(case)
    for t0 in range(0, xs.shape[0], 8):
        _compare(m, xs[t0:t0 + 8], rs[t0:t0 + 8], f"qwen3 tokens {t0}..{t0 + 7}")


def test_non_finite_token_does_not_reach_other_tokens_logits():
    # H = 512 is not a multiple of the router's 1024-column round: the
    # columns past H of token 0 must read as zero, not as token 1's values
    m, g = _small(q.QG_Q4_K, q.QG_Q6_K, E=8, k=2, H=512, seed=64)
    x = synth.activations(g, 2, m.H)
    x[1, 3] = np.inf
    x[1, 100] = np.nan
    res = synth.activations(g, 2, m.H)
    y, sel, w, logits = m.gpu(x, res)
    r = oracle.moe_ffn(x[0], res[0], m.router, m.gate_fmt, m.gate, m.gate_fmt, m.up, m.down_fmt,
                       m.down, m.H, m.E, m.k, m.F)
    assert np.all(np.isfinite(logits[0]))
    lb = np.abs(m.router.astype(np.float64)) @ np.abs(x[0].astype(np.float64))
    assert np.all(np.abs(logits[0] - r["logits"]) <= 1e-12 * lb)
    assert np.array_equal(sel[0], r["sel"])
    assert_agree(y[0], r["y"], r["bound"], "token 0 beside a non-finite token")


@pytest.mark.parametrize("T", [3, 6])
def test_hidden_of_32768_columns(T):
    # the widest hidden the chain takes (512 lane tiles of the single-token
    # kernels): 128 chunks of 256 columns per gate / up row, Q8_0 down rows
    # of 64 columns
    E, k, H, F = 4, 2, 32768, 64
    g = synth.rng(71 + T)
    router = synth.f32_matrix(g, E, H, 0.02)
    gate = synth.matrix(g, q.QG_Q4_K, E * F, H)
    up = synth.matrix(g, q.QG_Q4_K, E * F, H)
    down = synth.matrix(g, q.QG_Q8_0, E * H, F)
    m = MoeTokens(router, gate, up, down, q.QG_Q4_K, q.QG_Q8_0, E, k, H, F)
    x = synth.activations(g, T, H)
    res = synth.activations(g, T, H)
    _compare(m, x, res, f"hidden 32768, {T} tokens")
