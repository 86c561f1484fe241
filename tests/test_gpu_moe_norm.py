"""GPU parity of moe_ffn_norm (fused residual add + RMSNorm in front of the
MoE FFN) against the oracle.

The normed activations must equal the oracle's to one f32 ulp (both compute
the norm in f64 and round once; only the order of the f64 sum of squares
differs), the residual stream h = attn_out + hidden_in exactly, the expert
selection bit for bit, route weights to 1e-6 relative, and every output
row to 1e-4 * (|h| + sum_s sum_j |D a|) + 1e-6.
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

EPS = float(np.float32(synth.NORM_EPS))  # the f32 value the C ABI receives


class MoeNorm:
    def __init__(self, router, gate, up, down, gate_fmt, down_fmt, E, k, H, F, offset=0):
        self.E, self.k, self.H, self.F = E, k, H, F
        self.gate_fmt, self.down_fmt = gate_fmt, down_fmt
        self.router, self.gate, self.up, self.down = router, gate, up, down
        self.d_router = torch.from_numpy(np.ascontiguousarray(router)).to(dev())
        self.d_gate = DeviceBytes(gate, offset)
        self.d_up = DeviceBytes(up, offset)
        self.d_down = DeviceBytes(down, offset)
        self.ws_bytes = q.moe_ffn_norm_workspace_bytes(H, E, k, F)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev())

    def gpu(self, attn, hid, wn, alias=None, normed=True, eps=EPS):
        ad = torch.from_numpy(attn).to(dev())
        hd = torch.from_numpy(hid).to(dev())
        wd = torch.from_numpy(wn).to(dev())
        out = {"attn": ad, "hid": hd}.get(alias)
        if out is None:
            out = torch.full_like(hd, float("nan"))
        xn = torch.full_like(hd, float("nan")) if normed else None
        sel = torch.full((self.k,), -1, dtype=torch.int32, device=dev())
        w = torch.full((self.k,), float("nan"), device=dev())
        q.moe_ffn_norm(ad, hd, out, wd, eps, xn, self.d_router, self.gate_fmt, self.d_gate.ptr,
                       self.gate_fmt, self.d_up.ptr, self.down_fmt, self.d_down.ptr, self.H,
                       self.E, self.k, self.F, sel, w, self.ws, self.ws_bytes)
        torch.cuda.synchronize()
        logits = self.ws[:8 * self.E].view(torch.float64).cpu().numpy()
        return (out.cpu().numpy(), None if xn is None else xn.cpu().numpy(), sel.cpu().numpy(),
                w.cpu().numpy(), logits)

    def ref(self, attn, hid, wn):
        return oracle.moe_ffn_norm(attn, hid, wn, EPS, self.router, self.gate_fmt, self.gate,
                                   self.gate_fmt, self.up, self.down_fmt, self.down, self.H,
                                   self.E, self.k, self.F)


def _compare(m, attn, hid, wn, what, alias=None):
    r = m.ref(attn, hid, wn)
    y, xn, sel, w, logits = m.gpu(attn, hid, wn, alias=alias)
    assert np.array_equal(r["h"], attn + hid)
    spacing = np.spacing(np.abs(r["xn"])).astype(np.float64)
    assert np.all(np.abs(xn.astype(np.float64) - r["xn"]) <= spacing), what
    lb = np.abs(m.router.astype(np.float64)) @ np.abs(r["xn"].astype(np.float64))
    assert np.all(np.abs(logits - r["logits"]) <= 1e-12 * lb), what
    assert np.array_equal(sel, r["sel"]), (what, sel, r["sel"])
    assert np.allclose(w, r["w"], rtol=1e-6, atol=0), what
    assert_agree(y, r["y"], r["bound"], what)


def _small(gate_fmt, down_fmt, E=6, k=2, H=512, F=256, seed=31, offset=0):
    g = synth.rng(seed)
    router = synth.f32_matrix(g, E, H, 0.02)
    gate = synth.matrix(g, gate_fmt, E * F, H)
    up = synth.matrix(g, gate_fmt, E * F, H)
    down = synth.matrix(g, down_fmt, E * H, F)
    return MoeNorm(router, gate, up, down, gate_fmt, down_fmt, E, k, H, F, offset), g


@pytest.mark.parametrize("gate_fmt,down_fmt", [
    (q.QG_Q4_K, q.QG_Q6_K), (q.QG_Q5_K, q.QG_Q4_K), (q.QG_Q8_0, q.QG_Q4_0),
])
def test_small_moe_norm(gate_fmt, down_fmt):
    m, g = _small(gate_fmt, down_fmt, seed=31 + gate_fmt)
    for t in range(3):
        attn = synth.activations(g, 1, m.H)[0]
        hid = (4 * synth.activations(g, 1, m.H)[0]).astype(np.float32)
        wn = (1 + 0.1 * g.standard_normal(m.H)).astype(np.float32)
        _compare(m, attn, hid, wn, f"small norm {gate_fmt}/{down_fmt} token {t}")


@pytest.mark.parametrize("alias", ["attn", "hid"])
def test_output_may_alias_either_input(alias):
    m, g = _small(q.QG_Q4_K, q.QG_Q6_K, seed=41, offset=2)
    attn = synth.activations(g, 1, m.H)[0]
    hid = synth.activations(g, 1, m.H)[0]
    wn = (1 + 0.1 * g.standard_normal(m.H)).astype(np.float32)
    _compare(m, attn, hid, wn, f"alias {alias}", alias=alias)


def test_normed_output_is_optional():
    m, g = _small(q.QG_Q4_K, q.QG_Q6_K, seed=42)
    attn = synth.activations(g, 1, m.H)[0]
    hid = synth.activations(g, 1, m.H)[0]
    wn = np.ones(m.H, np.float32)
    y1, xn, sel1, _, _ = m.gpu(attn, hid, wn)
    y2, none, sel2, _, _ = m.gpu(attn, hid, wn, normed=False)
    assert none is None and np.array_equal(y1, y2) and np.array_equal(sel1, sel2)


def test_unit_rms_stream_matches_plain_moe_ffn():
    # attn_out = 0, hidden = +-1, weight = 1, eps = 0: xn = hidden exactly, so
    # the normed chain and moe_ffn(x = hidden, residual = hidden) agree bit for bit
    m, g = _small(q.QG_Q4_K, q.QG_Q6_K, seed=43)
    hid = np.where(g.standard_normal(m.H) < 0, -1.0, 1.0).astype(np.float32)
    y, xn, sel, w, _ = m.gpu(np.zeros(m.H, np.float32), hid, np.ones(m.H, np.float32), eps=0.0)
    assert np.array_equal(xn, hid)
    hd = torch.from_numpy(hid).to(dev())
    y2 = torch.empty_like(hd)
    sel2 = torch.empty(m.k, dtype=torch.int32, device=dev())
    w2 = torch.empty(m.k, device=dev())
    ws = torch.empty(q.moe_ffn_workspace_bytes(m.E, m.k, m.F), dtype=torch.uint8, device=dev())
    q.moe_ffn(hd, hd.clone(), y2, m.d_router, m.gate_fmt, m.d_gate.ptr, m.gate_fmt, m.d_up.ptr,
              m.down_fmt, m.d_down.ptr, m.H, m.E, m.k, m.F, sel2, w2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(sel, sel2.cpu().numpy())
    assert np.array_equal(w, w2.cpu().numpy())
    assert np.array_equal(y, y2.cpu().numpy())


def test_qwen3_moe_norm_shape_several_tokens():
    case = synth.MOE_CASE
    router, gate, up, down = synth.moe_weights(case)
    m = MoeNorm(router, gate, up, down, case.gate_fmt, case.down_fmt, case.n_experts,
                case.top_k, case.hidden, case.expert_dim)
    attn, hid, wn = synth.moe_norm_inputs(case)
    # a window of 16 of the 64 tokens
    for t in range(16):
        _compare(m, attn[t], hid[t], wn, f"qwen3 norm token {t}")


def test_wide_hidden_two_pass_norm():
    # H > 2048: the router kernel reduces the sum of squares over several
    # rounds before its dot products
    m, g = _small(q.QG_Q4_K, q.QG_Q6_K, E=4, k=2, H=4096, F=256, seed=44)
    for t in range(2):
        attn = synth.activations(g, 1, m.H)[0]
        hid = synth.activations(g, 1, m.H)[0]
        wn = (1 + 0.1 * g.standard_normal(m.H)).astype(np.float32)
        _compare(m, attn, hid, wn, f"wide norm token {t}")
