"""qgemv and moe_ffn captured in a HIP graph (as the benchmark runs them):
every replay must reproduce the eager result bit for bit, with eager work
and synchronisations between the replays."""
from __future__ import annotations

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gguf_quant_dequant_amd as q  # noqa: E402


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def test_qgemv_graph_replays_match_eager():
    cases = [(q.QG_Q4_K, 512, 4096, 1), (q.QG_Q6_K, 300, 2048, 4), (q.QG_Q4_0, 64, 1024, 8)]
    bufs = []
    for fmt, rows, cols, b in cases:
        g = synth.rng(900 + fmt)
        W = torch.from_numpy(synth.matrix(g, fmt, rows, cols).reshape(-1)).cuda()
        X = torch.from_numpy(synth.activations(g, b, cols)).cuda()
        bufs.append((fmt, rows, cols, b, W, X, torch.empty(b, rows, device="cuda")))

    def run():
        for fmt, rows, cols, b, W, X, Y in bufs:
            q.qgemv(fmt, W, rows, cols, X, Y, b)

    run()
    torch.cuda.synchronize()
    eager = [Y.clone() for *_, Y in bufs]
    graph = _capture(run)
    for rep in range(4):
        for *_, Y in bufs:
            Y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (fmt, *_, Y), ref in zip(bufs, eager):
            assert torch.equal(Y, ref), (rep, fmt)
        run()                      # eager work between replays
        torch.cuda.synchronize()


def test_moe_graph_replays_match_eager():
    E, k, H, F = 16, 4, 512, 256
    g = synth.rng(950)
    router = torch.from_numpy(synth.f32_matrix(g, E, H, 0.02)).cuda()
    gate = torch.from_numpy(synth.matrix(g, q.QG_Q4_K, E * F, H).reshape(-1)).cuda()
    up = torch.from_numpy(synth.matrix(g, q.QG_Q4_K, E * F, H).reshape(-1)).cuda()
    down = torch.from_numpy(synth.matrix(g, q.QG_Q6_K, E * H, F).reshape(-1)).cuda()
    xs = torch.from_numpy(synth.activations(g, 3, H)).cuda()
    rs = torch.from_numpy(synth.activations(g, 3, H)).cuda()
    ys = torch.empty_like(xs)
    sel = torch.empty(3, k, dtype=torch.int32, device="cuda")
    w = torch.empty(3, k, device="cuda")
    wsb = q.moe_ffn_workspace_bytes(E, k, F)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")

    def run():
        for t in range(3):
            q.moe_ffn(xs[t], rs[t], ys[t], router, q.QG_Q4_K, gate, q.QG_Q4_K, up, q.QG_Q6_K,
                      down, H, E, k, F, sel[t], w[t], ws, wsb)

    run()
    torch.cuda.synchronize()
    ref = (ys.clone(), sel.clone(), w.clone())
    graph = _capture(run)
    for rep in range(4):
        ys.fill_(float("nan"))
        sel.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys, ref[0]) and torch.equal(sel, ref[1]) and torch.equal(w, ref[2])
        run()
        torch.cuda.synchronize()
    assert np.isfinite(ys.cpu().numpy()).all()
