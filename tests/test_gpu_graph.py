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


def _replays_match(run, outs, what, reps=4):
    run()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    graph = _capture(run)
    for rep in range(reps):
        for o in outs:
            o.fill_(float("nan") if o.dtype.is_floating_point else -1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, eager):
            assert torch.equal(o, ref), (what, rep)
        run()                      # eager work between replays
        torch.cuda.synchronize()


def _moe_weights(seed, E, H, F):
    g = synth.rng(seed)
    router = torch.from_numpy(synth.f32_matrix(g, E, H, 0.02)).cuda()
    gate = torch.from_numpy(synth.matrix(g, q.QG_Q4_K, E * F, H).reshape(-1)).cuda()
    up = torch.from_numpy(synth.matrix(g, q.QG_Q4_K, E * F, H).reshape(-1)).cuda()
    down = torch.from_numpy(synth.matrix(g, q.QG_Q6_K, E * H, F).reshape(-1)).cuda()
    return g, router, gate, up, down


def test_moe_norm_graph_replays_match_eager():
    E, k, H, F = 16, 4, 512, 256
    g, router, gate, up, down = _moe_weights(960, E, H, F)
    attn = torch.from_numpy(synth.activations(g, 3, H)).cuda()
    hid = torch.from_numpy(synth.activations(g, 3, H)).cuda()
    wn = torch.from_numpy((1 + 0.1 * g.standard_normal(H)).astype(np.float32)).cuda()
    out = torch.empty_like(hid)
    xn = torch.empty_like(hid)
    sel = torch.empty(3, k, dtype=torch.int32, device="cuda")
    w = torch.empty(3, k, device="cuda")
    wsb = q.moe_ffn_norm_workspace_bytes(H, E, k, F)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")

    def run():
        for t in range(3):
            q.moe_ffn_norm(attn[t], hid[t], out[t], wn, 1e-6, xn[t], router, q.QG_Q4_K, gate,
                           q.QG_Q4_K, up, q.QG_Q6_K, down, H, E, k, F, sel[t], w[t], ws, wsb)

    _replays_match(run, [out, xn, sel, w], "moe_ffn_norm")


@pytest.mark.parametrize("T", [3, 8])
def test_moe_tokens_graph_replays_match_eager(T):
    E, k, H, F = 16, 4, 512, 256
    g, router, gate, up, down = _moe_weights(970 + T, E, H, F)
    x = torch.from_numpy(synth.activations(g, T, H)).cuda()
    res = torch.from_numpy(synth.activations(g, T, H)).cuda()
    y = torch.empty_like(x)
    sel = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, device="cuda")
    wsb = q.moe_ffn_tokens_workspace_bytes(T, E, k, F)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")

    def run():
        q.moe_ffn_tokens(x, res, y, router, q.QG_Q4_K, gate, q.QG_Q4_K, up, q.QG_Q6_K, down, T,
                         H, E, k, F, sel, w, ws, wsb)

    _replays_match(run, [y, sel, w], f"moe_ffn_tokens T={T}")


def test_q8act_and_sliced_gemv_graph_replays_match_eager():
    g = synth.rng(990)
    Wq = torch.from_numpy(synth.matrix(g, q.QG_Q6_K, 300, 2048).reshape(-1)).cuda()
    xq = torch.from_numpy(synth.activations(g, 1, 2048)[0]).cuda()
    yq = torch.empty(300, device="cuda")
    # batch 8 on 4096 columns and 8200 rows: two matrix-core column slices
    Ws = torch.from_numpy(synth.matrix(g, q.QG_Q5_K, 8200, 4096).reshape(-1)).cuda()
    Xs = torch.from_numpy(synth.activations(g, 8, 4096)).cuda()
    Ys = torch.empty(8, 8200, device="cuda")

    def run():
        q.qgemv_q8act(q.QG_Q6_K, Wq, 300, 2048, xq, yq)
        q.qgemv(q.QG_Q5_K, Ws, 8200, 4096, Xs, Ys, 8)

    _replays_match(run, [yq, Ys], "q8act + slices")


def test_qgemv_ws_graph_replays_match_eager():
    # the shared-operand kernel with its column ranges summed by the second
    # kernel (workspace written whole on every call), at batch 8 (packed
    # operands), 24 (two blocks of 16 rows) and 40 (two launches)
    g = synth.rng(995)
    cases = [(q.QG_Q5_K, 1000, 4352, 8), (q.QG_Q4_0, 300, 4096, 24), (q.QG_Q4_K, 200, 4096, 40)]
    bufs = []
    for fmt, rows, cols, b in cases:
        W = torch.from_numpy(synth.matrix(g, fmt, rows, cols).reshape(-1)).cuda()
        X = torch.from_numpy(synth.activations(g, b, cols)).cuda()
        need = q.qgemv_ws_bytes(fmt, rows, cols, b)
        assert need > 0
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        bufs.append((fmt, rows, cols, b, W, X, ws, torch.empty(b, rows, device="cuda")))

    def run():
        for fmt, rows, cols, b, W, X, ws, Y in bufs:
            q.qgemv_ws(fmt, W, rows, cols, X, Y, b, ws)

    # the workspaces are overwritten before each replay too: nothing may
    # depend on what an earlier call left there
    outs = [Y for *_, Y in bufs] + [ws for *_, ws, _ in bufs]
    _replays_match(run, outs, "qgemv_ws")
