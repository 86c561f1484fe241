"""moe_ffn_noalloc, the entry point that allocates nothing (its workspace is
the library's own device scratch array), against moe_ffn with a caller
workspace on the same inputs: two calls in a row, the second with smaller
sizes, each bit for bit equal to moe_ffn (the same kernels), and moe_ffn
itself within the oracle's tolerance.  Called through the C ABI (ctypes).
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


def _case(E, k, H, F, seed):
    g = synth.rng(seed)
    router = synth.f32_matrix(g, E, H, 0.02)
    gate = synth.matrix(g, q.QG_Q4_K, E * F, H)
    up = synth.matrix(g, q.QG_Q4_K, E * F, H)
    down = synth.matrix(g, q.QG_Q6_K, E * H, F)
    x = synth.activations(g, 1, H)[0]
    res = synth.activations(g, 1, H)[0]
    return router, gate, up, down, x, res


def _run_both(E, k, H, F, seed):
    router, gate, up, down, x, res = _case(E, k, H, F, seed)
    lib = q.load_library()
    dr = torch.from_numpy(router).to(dev())
    dg, du, dd = DeviceBytes(gate), DeviceBytes(up), DeviceBytes(down)
    xd = torch.from_numpy(x).to(dev())
    rd = torch.from_numpy(res).to(dev())
    st = torch.cuda.current_stream().cuda_stream
    out = []
    for noalloc in (True, False):
        y = torch.full_like(rd, float("nan"))
        sel = torch.full((k,), -1, dtype=torch.int32, device=dev())
        w = torch.full((k,), float("nan"), device=dev())
        if noalloc:
            rc = lib.moe_ffn_noalloc(xd.data_ptr(), rd.data_ptr(), y.data_ptr(), dr.data_ptr(),
                                     q.QG_Q4_K, dg.ptr, q.QG_Q4_K, du.ptr, q.QG_Q6_K, dd.ptr,
                                     H, E, k, F, sel.data_ptr(), w.data_ptr(), st)
        else:
            wsb = lib.moe_ffn_workspace_bytes(E, k, F)
            ws = torch.empty(wsb, dtype=torch.uint8, device=dev())
            rc = lib.moe_ffn(xd.data_ptr(), rd.data_ptr(), y.data_ptr(), dr.data_ptr(),
                             q.QG_Q4_K, dg.ptr, q.QG_Q4_K, du.ptr, q.QG_Q6_K, dd.ptr, H, E, k, F,
                             sel.data_ptr(), w.data_ptr(), ws.data_ptr(), wsb, st)
        assert rc == q.QG_OK, q.qg_last_error()
        torch.cuda.synchronize()
        out.append((y.cpu().numpy(), sel.cpu().numpy(), w.cpu().numpy()))
    r = oracle.moe_ffn(x, res, router, q.QG_Q4_K, gate, q.QG_Q4_K, up, q.QG_Q6_K, down,
                       H, E, k, F)
    return out, r


def test_noalloc_matches_moe_ffn_twice_second_smaller():
    for (E, k, H, F, seed) in ((128, 8, 2048, 768, 901), (16, 4, 512, 256, 902)):
        ((yn, sn, wn), (ya, sa, wa)), r = _run_both(E, k, H, F, seed)
        assert np.array_equal(sn, sa) and np.array_equal(sn, r["sel"]), (E, sn, sa)
        assert np.array_equal(wn.view(np.uint32), wa.view(np.uint32))
        assert np.array_equal(yn.view(np.uint32), ya.view(np.uint32))
        assert_agree(ya, r["y"], r["bound"], f"moe_ffn E{E}")


def test_noalloc_refuses_sizes_beyond_its_scratch():
    lib = q.load_library()
    # 32 routes of 8192 activations: 1 MiB of activations alone
    assert lib.moe_ffn_workspace_bytes(64, 32, 8192) > (1 << 20)
    z = torch.zeros(8, device=dev())
    rc = lib.moe_ffn_noalloc(z.data_ptr(), z.data_ptr(), z.data_ptr(), z.data_ptr(), q.QG_Q4_K,
                             z.data_ptr(), q.QG_Q4_K, z.data_ptr(), q.QG_Q6_K, z.data_ptr(),
                             256, 64, 32, 8192, None, None, None)
    assert rc == q.QG_EUNSUPPORTED
    assert "scratch" in q.qg_last_error()
