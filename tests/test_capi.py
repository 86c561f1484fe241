"""The C ABI without a GPU: the library loads, exports every declared symbol,
and refuses invalid arguments (validation runs before any HIP call)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import gguf_quant_dequant_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemv.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(q.LIB_PATH):
        from gguf_quant_dequant_amd import build
        build.build(force=True)
    return q.load_library()


def test_header_declares_the_documented_entry_points():
    assert declared_functions() == sorted(q.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_geometry_helpers(lib):
    assert [q.qg_block_elems(f) for f in (0, 2, 8, 12, 13, 14)] == [1, 32, 32, 256, 256, 256]
    assert [q.qg_block_bytes(f) for f in (0, 2, 8, 12, 13, 14)] == [4, 18, 34, 144, 176, 210]
    assert q.qg_block_elems(7) == 0 and q.qg_block_bytes(99) == 0
    assert q.qg_row_bytes(q.QG_Q6_K, 768) == 630
    assert q.qg_row_bytes(q.QG_Q4_K, 4096) == 2304
    assert q.qg_row_bytes(q.QG_Q4_0, 14336) == 8064
    assert q.qg_row_bytes(q.QG_Q4_K, 100) == -1
    assert q.qg_row_bytes(q.QG_Q8_0, 0) == -1


P = 0x10000  # a fake, aligned, never-dereferenced pointer value


@pytest.mark.parametrize("args,code,msg", [
    ((12, 0, 4, 256, P, P, 1), q.QG_EINVAL, "non-NULL"),
    ((12, P, 0, 256, P, P, 1), q.QG_EINVAL, "positive"),
    ((12, P, 4, -256, P, P, 1), q.QG_EINVAL, "positive"),
    ((12, P, 4, 255, P, P, 1), q.QG_EUNSUPPORTED, "multiple of 256"),
    ((2, P, 4, 48, P, P, 1), q.QG_EUNSUPPORTED, "multiple of 32"),
    ((12, P, 4, 256, P, P, 0), q.QG_EUNSUPPORTED, "batch"),
    ((12, P, 4, 256, P, P, 65), q.QG_EUNSUPPORTED, "batch"),
    ((12, P, 4, 256, P, P, 0), q.QG_EUNSUPPORTED, "batch"),
    ((5, P, 4, 256, P, P, 1), q.QG_EUNSUPPORTED, "unknown format"),
    ((12, P + 1, 4, 256, P, P, 1), q.QG_EINVAL, "aligned"),
    ((0, P + 2, 4, 256, P, P, 1), q.QG_EINVAL, "aligned"),
    ((12, P, 4, 256, P + 2, P, 1), q.QG_EINVAL, "aligned"),
    ((0, P, 4, 6, P, P, 1), q.QG_EUNSUPPORTED, "multiple of 4"),
    ((12, P, 4, 65792, P, P, 1), q.QG_EUNSUPPORTED, "65536"),
    ((12, P, 1 << 31, 256, P, P, 1), q.QG_EUNSUPPORTED, "2^31"),
])
def test_qgemv_refuses_before_launching(lib, args, code, msg):
    rc = lib.qgemv(*args, None)
    assert rc == code
    assert msg in q.qg_last_error()


def _moe_args(**over):
    a = dict(x=P, residual=P, y=P + 64, router=P, gate_fmt=12, gate=P, up_fmt=12, up=P,
             down_fmt=14, down=P, hidden=2048, n_experts=128, top_k=8, expert_dim=768,
             sel=P, w=P, ws=P, wsb=q.moe_ffn_workspace_bytes(128, 8, 768))
    a.update(over)
    return a


def _call_moe(lib, a):
    return lib.moe_ffn(a["x"], a["residual"], a["y"], a["router"], a["gate_fmt"], a["gate"],
                       a["up_fmt"], a["up"], a["down_fmt"], a["down"], a["hidden"],
                       a["n_experts"], a["top_k"], a["expert_dim"], a["sel"], a["w"], a["ws"],
                       a["wsb"], None)


@pytest.mark.parametrize("over,code,msg", [
    (dict(x=0), q.QG_EINVAL, "non-NULL"),
    (dict(ws=0), q.QG_EINVAL, "non-NULL"),
    (dict(top_k=129), q.QG_EINVAL, "top_k"),
    (dict(top_k=0), q.QG_EINVAL, "positive"),
    (dict(top_k=33, n_experts=128), q.QG_EUNSUPPORTED, "top_k <="),
    (dict(n_experts=2048), q.QG_EUNSUPPORTED, "n_experts <="),
    (dict(up_fmt=13), q.QG_EUNSUPPORTED, "share a format"),
    (dict(gate_fmt=0, up_fmt=0), q.QG_EUNSUPPORTED, "block format"),
    (dict(hidden=2000), q.QG_EUNSUPPORTED, "multiple of"),
    (dict(expert_dim=700), q.QG_EUNSUPPORTED, "multiple of"),
    (dict(wsb=100), q.QG_EINVAL, "workspace"),
    (dict(ws=P + 8), q.QG_EINVAL, "16-byte"),
    (dict(y=P), q.QG_EINVAL, "alias"),
    (dict(down=P + 1), q.QG_EINVAL, "2-byte"),
])
def test_moe_ffn_refuses_before_launching(lib, over, code, msg):
    assert _call_moe(lib, _moe_args(**over)) == code
    assert msg in q.qg_last_error()


def test_workspace_size(lib):
    # f64 logits, k int32 routes, k f32 weights, k*F f32 activations, 16-B sections
    assert q.moe_ffn_workspace_bytes(128, 8, 768) == 1024 + 32 + 32 + 8 * 768 * 4
    assert q.moe_ffn_workspace_bytes(6, 2, 256) == 48 + 16 + 16 + 2 * 256 * 4
    assert q.moe_ffn_workspace_bytes(4, 5, 256) == 0


@pytest.mark.parametrize("args,code", [
    ((0, 8, 2, P, P), q.QG_EINVAL),
    ((P, 8, 9, P, P), q.QG_EINVAL),
    ((P, 2048, 8, P, P), q.QG_EUNSUPPORTED),
    ((P, 64, 33, P, P), q.QG_EUNSUPPORTED),
    ((P + 4, 8, 2, P, P), q.QG_EINVAL),
])
def test_route_topk_refuses_before_launching(lib, args, code):
    assert lib.qg_route_topk(*args, None) == code


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(q.QGError):
        q._lib_backup = q._lib
        try:
            q._lib = None
            q.load_library(str(tmp_path / "nope.so"))
        finally:
            q._lib = q._lib_backup


def _norm_args(**over):
    a = dict(attn=P, hid=P + 64, out=P + 128, gamma=P + 192, eps=1e-6, normed=P + 256, router=P,
             gate_fmt=12, gate=P, up_fmt=12, up=P, down_fmt=14, down=P, hidden=2048,
             n_experts=128, top_k=8, expert_dim=768, sel=P, w=P, ws=P,
             wsb=q.moe_ffn_norm_workspace_bytes(2048, 128, 8, 768))
    a.update(over)
    return a


def _call_norm(lib, a):
    return lib.moe_ffn_norm(a["attn"], a["hid"], a["out"], a["gamma"], a["eps"], a["normed"],
                            a["router"], a["gate_fmt"], a["gate"], a["up_fmt"], a["up"],
                            a["down_fmt"], a["down"], a["hidden"], a["n_experts"], a["top_k"],
                            a["expert_dim"], a["sel"], a["w"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("over,code,msg", [
    (dict(gamma=0), q.QG_EINVAL, "norm_weight"),
    (dict(attn=0), q.QG_EINVAL, "non-NULL"),
    (dict(eps=-1e-6), q.QG_EINVAL, "eps"),
    (dict(eps=float("nan")), q.QG_EINVAL, "eps"),
    (dict(eps=float("inf")), q.QG_EINVAL, "eps"),
    (dict(normed=P + 192), q.QG_EINVAL, "normed"),
    (dict(normed=P + 64), q.QG_EINVAL, "normed"),
    (dict(gamma=P + 2), q.QG_EINVAL, "4-byte"),
    (dict(wsb=q.moe_ffn_workspace_bytes(128, 8, 768)), q.QG_EINVAL, "workspace"),
    (dict(top_k=33), q.QG_EUNSUPPORTED, "top_k <="),
])
def test_moe_ffn_norm_refuses_before_launching(lib, over, code, msg):
    assert _call_norm(lib, _norm_args(**over)) == code
    assert "moe_ffn_norm" in q.qg_last_error() and msg in q.qg_last_error()


def test_norm_workspace_size(lib):
    # the moe_ffn workspace plus H f32 normed activations, 16-byte sections
    assert q.moe_ffn_norm_workspace_bytes(2048, 128, 8, 768) == \
        q.moe_ffn_workspace_bytes(128, 8, 768) + 2048 * 4
    assert q.moe_ffn_norm_workspace_bytes(100, 6, 2, 256) == \
        q.moe_ffn_workspace_bytes(6, 2, 256) + 400
    assert q.moe_ffn_norm_workspace_bytes(0, 6, 2, 256) == 0
    assert q.moe_ffn_norm_workspace_bytes(256, 4, 5, 256) == 0


def _tok_args(**over):
    a = dict(x=P, residual=P, y=P + 64, router=P, gate_fmt=12, gate=P, up_fmt=12, up=P,
             down_fmt=14, down=P, tokens=4, hidden=2048, n_experts=128, top_k=8,
             expert_dim=768, sel=P, w=P, ws=P,
             wsb=q.moe_ffn_tokens_workspace_bytes(4, 128, 8, 768))
    a.update(over)
    return a


def _call_tok(lib, a):
    return lib.moe_ffn_tokens(a["x"], a["residual"], a["y"], a["router"], a["gate_fmt"],
                              a["gate"], a["up_fmt"], a["up"], a["down_fmt"], a["down"],
                              a["tokens"], a["hidden"], a["n_experts"], a["top_k"],
                              a["expert_dim"], a["sel"], a["w"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("over,code,msg", [
    (dict(tokens=0), q.QG_EINVAL, "tokens must be positive"),
    (dict(tokens=9), q.QG_EUNSUPPORTED, "1..8"),
    (dict(tokens=8, top_k=9, wsb=1 << 30), q.QG_EUNSUPPORTED, "tokens * top_k"),
    (dict(wsb=q.moe_ffn_workspace_bytes(128, 8, 768)), q.QG_EINVAL, "workspace"),
    (dict(x=0), q.QG_EINVAL, "non-NULL"),
    (dict(y=P), q.QG_EINVAL, "alias"),
])
def test_moe_ffn_tokens_refuses_before_launching(lib, over, code, msg):
    assert _call_tok(lib, _tok_args(**over)) == code
    assert "moe_ffn_tokens" in q.qg_last_error() and msg in q.qg_last_error()


def test_tokens_workspace_size(lib):
    # T * E f64 logits, T * k routes and weights, T * k * F activations,
    # 16-byte sections
    assert q.moe_ffn_tokens_workspace_bytes(1, 128, 8, 768) == q.moe_ffn_workspace_bytes(128, 8, 768)
    assert q.moe_ffn_tokens_workspace_bytes(4, 128, 8, 768) == \
        4 * 128 * 8 + 4 * 8 * 4 + 4 * 8 * 4 + 4 * 8 * 768 * 4
    assert q.moe_ffn_tokens_workspace_bytes(3, 6, 2, 256) == 144 + 32 + 32 + 3 * 2 * 256 * 4
    assert q.moe_ffn_tokens_workspace_bytes(0, 6, 2, 256) == 0


@pytest.mark.parametrize("args,code,msg", [
    ((0, P, 4, 256, P, P), q.QG_EUNSUPPORTED, "no int8 path"),
    ((12, 0, 4, 256, P, P), q.QG_EINVAL, "non-NULL"),
    ((12, P, 0, 256, P, P), q.QG_EINVAL, "positive"),
    ((12, P, 4, 255, P, P), q.QG_EUNSUPPORTED, "multiple of 256"),
    ((12, P + 1, 4, 256, P, P), q.QG_EINVAL, "2-byte"),
    ((12, P, 4, 256, P + 2, P), q.QG_EINVAL, "4-byte"),
    ((12, P, 4, 33024, P, P), q.QG_EUNSUPPORTED, "row width"),
])
def test_qgemv_q8act_refuses_before_launching(lib, args, code, msg):
    assert lib.qgemv_q8act(*args, None) == code
    assert "qgemv_q8act" in q.qg_last_error() and msg in q.qg_last_error()
