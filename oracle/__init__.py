"""CPU oracle for the GGUF dequantise-and-dot GEMV and the stacked-expert MoE FFN.

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  The product library
never imports, links or runs anything here, and nothing here imports the
product library.

The arithmetic lives in ``qref.c`` (plain C, double precision, built with
``-ffp-contract=off``); this module only builds it and marshals numpy arrays.
Each C function names the web page and the item on it that it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qref.c")
_LIB_PATH = os.path.join(_HERE, "libqref.so")

F32, Q4_0, Q8_0, Q4_K, Q5_K, Q6_K = 0, 2, 8, 12, 13, 14
OK, EINVAL, EUNSUPPORTED = 0, 1, 2

_lib: Optional[ctypes.CDLL] = None


def build(force: bool = True) -> str:
    """Compile qref.c into libqref.so with gcc (plain C, no contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    ci = ctypes.c_int
    lib.qref_block_elems.argtypes = [ci]
    lib.qref_block_elems.restype = ci
    lib.qref_block_bytes.argtypes = [ci]
    lib.qref_block_bytes.restype = ci
    lib.qref_row_bytes.argtypes = [ci, i64]
    lib.qref_row_bytes.restype = i64
    lib.qref_f16.argtypes = [ctypes.c_uint16]
    lib.qref_f16.restype = ctypes.c_double
    lib.qref_dequant_block.argtypes = [ci, P, P]
    lib.qref_dequant_block.restype = ci
    lib.qref_dequant_row.argtypes = [ci, P, i64, P]
    lib.qref_dequant_row.restype = ci
    lib.qref_gemv_rows.argtypes = [ci, P, i64, i64, P, ci, P, i64, P, P]
    lib.qref_gemv_rows.restype = ci
    lib.qref_gemv.argtypes = [ci, P, i64, i64, P, ci, P, P]
    lib.qref_gemv.restype = ci
    lib.qref_route.argtypes = [P, ci, ci, P, P]
    lib.qref_route.restype = ci
    lib.qref_silu.argtypes = [ctypes.c_double]
    lib.qref_silu.restype = ctypes.c_double
    lib.qref_add_rmsnorm.restype = ci
    lib.qref_add_rmsnorm.argtypes = [P, P, P, ctypes.c_double, i64, P, P]
    lib.qref_moe_ffn_norm.restype = ci
    lib.qref_moe_ffn_norm.argtypes = [P, P, P, ctypes.c_double, P, ci, P, ci, P, ci, P, i64, i64,
                                      i64, i64, P, P, P, P, P, P, P, P]
    lib.qref_quantize_q8.restype = ci
    lib.qref_quantize_q8.argtypes = [P, i64, P, P]
    lib.qref_gemv_q8act.restype = ci
    lib.qref_gemv_q8act.argtypes = [ci, P, i64, i64, P, ci, P, P]
    lib.qref_moe_ffn.argtypes = [P, P, P, ci, P, ci, P, ci, P, i64, i64, i64, i64,
                                 P, P, P, P, P, P]
    lib.qref_moe_ffn.restype = ci
    lib.qref_moe_q8act_bound.argtypes = [P, P, P, ci, P, ci, P, ci, P, i64, i64, i64, i64, P]
    lib.qref_moe_q8act_bound.restype = ci
    lib.qref_moe_ffn_q8act.argtypes = [P, P, P, ci, P, ci, P, ci, P, i64, i64, i64, i64,
                                       ctypes.c_double, P, P, P, P, P]
    lib.qref_moe_ffn_q8act.restype = ci
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]) -> Optional[int]:
    return None if a is None else a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != OK:
        raise ValueError(f"oracle {what} failed with code {rc}")


def block_elems(fmt: int) -> int:
    return _load().qref_block_elems(fmt)


def block_bytes(fmt: int) -> int:
    return _load().qref_block_bytes(fmt)


def row_bytes(fmt: int, cols: int) -> int:
    return _load().qref_row_bytes(fmt, cols)


def f16(bits: int) -> float:
    return _load().qref_f16(bits)


def dequant_block(fmt: int, blk: bytes | np.ndarray) -> np.ndarray:
    b = np.frombuffer(bytes(blk), dtype=np.uint8).copy()
    assert b.size == block_bytes(fmt)
    out = np.empty(block_elems(fmt), dtype=np.float64)
    _check(_load().qref_dequant_block(fmt, _ptr(b), _ptr(out)), "dequant_block")
    return out


def dequant_row(fmt: int, row: np.ndarray, cols: int) -> np.ndarray:
    r = np.ascontiguousarray(row, dtype=np.uint8)
    assert r.size >= row_bytes(fmt, cols)
    out = np.empty(cols, dtype=np.float64)
    _check(_load().qref_dequant_row(fmt, _ptr(r), cols, _ptr(out)), "dequant_row")
    return out


def dequant_matrix(fmt: int, W: np.ndarray, rows: int, cols: int) -> np.ndarray:
    rb = row_bytes(fmt, cols)
    Wb = np.ascontiguousarray(W).view(np.uint8).reshape(-1)
    return np.stack([dequant_row(fmt, Wb[r * rb:(r + 1) * rb], cols) for r in range(rows)])


def gemv(fmt: int, W: np.ndarray, rows: int, cols: int, X: np.ndarray,
         row_idx: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Y[b][i] = sum_c deq(W)[row_i][c] * X[b][c] in f64, and sum |w x|.

    X has shape [batch][cols] (float32).  Returns (Y, Yabs), each
    [batch][n] float64 where n = rows or len(row_idx)."""
    Wb = np.ascontiguousarray(W).view(np.uint8).reshape(-1)
    X = np.ascontiguousarray(X, dtype=np.float32)
    if X.ndim == 1:
        X = X[None, :]
    batch = X.shape[0]
    assert X.shape[1] == cols
    if row_idx is None:
        Y = np.empty((batch, rows), dtype=np.float64)
        A = np.empty((batch, rows), dtype=np.float64)
        _check(_load().qref_gemv(fmt, _ptr(Wb), rows, cols, _ptr(X), batch, _ptr(Y), _ptr(A)),
               "gemv")
    else:
        idx = np.ascontiguousarray(row_idx, dtype=np.int64)
        Y = np.empty((batch, idx.size), dtype=np.float64)
        A = np.empty((batch, idx.size), dtype=np.float64)
        _check(_load().qref_gemv_rows(fmt, _ptr(Wb), rows, cols, _ptr(X), batch, _ptr(idx),
                                      idx.size, _ptr(Y), _ptr(A)), "gemv_rows")
    return Y, A


def route(logits: np.ndarray, top_k: int) -> Tuple[np.ndarray, np.ndarray]:
    """(sel int32[k], w float64[k]) in rank order."""
    lg = np.ascontiguousarray(logits, dtype=np.float64)
    sel = np.empty(top_k, dtype=np.int32)
    w = np.empty(top_k, dtype=np.float64)
    _check(_load().qref_route(_ptr(lg), lg.size, top_k, _ptr(sel), _ptr(w)), "route")
    return sel, w


def silu(g: float) -> float:
    return _load().qref_silu(g)


def moe_ffn(x, residual, router, gate_fmt, gate, up_fmt, up, down_fmt, down,
            hidden, n_experts, top_k, expert_dim) -> dict:
    """The stacked-expert MoE FFN for one token, everything in f64.

    Returns a dict with y[H], bound[H], logits[E], sel[k], w[k], act[k][F]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    residual = np.ascontiguousarray(residual, dtype=np.float32)
    router = np.ascontiguousarray(router, dtype=np.float32)
    gate = np.ascontiguousarray(gate).view(np.uint8).reshape(-1)
    up = np.ascontiguousarray(up).view(np.uint8).reshape(-1)
    down = np.ascontiguousarray(down).view(np.uint8).reshape(-1)
    y = np.empty(hidden, dtype=np.float64)
    bound = np.empty(hidden, dtype=np.float64)
    logits = np.empty(n_experts, dtype=np.float64)
    sel = np.empty(top_k, dtype=np.int32)
    w = np.empty(top_k, dtype=np.float64)
    act = np.empty((top_k, expert_dim), dtype=np.float64)
    rc = _load().qref_moe_ffn(_ptr(x), _ptr(residual), _ptr(router), gate_fmt, _ptr(gate),
                              up_fmt, _ptr(up), down_fmt, _ptr(down), hidden, n_experts,
                              top_k, expert_dim, _ptr(y), _ptr(bound), _ptr(logits),
                              _ptr(sel), _ptr(w), _ptr(act))
    _check(rc, "moe_ffn")
    return dict(y=y, bound=bound, logits=logits, sel=sel, w=w, act=act)


def add_rmsnorm(x, residual, weight, eps: float):
    """Fused residual add + RMSNorm: (h, xn) with h = x + residual in f32 and
    xn = (h / sqrt(mean(h^2) + eps)) * weight computed in f64, rounded to f32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    residual = np.ascontiguousarray(residual, dtype=np.float32)
    weight = np.ascontiguousarray(weight, dtype=np.float32)
    n = x.shape[0]
    h = np.empty(n, dtype=np.float32)
    xn = np.empty(n, dtype=np.float32)
    _check(_load().qref_add_rmsnorm(_ptr(x), _ptr(residual), _ptr(weight), float(eps), n,
                                    _ptr(h), _ptr(xn)), "add_rmsnorm")
    return h, xn


def moe_ffn_norm(attn_out, hidden_in, norm_weight, eps, router, gate_fmt, gate, up_fmt, up,
                 down_fmt, down, hidden, n_experts, top_k, expert_dim) -> dict:
    """The MoE FFN behind the fused add + RMSNorm, everything in f64.

    Returns the moe_ffn dict plus h[H] (the new residual stream before the
    experts) and xn[H] (the normed activations the router and experts read)."""
    attn_out = np.ascontiguousarray(attn_out, dtype=np.float32)
    hidden_in = np.ascontiguousarray(hidden_in, dtype=np.float32)
    norm_weight = np.ascontiguousarray(norm_weight, dtype=np.float32)
    router = np.ascontiguousarray(router, dtype=np.float32)
    gate = np.ascontiguousarray(gate).view(np.uint8).reshape(-1)
    up = np.ascontiguousarray(up).view(np.uint8).reshape(-1)
    down = np.ascontiguousarray(down).view(np.uint8).reshape(-1)
    y = np.empty(hidden, dtype=np.float64)
    bound = np.empty(hidden, dtype=np.float64)
    logits = np.empty(n_experts, dtype=np.float64)
    sel = np.empty(top_k, dtype=np.int32)
    w = np.empty(top_k, dtype=np.float64)
    act = np.empty((top_k, expert_dim), dtype=np.float64)
    h = np.empty(hidden, dtype=np.float32)
    xn = np.empty(hidden, dtype=np.float32)
    rc = _load().qref_moe_ffn_norm(_ptr(attn_out), _ptr(hidden_in), _ptr(norm_weight), float(eps),
                                   _ptr(router), gate_fmt, _ptr(gate), up_fmt, _ptr(up), down_fmt,
                                   _ptr(down), hidden, n_experts, top_k, expert_dim, _ptr(y),
                                   _ptr(bound), _ptr(logits), _ptr(sel), _ptr(w), _ptr(act),
                                   _ptr(h), _ptr(xn))
    _check(rc, "moe_ffn_norm")
    return dict(y=y, bound=bound, logits=logits, sel=sel, w=w, act=act, h=h, xn=xn)


def moe_ffn_tokens(x, residual, router, gate_fmt, gate, up_fmt, up, down_fmt, down,
                   hidden, n_experts, top_k, expert_dim) -> dict:
    """T decode tokens through the MoE FFN: by definition each token on its
    own (the aprender-serve page's moe_layer runs per token), so this is
    moe_ffn applied to every row of x [T][H] and residual [T][H].

    Returns y[T][H], bound[T][H], logits[T][E], sel[T][k], w[T][k]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    residual = np.ascontiguousarray(residual, dtype=np.float32)
    per = [moe_ffn(x[t], residual[t], router, gate_fmt, gate, up_fmt, up, down_fmt, down,
                   hidden, n_experts, top_k, expert_dim) for t in range(x.shape[0])]
    return {key: np.stack([r[key] for r in per]) for key in ("y", "bound", "logits", "sel", "w")}


def quantize_q8(x):
    """int8 activations of the int8-activation GEMV: per 16-column group,
    d = max|x| / 127, id = 1 / d and q = rint(x * id), all f32.  Returns (q int8 [n],
    d float32 [n / 16])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    n = x.shape[0]
    q = np.empty(n, dtype=np.int8)
    d = np.empty(n // 16, dtype=np.float32)
    _check(_load().qref_quantize_q8(_ptr(x), n, _ptr(q), _ptr(d)), "quantize_q8")
    return q, d


def gemv_q8act(fmt: int, W: np.ndarray, rows: int, cols: int, X: np.ndarray):
    """GEMV on int8-quantised activations, in f64: (Y [batch][rows], sum of
    |w * x_q| [batch][rows])."""
    X = np.ascontiguousarray(X, dtype=np.float32).reshape(-1, cols)
    W = np.ascontiguousarray(W).view(np.uint8).reshape(-1)
    batch = X.shape[0]
    Y = np.empty((batch, rows), dtype=np.float64)
    A = np.empty((batch, rows), dtype=np.float64)
    _check(_load().qref_gemv_q8act(fmt, _ptr(W), rows, cols, _ptr(X), batch, _ptr(Y), _ptr(A)),
           "gemv_q8act")
    return Y, A


def moe_q8act_bound(x, residual, router, gate_fmt, gate, up_fmt, up, down_fmt, down,
                    hidden, n_experts, top_k, expert_dim) -> np.ndarray:
    """Per output row, the most the int8-activation MoE FFN may depart from
    moe_ffn's exact y (quantisation of x and of the slots' activations,
    propagated through gate/up, SwiGLU and down; see qref.c)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    residual = np.ascontiguousarray(residual, dtype=np.float32)
    router = np.ascontiguousarray(router, dtype=np.float32)
    gate = np.ascontiguousarray(gate).view(np.uint8).reshape(-1)
    up = np.ascontiguousarray(up).view(np.uint8).reshape(-1)
    down = np.ascontiguousarray(down).view(np.uint8).reshape(-1)
    qb = np.empty(hidden, dtype=np.float64)
    _check(_load().qref_moe_q8act_bound(_ptr(x), _ptr(residual), _ptr(router), gate_fmt,
                                        _ptr(gate), up_fmt, _ptr(up), down_fmt, _ptr(down),
                                        hidden, n_experts, top_k, expert_dim, _ptr(qb)),
           "moe_q8act_bound")
    return qb


def moe_ffn_q8act(x, residual, router, gate_fmt, gate, up_fmt, up, down_fmt, down,
                  hidden, n_experts, top_k, expert_dim, tie_window: float = 0.0) -> dict:
    """The MoE FFN with its expert GEMVs on int8 activations (see qref.c).

    Returns y[H], bound[H] (|residual| + sum |D aq|), tie[H] (the row's
    sensitivity to one-step changes of codes within tie_window of a rounding
    tie), sel[k], w[k]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    residual = np.ascontiguousarray(residual, dtype=np.float32)
    router = np.ascontiguousarray(router, dtype=np.float32)
    gate = np.ascontiguousarray(gate).view(np.uint8).reshape(-1)
    up = np.ascontiguousarray(up).view(np.uint8).reshape(-1)
    down = np.ascontiguousarray(down).view(np.uint8).reshape(-1)
    y = np.empty(hidden, dtype=np.float64)
    bound = np.empty(hidden, dtype=np.float64)
    tie = np.empty(hidden, dtype=np.float64)
    sel = np.empty(top_k, dtype=np.int32)
    w = np.empty(top_k, dtype=np.float64)
    _check(_load().qref_moe_ffn_q8act(_ptr(x), _ptr(residual), _ptr(router), gate_fmt, _ptr(gate),
                                      up_fmt, _ptr(up), down_fmt, _ptr(down), hidden, n_experts,
                                      top_k, expert_dim, float(tie_window), _ptr(y), _ptr(bound),
                                      _ptr(tie), _ptr(sel), _ptr(w)), "moe_ffn_q8act")
    return dict(y=y, bound=bound, tie=tie, sel=sel, w=w)
