"""Python binding of the gfx950 fused dequantise-and-dot library (include/qgemv.h).

Argument marshalling only: every function forwards to the C ABI of
``libqgemv.so`` under the same name, and every step of the computation runs
in its HIP kernels.  Tensors are passed as device pointers (``data_ptr()``);
PyTorch supplies the device memory and the current stream.  There is no CPU
fallback: if the library is missing, calls raise ``QGError``.

The library binds to the HIP runtime that PyTorch already loaded (both carry
the soname ``libamdhip64.so.7``), so torch's stream handles are valid here.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqgemv.so")

QG_F32, QG_Q4_0, QG_Q8_0, QG_Q4_K, QG_Q5_K, QG_Q6_K = 0, 2, 8, 12, 13, 14
FORMATS = {"F32": QG_F32, "Q4_0": QG_Q4_0, "Q8_0": QG_Q8_0, "Q4_K": QG_Q4_K,
           "Q5_K": QG_Q5_K, "Q6_K": QG_Q6_K}
QG_OK, QG_EINVAL, QG_EUNSUPPORTED, QG_ELAUNCH = 0, 1, 2, 3

# Every symbol the header declares, with its ctypes signature.
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
SIGNATURES = {
    "qg_block_elems": ([_INT], _INT),
    "qg_block_bytes": ([_INT], _INT),
    "qg_row_bytes": ([_INT, _I64], _I64),
    "qg_last_error": ([], ctypes.c_char_p),
    "qg_last_kernel": ([], ctypes.c_char_p),
    "qgemv": ([_INT, _P, _I64, _I64, _P, _P, _INT, _P], _INT),
    "qgemv_ws": ([_INT, _P, _I64, _I64, _P, _P, _INT, _P, ctypes.c_size_t, _P], _INT),
    "qgemv_ws_bytes": ([_INT, _I64, _I64, _INT], ctypes.c_size_t),
    "qgemv_q8act": ([_INT, _P, _I64, _I64, _P, _P, _P], _INT),
    "moe_ffn_workspace_bytes": ([_I64, _I64, _I64], ctypes.c_size_t),
    "moe_ffn": ([_P, _P, _P, _P, _INT, _P, _INT, _P, _INT, _P, _I64, _I64, _I64, _I64,
                 _P, _P, _P, ctypes.c_size_t, _P], _INT),
    "moe_ffn_q8act": ([_P, _P, _P, _P, _INT, _P, _INT, _P, _INT, _P, _I64, _I64, _I64, _I64,
                       _P, _P, _P, ctypes.c_size_t, _P], _INT),
    "moe_ffn_noalloc": ([_P, _P, _P, _P, _INT, _P, _INT, _P, _INT, _P, _I64, _I64, _I64, _I64,
                         _P, _P, _P], _INT),
    "qg_route_topk": ([_P, _I64, _I64, _P, _P, _P], _INT),
    "qg_stream_read": ([_P, ctypes.c_size_t, _P, _INT, _P], _INT),
    "moe_ffn_tokens_workspace_bytes": ([_I64, _I64, _I64, _I64], ctypes.c_size_t),
    "moe_ffn_tokens": ([_P, _P, _P, _P, _INT, _P, _INT, _P, _INT, _P, _I64, _I64, _I64, _I64,
                        _I64, _P, _P, _P, ctypes.c_size_t, _P], _INT),
    "moe_ffn_norm_workspace_bytes": ([_I64, _I64, _I64, _I64], ctypes.c_size_t),
    "moe_ffn_norm": ([_P, _P, _P, _P, ctypes.c_float, _P, _P, _INT, _P, _INT, _P, _INT, _P,
                      _I64, _I64, _I64, _I64, _P, _P, _P, ctypes.c_size_t, _P], _INT),
}


class QGError(RuntimeError):
    """A non-QG_OK return of the library, or the library missing."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libqgemv.so (after torch, so the HIP runtime is shared)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise QGError(-1, f"{path} is not built; run gguf_quant_dequant_amd.build.build()")
    try:
        import torch  # noqa: F401  -- loads the HIP runtime this library binds to
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, name: str) -> None:
    if rc != QG_OK:
        raise QGError(rc, f"{name}: {qg_last_error()}")


def qg_block_elems(fmt: int) -> int:
    return load_library().qg_block_elems(fmt)


def qg_block_bytes(fmt: int) -> int:
    return load_library().qg_block_bytes(fmt)


def qg_row_bytes(fmt: int, cols: int) -> int:
    return load_library().qg_row_bytes(fmt, cols)


def qg_last_error() -> str:
    return load_library().qg_last_error().decode()


def qg_last_kernel() -> str:
    """The arithmetic of the last successful qgemv / qgemv_ws / qgemv_q8act on this thread."""
    return load_library().qg_last_kernel().decode()


def qgemv(fmt: int, W, rows: int, cols: int, X, Y, batch: int, stream=None) -> None:
    """Y[b][r] = sum_c deq(W)[r][c] * X[b][c] on the GPU (see include/qgemv.h)."""
    rc = load_library().qgemv(fmt, _ptr(W), rows, cols, _ptr(X), _ptr(Y), batch,
                              _stream(stream))
    _check(rc, "qgemv")


def moe_ffn_workspace_bytes(n_experts: int, top_k: int, expert_dim: int) -> int:
    return load_library().moe_ffn_workspace_bytes(n_experts, top_k, expert_dim)


def moe_ffn(x, residual, y, router, gate_fmt: int, gate, up_fmt: int, up, down_fmt: int, down,
            hidden: int, n_experts: int, top_k: int, expert_dim: int, sel_experts=None,
            sel_weights=None, workspace=None, workspace_bytes: Optional[int] = None,
            stream=None) -> None:
    """One token through the stacked-expert MoE FFN (see include/qgemv.h)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    rc = load_library().moe_ffn(_ptr(x), _ptr(residual), _ptr(y), _ptr(router), gate_fmt,
                                _ptr(gate), up_fmt, _ptr(up), down_fmt, _ptr(down), hidden,
                                n_experts, top_k, expert_dim, _ptr(sel_experts),
                                _ptr(sel_weights), _ptr(workspace), workspace_bytes,
                                _stream(stream))
    _check(rc, "moe_ffn")


def moe_ffn_q8act(x, residual, y, router, gate_fmt: int, gate, up_fmt: int, up, down_fmt: int,
                  down, hidden: int, n_experts: int, top_k: int, expert_dim: int,
                  sel_experts=None, sel_weights=None, workspace=None,
                  workspace_bytes: Optional[int] = None, stream=None) -> None:
    """moe_ffn with the expert GEMVs on int8-quantised activations (see include/qgemv.h)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    rc = load_library().moe_ffn_q8act(_ptr(x), _ptr(residual), _ptr(y), _ptr(router), gate_fmt,
                                      _ptr(gate), up_fmt, _ptr(up), down_fmt, _ptr(down), hidden,
                                      n_experts, top_k, expert_dim, _ptr(sel_experts),
                                      _ptr(sel_weights), _ptr(workspace), workspace_bytes,
                                      _stream(stream))
    _check(rc, "moe_ffn_q8act")


def moe_ffn_noalloc(x, residual, y, router, gate_fmt: int, gate, up_fmt: int, up,
                    down_fmt: int, down, hidden: int, n_experts: int, top_k: int,
                    expert_dim: int, sel_experts=None, sel_weights=None, stream=None) -> None:
    """moe_ffn with the library's own scratch array as its workspace (see include/qgemv.h)."""
    rc = load_library().moe_ffn_noalloc(_ptr(x), _ptr(residual), _ptr(y), _ptr(router), gate_fmt,
                                        _ptr(gate), up_fmt, _ptr(up), down_fmt, _ptr(down),
                                        hidden, n_experts, top_k, expert_dim, _ptr(sel_experts),
                                        _ptr(sel_weights), _stream(stream))
    _check(rc, "moe_ffn_noalloc")


def qg_route_topk(logits, n_experts: int, top_k: int, sel_experts, sel_weights,
                  stream=None) -> None:
    """Softmax / top-k / renormalise on given f64 logits (see include/qgemv.h)."""
    rc = load_library().qg_route_topk(_ptr(logits), n_experts, top_k, _ptr(sel_experts),
                                      _ptr(sel_weights), _stream(stream))
    _check(rc, "qg_route_topk")


def moe_ffn_norm_workspace_bytes(hidden: int, n_experts: int, top_k: int,
                                 expert_dim: int) -> int:
    return load_library().moe_ffn_norm_workspace_bytes(hidden, n_experts, top_k, expert_dim)


def moe_ffn_norm(attn_out, hidden_in, hidden_out, norm_weight, eps: float, normed, router,
                 gate_fmt: int, gate, up_fmt: int, up, down_fmt: int, down, hidden: int,
                 n_experts: int, top_k: int, expert_dim: int, sel_experts=None,
                 sel_weights=None, workspace=None, workspace_bytes: Optional[int] = None,
                 stream=None) -> None:
    """The MoE FFN behind the fused residual add + RMSNorm (see include/qgemv.h)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    rc = load_library().moe_ffn_norm(_ptr(attn_out), _ptr(hidden_in), _ptr(hidden_out),
                                     _ptr(norm_weight), float(eps), _ptr(normed), _ptr(router),
                                     gate_fmt, _ptr(gate), up_fmt, _ptr(up), down_fmt, _ptr(down),
                                     hidden, n_experts, top_k, expert_dim, _ptr(sel_experts),
                                     _ptr(sel_weights), _ptr(workspace), workspace_bytes,
                                     _stream(stream))
    _check(rc, "moe_ffn_norm")


def moe_ffn_tokens_workspace_bytes(tokens: int, n_experts: int, top_k: int,
                                   expert_dim: int) -> int:
    return load_library().moe_ffn_tokens_workspace_bytes(tokens, n_experts, top_k, expert_dim)


def moe_ffn_tokens(x, residual, y, router, gate_fmt: int, gate, up_fmt: int, up, down_fmt: int,
                   down, tokens: int, hidden: int, n_experts: int, top_k: int, expert_dim: int,
                   sel_experts=None, sel_weights=None, workspace=None,
                   workspace_bytes: Optional[int] = None, stream=None) -> None:
    """T decode tokens through the stacked-expert MoE FFN (see include/qgemv.h)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    rc = load_library().moe_ffn_tokens(_ptr(x), _ptr(residual), _ptr(y), _ptr(router), gate_fmt,
                                       _ptr(gate), up_fmt, _ptr(up), down_fmt, _ptr(down), tokens,
                                       hidden, n_experts, top_k, expert_dim, _ptr(sel_experts),
                                       _ptr(sel_weights), _ptr(workspace), workspace_bytes,
                                       _stream(stream))
    _check(rc, "moe_ffn_tokens")


def qgemv_ws_bytes(fmt: int, rows: int, cols: int, batch: int) -> int:
    return load_library().qgemv_ws_bytes(fmt, rows, cols, batch)


def qgemv_ws(fmt: int, W, rows: int, cols: int, X, Y, batch: int, workspace=None,
             workspace_bytes: Optional[int] = None, stream=None) -> None:
    """qgemv with a caller-provided workspace for batch >= 2 (see include/qgemv.h)."""
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load_library().qgemv_ws(fmt, _ptr(W), rows, cols, _ptr(X), _ptr(Y), batch,
                                 _ptr(workspace), workspace_bytes, _stream(stream))
    _check(rc, "qgemv_ws")


def qgemv_q8act(fmt: int, W, rows: int, cols: int, X, Y, stream=None) -> None:
    """Y = deq(W) * X at batch 1 on int8-quantised activations (see include/qgemv.h)."""
    rc = load_library().qgemv_q8act(fmt, _ptr(W), rows, cols, _ptr(X), _ptr(Y), _stream(stream))
    _check(rc, "qgemv_q8act")


def qg_stream_read(buf, nbytes: int, out, grid: int = 0, stream=None) -> None:
    """Read nbytes of buf once (the streaming floor; see include/qgemv.h)."""
    rc = load_library().qg_stream_read(_ptr(buf), nbytes, _ptr(out), grid, _stream(stream))
    _check(rc, "qg_stream_read")
