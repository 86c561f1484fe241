"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the method: it only draws random field
values and writes them at their byte offsets inside GGUF blocks.  Both the
oracle and the HIP path read the same bytes, so neither depends on how the
bytes were drawn.

Generator: numpy's PCG64 bit generator (``numpy.random.default_rng(seed)``),
a published, platform-independent generator.  Recipes follow the value
distributions of the workloads (all bounds inclusive):

* f16 scale fields: a uniform float64 draw in [lo, hi], rounded to the
  nearest f16 (ties to even) by numpy.
* Q8_0: d ~ U[1e-3, 1e-2]; q ~ U{-127..127} int8.
* Q4_0: d ~ U[1e-3, 1e-2]; every packed byte uniform (both nibbles U{0..15}).
* Q4_K: d, dmin ~ U[1e-3, 1e-2]; the 12 packed scale bytes uniform (the
  packing is a bijection onto 16 six-bit values, so this is the same as
  drawing every scale and min from U{0..63}); quant bytes uniform.
* Q5_K: as Q4_K, plus the 32 high-bit bytes uniform.
* Q6_K: ql and qh bytes uniform; sixteen scales ~ U{-64..63} int8;
  d ~ U[1e-4, 1e-3].
* F32 router: N(0, 0.02^2); activations and residual: N(0, 1), drawn in
  float64 and rounded to float32.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Tuple

import numpy as np

F32, Q4_0, Q8_0, Q4_K, Q5_K, Q6_K = 0, 2, 8, 12, 13, 14
FMT_NAMES = {F32: "F32", Q4_0: "Q4_0", Q8_0: "Q8_0", Q4_K: "Q4_K", Q5_K: "Q5_K", Q6_K: "Q6_K"}

# (elements per block, bytes per block): the GGUF block geometry.
GEOMETRY = {F32: (1, 4), Q4_0: (32, 18), Q8_0: (32, 34), Q4_K: (256, 144),
            Q5_K: (256, 176), Q6_K: (256, 210)}


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def _f16_field(g: np.random.Generator, n: int, lo: float, hi: float) -> np.ndarray:
    """n f16 values ~ U[lo, hi] as little-endian byte pairs [n][2]."""
    v = g.uniform(lo, hi, size=n).astype(np.float16)
    return v.view(np.uint8).reshape(n, 2)


def _u8(g: np.random.Generator, shape) -> np.ndarray:
    return g.integers(0, 256, size=shape, dtype=np.uint8)


def blocks(g: np.random.Generator, fmt: int, nblocks: int) -> np.ndarray:
    """nblocks random blocks of format fmt, as uint8 [nblocks][block_bytes]."""
    qk, bb = GEOMETRY[fmt]
    out = np.empty((nblocks, bb), dtype=np.uint8)
    if fmt == Q8_0:
        out[:, 0:2] = _f16_field(g, nblocks, 1e-3, 1e-2)
        out[:, 2:34] = g.integers(-127, 128, size=(nblocks, 32), dtype=np.int8).view(np.uint8)
    elif fmt == Q4_0:
        out[:, 0:2] = _f16_field(g, nblocks, 1e-3, 1e-2)
        out[:, 2:18] = _u8(g, (nblocks, 16))
    elif fmt in (Q4_K, Q5_K):
        out[:, 0:2] = _f16_field(g, nblocks, 1e-3, 1e-2)   # d
        out[:, 2:4] = _f16_field(g, nblocks, 1e-3, 1e-2)   # dmin
        out[:, 4:bb] = _u8(g, (nblocks, bb - 4))           # scales, (qh,) qs
    elif fmt == Q6_K:
        out[:, 0:192] = _u8(g, (nblocks, 192))             # ql, qh
        out[:, 192:208] = g.integers(-64, 64, size=(nblocks, 16), dtype=np.int8).view(np.uint8)
        out[:, 208:210] = _f16_field(g, nblocks, 1e-4, 1e-3)
    elif fmt == F32:
        raise ValueError("use f32_matrix for F32 weights")
    else:
        raise ValueError(f"unknown format {fmt}")
    return out


def matrix(g: np.random.Generator, fmt: int, rows: int, cols: int) -> np.ndarray:
    """A [rows][row_bytes] uint8 matrix of random blocks (row-major, no padding)."""
    qk, bb = GEOMETRY[fmt]
    assert cols % qk == 0
    nb = rows * (cols // qk)
    return blocks(g, fmt, nb).reshape(rows, (cols // qk) * bb)


def f32_matrix(g: np.random.Generator, rows: int, cols: int, std: float) -> np.ndarray:
    return (g.standard_normal((rows, cols)) * std).astype(np.float32)


def activations(g: np.random.Generator, batch: int, cols: int) -> np.ndarray:
    return g.standard_normal((batch, cols)).astype(np.float32)


# --------------------------------------------------------------------------
# The workloads, by shape.  Seeds 101..105; a second sweep uses 201..205.

@dataclass(frozen=True)
class GemvCase:
    name: str
    fmt: int
    rows: int
    cols: int
    batches: Tuple[int, ...]
    seed: int


@dataclass(frozen=True)
class MoeCase:
    name: str
    hidden: int = 2048
    n_experts: int = 128
    top_k: int = 8
    expert_dim: int = 768
    gate_fmt: int = Q4_K
    up_fmt: int = Q4_K
    down_fmt: int = Q6_K
    tokens: int = 64
    seed: int = 104


GEMV_CASES: Dict[str, GemvCase] = {
    "q8_0_256x1024": GemvCase("q8_0_256x1024", Q8_0, 256, 1024, (1,), 101),
    "q4_k_4096x4096": GemvCase("q4_k_4096x4096", Q4_K, 4096, 4096, (1,), 102),
    "q6_k_151936x2048": GemvCase("q6_k_151936x2048", Q6_K, 151936, 2048, (1,), 103),
    "q5_k_14336x4096": GemvCase("q5_k_14336x4096", Q5_K, 14336, 4096, (1, 4, 8), 105),
    "q4_0_4096x14336": GemvCase("q4_0_4096x14336", Q4_0, 4096, 14336, (1, 4, 8), 105),
}

MOE_CASE = MoeCase("qwen3_30b_a3b_moe_ffn")


def gemv_inputs(case: GemvCase, batch: int, seed_offset: int = 0):
    """(W uint8 [rows][row_bytes], X float32 [batch][cols]) for a GEMV case."""
    g = rng(case.seed + seed_offset)
    W = matrix(g, case.fmt, case.rows, case.cols)
    X = activations(g, batch, case.cols)
    return W, X


def moe_weights(case: MoeCase, seed_offset: int = 0):
    """Router F32 [E][H], gate/up stacks [E][F][row_bytes(H)], down [E][H][row_bytes(F)]."""
    g = rng(case.seed + seed_offset)
    E, H, F = case.n_experts, case.hidden, case.expert_dim
    router = f32_matrix(g, E, H, 0.02)
    gate = matrix(g, case.gate_fmt, E * F, H).reshape(E, F, -1)
    up = matrix(g, case.up_fmt, E * F, H).reshape(E, F, -1)
    down = matrix(g, case.down_fmt, E * H, F).reshape(E, H, -1)
    return router, gate, up, down


def moe_tokens(case: MoeCase, seed_offset: int = 0):
    """x [T][H] and residual [T][H], float32 N(0, 1)."""
    g = rng(case.seed + 1000 + seed_offset)
    x = activations(g, case.tokens, case.hidden)
    residual = activations(g, case.tokens, case.hidden)
    return x, residual


# Qwen3's RMSNorm epsilon; the norm step in front of the MoE router uses it.
NORM_EPS = 1e-6


def moe_norm_inputs(case: MoeCase, seed_offset: int = 0):
    """Inputs of the fused residual add + RMSNorm in front of the MoE:
    attn_out [T][H] and hidden_in [T][H] float32 N(0, 1), and the norm
    weight [H] float32 1 + N(0, 0.1^2)."""
    g = rng(case.seed + 2000 + seed_offset)
    attn = activations(g, case.tokens, case.hidden)
    hidden = activations(g, case.tokens, case.hidden)
    weight = (1.0 + 0.1 * g.standard_normal(case.hidden)).astype(np.float32)
    return attn, hidden, weight
