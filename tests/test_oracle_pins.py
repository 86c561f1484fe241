"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test names what fixes the expected value: an IEEE table or library
conversion, a hand-worked block from the golden file, a placement map built
from the kernels' loop structure (a different formulation from the oracle's
per-element index formulas), exact rational arithmetic, or an invariant of
the mathematics.  All run on the CPU.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import F32, Q4_0, Q8_0, Q4_K, Q5_K, Q6_K

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_blocks.txt")
BLOCK_BYTES = {Q8_0: 34, Q4_0: 18, Q4_K: 144, Q5_K: 176, Q6_K: 210}
BLOCK_ELEMS = {Q8_0: 32, Q4_0: 32, Q4_K: 256, Q5_K: 256, Q6_K: 256}


# ---------------------------------------------------------------- f16 (P1)

def test_f16_exhaustive_matches_numpy_conversion():
    """All 65,536 bit patterns against numpy's binary16 -> binary64 cast."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16(int(b)) for b in bits], dtype=np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # the sign of zero survives too
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


@pytest.mark.parametrize("bits,value", [
    (0x3C00, 1.0), (0x3800, 0.5), (0xC000, -2.0), (0x7BFF, 65504.0),
    (0x0001, 2.0 ** -24), (0x0400, 2.0 ** -14), (0x03FF, 1023 * 2.0 ** -24),
    (0x7C00, np.inf), (0xFC00, -np.inf), (0x0000, 0.0), (0x8000, -0.0),
])
def test_f16_ieee_table(bits, value):
    assert oracle.f16(bits) == value


def test_f16_nan_patterns():
    for b in (0x7E00, 0x7C01, 0xFE00, 0xFFFF):
        assert np.isnan(oracle.f16(b))


# ------------------------------------------------- hand-worked blocks (P2)

def _parse_hex(spec: str) -> bytes:
    out = bytearray()
    for piece in spec.split():
        if "x" in piece:
            n, byte = piece.split("x")
            out += bytes([int(byte, 16)]) * int(n)
        else:
            out += bytes.fromhex(piece)
    return bytes(out)


def _load_golden():
    stanzas, cur = [], {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if line.startswith("#"):
                continue
            if not line:
                if cur:
                    stanzas.append(cur)
                    cur = {}
                continue
            k, v = line.split("=", 1)
            cur[k.strip()] = v.strip()
    if cur:
        stanzas.append(cur)
    return stanzas


GOLDEN_STANZAS = _load_golden()


def test_golden_file_has_every_format():
    assert {int(s["fmt"]) for s in GOLDEN_STANZAS} == {Q8_0, Q4_0, Q4_K, Q5_K, Q6_K}


@pytest.mark.parametrize("st", GOLDEN_STANZAS, ids=[s["name"] for s in GOLDEN_STANZAS])
def test_hand_worked_block(st):
    fmt = int(st["fmt"])
    blk = _parse_hex(st["hex"])
    assert len(blk) == BLOCK_BYTES[fmt], st["name"]
    v = oracle.dequant_block(fmt, blk)
    assert v.sum() == float(st["sum1"])
    if "sumi" in st:
        assert (v * np.arange(v.size)).sum() == float(st["sumi"])
    listed = set()
    for pair in st.get("elems", "").split():
        i, val = pair.split("=")
        assert v[int(i)] == float(val), (st["name"], i)
        listed.add(int(i))
    if "rest" in st:
        rest = [v[i] for i in range(v.size) if i not in listed]
        assert all(r == float(st["rest"]) for r in rest)


# ---------------------------------------------- placement maps (P2, exhaustive)
#
# The maps below enumerate the page kernels' loop nests (outer sub-block or
# half, inner l) to list, for every element, where its bits live.  The
# oracle instead computes each element's location from a closed-form index
# formula; the two must agree for every element.

def _q4k_like_map():
    """element -> (qs byte index within qs, use_high_nibble, qh bit)."""
    m = {}
    for oi in range(4):              # pairs of 32-element sub-blocks
        for l in range(32):
            m[64 * oi + l] = (32 * oi + l, False, 2 * oi)
            m[64 * oi + 32 + l] = (32 * oi + l, True, 2 * oi + 1)
    return m


def _q6k_map():
    """element -> (ql index, high nibble?, qh index, qh shift, scale index)."""
    m = {}
    for half in range(2):
        for l in range(32):
            base = 128 * half
            ql0, qh0, sc0 = 64 * half, 32 * half, 8 * half
            m[base + l] = (ql0 + l, False, qh0 + l, 0, sc0 + l // 16)
            m[base + 32 + l] = (ql0 + l + 32, False, qh0 + l, 2, sc0 + l // 16 + 2)
            m[base + 64 + l] = (ql0 + l, True, qh0 + l, 4, sc0 + l // 16 + 4)
            m[base + 96 + l] = (ql0 + l + 32, True, qh0 + l, 6, sc0 + l // 16 + 6)
    return m


def _ones_scale_bytes():
    # every 6-bit scale 1 and every min 0 (see HW4 in the golden file)
    return bytes([1, 1, 1, 1, 0, 0, 0, 0, 1, 1, 1, 1])


def test_placement_q8_0():
    for e in range(32):
        q = bytearray(32)
        q[e] = 5
        v = oracle.dequant_block(Q8_0, bytes.fromhex("003c") + bytes(q))
        want = np.zeros(32)
        want[e] = 5
        assert np.array_equal(v, want), e


def test_placement_q4_0():
    for e in range(32):
        qs = bytearray([0x88] * 16)          # nibble 8 decodes to 0
        j = e % 16
        if e < 16:
            qs[j] = (qs[j] & 0xF0) | 13
        else:
            qs[j] = (qs[j] & 0x0F) | (13 << 4)
        v = oracle.dequant_block(Q4_0, bytes.fromhex("003c") + bytes(qs))
        want = np.zeros(32)
        want[e] = 5
        assert np.array_equal(v, want), e


def test_placement_q4_k():
    mp = _q4k_like_map()
    assert sorted(mp) == list(range(256))
    for e in range(256):
        qs = bytearray(128)
        idx, hi, _ = mp[e]
        qs[idx] = (7 << 4) if hi else 7
        blk = bytes.fromhex("003c0000") + _ones_scale_bytes() + bytes(qs)
        v = oracle.dequant_block(Q4_K, blk)
        want = np.zeros(256)
        want[e] = 7
        assert np.array_equal(v, want), e


def test_placement_q5_k():
    mp = _q4k_like_map()
    for e in range(256):
        qs = bytearray(128)
        qh = bytearray(32)
        idx, hi, bit = mp[e]
        qs[idx] = (3 << 4) if hi else 3
        qh[idx % 32] |= 1 << bit
        blk = bytes.fromhex("003c0000") + _ones_scale_bytes() + bytes(qh) + bytes(qs)
        v = oracle.dequant_block(Q5_K, blk)
        want = np.zeros(256)
        want[e] = 19
        assert np.array_equal(v, want), e


def test_placement_q6_k():
    mp = _q6k_map()
    assert sorted(mp) == list(range(256))
    for e in range(256):
        ql = bytearray(128)
        qh = bytearray([0xAA] * 64)          # top bits 2 everywhere: q = 32 -> 0
        qli, hi, qhi, sh, sci = mp[e]
        ql[qli] |= (5 << 4) if hi else 5
        qh[qhi] |= 3 << sh                    # top bits 3
        sc = bytearray([1] * 16)
        sc[sci] = 2
        blk = bytes(ql) + bytes(qh) + bytes(sc) + bytes.fromhex("003c")
        v = oracle.dequant_block(Q6_K, blk)
        want = np.zeros(256)
        want[e] = 2 * (5 + 48 - 32)
        assert np.array_equal(v, want), e


def test_q6_k_scale_groups_are_16_wide_and_signed():
    # scale j governs elements 16j..16j+15; negative scales stay negative
    for j in range(16):
        sc = bytearray([0] * 16)
        sc[j] = 0x80                              # -128
        blk = bytes(128) + bytes(64) + bytes(sc) + bytes.fromhex("003c")
        v = oracle.dequant_block(Q6_K, blk)
        want = np.zeros(256)
        want[16 * j:16 * j + 16] = -128 * -32
        assert np.array_equal(v, want), j


# ---------------------------------------- structural round trips (P2)

def _pack_kquant_scales(sc, m):
    """Test-side packer of eight 6-bit scales and mins into 12 bytes."""
    S = [0] * 12
    for s in range(4):
        S[s] = (sc[s] & 63) | ((sc[s + 4] >> 4) << 6)
        S[s + 4] = (m[s] & 63) | ((m[s + 4] >> 4) << 6)
        S[s + 8] = (sc[s + 4] & 15) | ((m[s + 4] & 15) << 4)
    return bytes(S)


def test_kquant_scale_packing_is_a_bijection():
    """unpack(pack(f)) == f for every value of every field, and 12 random
    bytes always unpack to sixteen 6-bit values that pack back to them."""
    for s in range(8):
        for val in range(64):
            sc = [0] * 8
            m = [0] * 8
            sc[s] = val
            blk = (bytes.fromhex("003c0000") + _pack_kquant_scales(sc, m)
                   + bytes([0x11] * 128))       # q = 1 everywhere
            v = oracle.dequant_block(Q4_K, blk)
            want = np.zeros(256)
            want[32 * s:32 * s + 32] = val
            assert np.array_equal(v, want), (s, val)
            sc[s] = 0
            m[s] = val                           # dmin = 1 below
            blk = (bytes.fromhex("003c003c") + _pack_kquant_scales(sc, m) + bytes(128))
            v = oracle.dequant_block(Q4_K, blk)
            want = np.zeros(256)
            want[32 * s:32 * s + 32] = -val
            assert np.array_equal(v, want), (s, val)


@pytest.mark.parametrize("fmt", [Q4_K, Q5_K])
def test_kquant_random_fields_round_trip(fmt):
    """Random fields -> bytes (test-side packer) -> oracle == d*sc*q - dmin*m."""
    g = np.random.default_rng(7)
    mp = _q4k_like_map()
    for _ in range(40):
        d = np.float16(g.uniform(-2, 2))
        dmin = np.float16(g.uniform(-2, 2))
        sc = g.integers(0, 64, 8)
        m = g.integers(0, 64, 8)
        q = g.integers(0, 32 if fmt == Q5_K else 16, 256)
        qs = bytearray(128)
        qh = bytearray(32)
        for e in range(256):
            idx, hi, bit = mp[e]
            qs[idx] |= (int(q[e]) & 15) << (4 if hi else 0)
            if q[e] >= 16:
                qh[idx % 32] |= 1 << bit
        head = d.tobytes() + dmin.tobytes() + _pack_kquant_scales(sc, m)
        blk = head + (bytes(qh) if fmt == Q5_K else b"") + bytes(qs)
        v = oracle.dequant_block(fmt, blk)
        s = np.arange(256) // 32
        want = float(d) * sc[s] * q - float(dmin) * m[s]
        assert np.array_equal(v, want)


def test_q6_k_random_fields_round_trip():
    g = np.random.default_rng(8)
    mp = _q6k_map()
    for _ in range(40):
        d = np.float16(g.uniform(-2, 2))
        sc = g.integers(-128, 128, 16)
        q = g.integers(0, 64, 256)
        ql = bytearray(128)
        qh = bytearray(64)
        for e in range(256):
            qli, hi, qhi, sh, _ = mp[e]
            ql[qli] |= (int(q[e]) & 15) << (4 if hi else 0)
            qh[qhi] |= (int(q[e]) >> 4) << sh
        blk = bytes(ql) + bytes(qh) + sc.astype(np.int8).tobytes() + d.tobytes()
        v = oracle.dequant_block(Q6_K, blk)
        want = float(d) * sc[np.arange(256) // 16] * (q - 32)
        assert np.array_equal(v, want)


def _maxabs_q8_0(x):
    """Test-side max-abs Q8_0 quantiser: d = max|x| / 127, q = round(x/d)."""
    amax = np.abs(x).max()
    d = np.float16(amax / 127)
    q = np.clip(np.rint(x / np.float64(d)), -127, 127).astype(np.int8)
    return d.tobytes() + q.tobytes()


def _maxabs_q4_0(x):
    """Test-side Q4_0 quantiser: d = (signed value of largest magnitude) / -8,
    q = round(x/d) + 8 clamped to 0..15."""
    i = np.argmax(np.abs(x))
    d = np.float16(x[i] / -8)
    q = np.clip(np.rint(x / np.float64(d)) + 8, 0, 15).astype(np.uint8)
    packed = (q[:16] | (q[16:] << 4)).astype(np.uint8)
    return d.tobytes() + packed.tobytes()


def test_q8_0_dequant_of_quant_round_trips_exact_inputs():
    g = np.random.default_rng(9)
    for _ in range(50):
        q = g.integers(-127, 128, 32)
        q[g.integers(0, 32)] = 127 * (1 if g.random() < 0.5 else -1)
        x = q * 2.0 ** -7
        v = oracle.dequant_block(Q8_0, _maxabs_q8_0(x))
        assert np.array_equal(v, x)


def test_q4_0_dequant_of_quant_round_trips_exact_inputs():
    g = np.random.default_rng(10)
    for _ in range(50):
        q = g.integers(1, 16, 32)
        q[g.integers(0, 32)] = 0               # -8 is the largest magnitude
        x = (q - 8) * 2.0 ** -4
        v = oracle.dequant_block(Q4_0, _maxabs_q4_0(x))
        assert np.array_equal(v, x)


def test_special_scales_and_codes():
    # q = -128 is a legal Q8_0 code even though the workloads draw [-127, 127]
    v = oracle.dequant_block(Q8_0, bytes.fromhex("003c") + bytes([0x80]) + bytes(31))
    assert v[0] == -128 and not v[1:].any()
    # NaN scale: every element NaN; infinite scale times a zero code is NaN
    v = oracle.dequant_block(Q8_0, bytes.fromhex("007e") + bytes(32))
    assert np.isnan(v).all()
    v = oracle.dequant_block(Q8_0, bytes.fromhex("007c") + bytes([1]) + bytes(31))
    assert v[0] == np.inf and np.isnan(v[1:]).all()
    # subnormal scale
    v = oracle.dequant_block(Q8_0, bytes.fromhex("0100") + bytes([3]) + bytes(31))
    assert v[0] == 3 * 2.0 ** -24
    # negative f16 scale
    v = oracle.dequant_block(Q4_0, bytes.fromhex("00bc") + bytes([0x0F]) + bytes([0x88] * 15))
    assert v[0] == -7 and v[16] == 8 and not v[1:16].any()


# -------------------------------------------------- f64 dot products (P3)

FORMATS = [Q8_0, Q4_0, Q4_K, Q5_K, Q6_K]


def _random_matrix(fmt, rows, cols, seed):
    import synth
    return synth.matrix(synth.rng(seed), fmt, rows, cols)


@pytest.mark.parametrize("fmt", FORMATS)
def test_gemv_matches_exact_rational_sum(fmt):
    rows, cols = 3, 512
    W = _random_matrix(fmt, rows, cols, 11 + fmt)
    x = np.random.default_rng(12).standard_normal((2, cols)).astype(np.float32)
    Y, A = oracle.gemv(fmt, W, rows, cols, x)
    n = cols
    gamma = n * 2.0 ** -53 / (1 - n * 2.0 ** -53)
    for r in range(rows):
        w = oracle.dequant_row(fmt, W[r], cols)
        for b in range(2):
            exact = sum(Fraction(float(w[c])) * Fraction(float(x[b, c])) for c in range(cols))
            eabs = sum(abs(Fraction(float(w[c])) * Fraction(float(x[b, c]))) for c in range(cols))
            assert abs(Fraction(Y[b, r]) - exact) <= Fraction(gamma) * eabs
            assert abs(Fraction(A[b, r]) - eabs) <= Fraction(gamma) * eabs


def test_f32_rows_are_plain_floats():
    W = np.random.default_rng(3).standard_normal((4, 64)).astype(np.float32)
    x = np.random.default_rng(4).standard_normal((1, 64)).astype(np.float32)
    Y, _ = oracle.gemv(F32, W, 4, 64, x)
    exact = [sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(W[r], x[0]))
             for r in range(4)]
    for r in range(4):
        assert abs(Fraction(Y[0, r]) - exact[r]) <= Fraction(1, 10 ** 12)


# --------------------------------------------------- GEMV invariants (P4)

@pytest.mark.parametrize("fmt", FORMATS)
def test_one_hot_x_extracts_a_column_exactly(fmt):
    rows, cols = 4, 512
    W = _random_matrix(fmt, rows, cols, 20 + fmt)
    D = oracle.dequant_matrix(fmt, W, rows, cols)
    for j in (0, 1, 31, 32, 255, 256, 300, 511):
        x = np.zeros((1, cols), dtype=np.float32)
        x[0, j] = 1.0
        Y, _ = oracle.gemv(fmt, W, rows, cols, x)
        assert np.array_equal(Y[0], D[:, j])


@pytest.mark.parametrize("fmt", FORMATS)
def test_linearity_in_x(fmt):
    rows, cols = 4, 256
    W = _random_matrix(fmt, rows, cols, 30 + fmt)
    g = np.random.default_rng(31)
    # small integers: every sum below is exact in f32 and in f64
    x1 = g.integers(-8, 9, (1, cols)).astype(np.float32)
    x2 = g.integers(-8, 9, (1, cols)).astype(np.float32)
    a, b = 2.0, -0.5
    Y1, _ = oracle.gemv(fmt, W, rows, cols, x1)
    Y2, _ = oracle.gemv(fmt, W, rows, cols, x2)
    Y3, A3 = oracle.gemv(fmt, W, rows, cols, (a * x1 + b * x2).astype(np.float32))
    lhs = Y3[0]
    rhs = a * Y1[0] + b * Y2[0]
    assert np.all(np.abs(lhs - rhs) <= 1e-14 * (A3[0] + 1))


@pytest.mark.parametrize("fmt", FORMATS)
def test_batch_columns_equal_single_runs(fmt):
    rows, cols = 5, 512
    W = _random_matrix(fmt, rows, cols, 40 + fmt)
    X = np.random.default_rng(41).standard_normal((8, cols)).astype(np.float32)
    Y, A = oracle.gemv(fmt, W, rows, cols, X)
    for b in range(8):
        y1, a1 = oracle.gemv(fmt, W, rows, cols, X[b:b + 1])
        assert np.array_equal(Y[b], y1[0]) and np.array_equal(A[b], a1[0])


def test_all_ones_x_gives_hand_worked_row_sums():
    # a row made of the HW3 block twice: sum 2 * 1344
    blk = _parse_hex([s for s in GOLDEN_STANZAS if s["name"] == "HW3_q4_k"][0]["hex"])
    W = np.frombuffer(blk * 2, dtype=np.uint8).reshape(1, -1)
    Y, _ = oracle.gemv(Q4_K, W, 1, 512, np.ones((1, 512), dtype=np.float32))
    assert Y[0, 0] == 2688


def test_sampled_rows_equal_full_gemv():
    W = _random_matrix(Q6_K, 9, 512, 50)
    x = np.random.default_rng(51).standard_normal((2, 512)).astype(np.float32)
    Y, A = oracle.gemv(Q6_K, W, 9, 512, x)
    idx = np.array([8, 0, 3])
    Ys, As = oracle.gemv(Q6_K, W, 9, 512, x, row_idx=idx)
    assert np.array_equal(Ys, Y[:, idx]) and np.array_equal(As, A[:, idx])


def test_row_bytes_and_argument_errors():
    assert oracle.row_bytes(Q4_K, 4096) == 16 * 144
    assert oracle.row_bytes(Q6_K, 768) == 3 * 210
    assert oracle.row_bytes(Q8_0, 1024) == 32 * 34
    assert oracle.row_bytes(Q4_0, 14336) == 448 * 18
    assert oracle.row_bytes(Q5_K, 4096) == 16 * 176
    assert oracle.row_bytes(Q4_K, 100) == -1
    assert oracle.row_bytes(99, 256) == -1
    with pytest.raises(ValueError):
        oracle.gemv(Q4_K, np.zeros(144, np.uint8), 1, 255, np.zeros((1, 255), np.float32))


# ------------------------------------------------------- routing (P5)

def _brute_rank_topk(logits, k):
    """O(E^2) rank: expert i's rank is the number of experts that beat it
    (a larger logit, or an equal logit at a lower index)."""
    E = len(logits)
    rank = [sum(1 for j in range(E) if logits[j] > logits[i] or
                (logits[j] == logits[i] and j < i)) for i in range(E)]
    order = sorted(range(E), key=lambda i: rank[i])
    return order[:k]


def test_route_matches_brute_force_rank_random():
    g = np.random.default_rng(60)
    for _ in range(200):
        E = int(g.integers(1, 130))
        k = int(g.integers(1, E + 1))
        lg = g.standard_normal(E) * 3
        sel, w = oracle.route(lg, k)
        assert list(sel) == _brute_rank_topk(list(lg), k)


def test_route_exhaustive_ties():
    """Every vector in {0,1,2}^6 and every k: ties go to the lower index."""
    import itertools
    for vals in itertools.product([0.0, 1.0, 2.0], repeat=6):
        for k in range(1, 7):
            sel, w = oracle.route(np.array(vals), k)
            assert list(sel) == _brute_rank_topk(list(vals), k), (vals, k)


def test_route_weight_invariants():
    from scipy.special import softmax
    g = np.random.default_rng(61)
    for _ in range(100):
        E = int(g.integers(2, 129))
        k = int(g.integers(1, E + 1))
        lg = g.standard_normal(E) * 2
        sel, w = oracle.route(lg, k)
        assert abs(w.sum() - 1) <= 1e-15 * k
        assert np.all(np.diff(w) <= 0)                 # rank order = weight order
        # adding a constant to every logit changes nothing
        sel2, w2 = oracle.route(lg + 7.25, k)
        assert np.array_equal(sel, sel2) and np.allclose(w, w2, rtol=1e-13, atol=0)
        # k = E is the plain softmax (library routine), in rank order
        selE, wE = oracle.route(lg, E)
        assert np.allclose(wE, softmax(lg)[selE], rtol=1e-13, atol=0)
        # k = 1 has weight exactly 1
        sel1, w1 = oracle.route(lg, 1)
        assert w1[0] == 1.0 and sel1[0] == int(np.argmax(lg))
        # relabelling experts permutes the selection
        perm = g.permutation(E)
        lgp = np.empty(E)
        lgp[perm] = lg
        selp, wp = oracle.route(lgp, k)
        assert np.array_equal(selp, perm[sel]) or _has_tie(lg, k)
        # weights are softmax probabilities renormalised over the chosen set
        p = softmax(lg)
        assert np.allclose(w, p[sel] / p[sel].sum(), rtol=1e-13, atol=0)


def _has_tie(lg, k):
    s = np.sort(lg)[::-1]
    return k < len(s) and s[k - 1] == s[k]


def test_route_nan_ranks_last():
    lg = np.array([np.nan, 1.0, -np.inf, 0.5])
    sel, _ = oracle.route(lg, 3)
    assert list(sel) == [1, 3, 2]


def test_route_argument_errors():
    with pytest.raises(ValueError):
        oracle.route(np.zeros(4), 5)
    with pytest.raises(ValueError):
        oracle.route(np.zeros(4), 0)


# ---------------------------------------------------------- SiLU (P6)

def test_silu_identities():
    from scipy.special import expit
    assert oracle.silu(0.0) == 0.0
    g = np.random.default_rng(70).standard_normal(1000) * 10
    for v in g:
        s, t = oracle.silu(v), oracle.silu(-v)
        # silu(g) - silu(-g) = g exactly in real arithmetic
        assert abs((s - t) - v) <= 8 * np.finfo(float).eps * max(abs(v), 1)
        # against the library logistic function
        assert abs(s - v * expit(v)) <= 4 * np.finfo(float).eps * max(abs(s), 1e-300)
    for big in (40.0, 100.0, 700.0):
        assert oracle.silu(big) / big == 1.0
    assert oracle.silu(-800.0) == -0.0 or abs(oracle.silu(-800.0)) < 1e-300
