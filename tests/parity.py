"""The comparison rule shared by every parity test.

Per output element: |y - y_ref| <= REL * sum_i |w_i x_i| + ABS, where the sum
is computed by the oracle over the dequantised weights.  A NaN agrees only
with a NaN and an infinity only with the same-signed infinity.  Integer
results (expert indices) are compared for exact equality elsewhere.
"""
from __future__ import annotations

import numpy as np

REL = 1e-4
ABS = 1e-6


def agree_mask(y, y_ref, bound, rel: float = REL, abs_: float = ABS) -> np.ndarray:
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    bound = np.asarray(bound, dtype=np.float64)
    both_nan = np.isnan(y) & np.isnan(y_ref)
    both_inf = np.isinf(y) & np.isinf(y_ref) & (np.sign(y) == np.sign(y_ref))
    with np.errstate(invalid="ignore"):
        close = np.abs(y - y_ref) <= rel * bound + abs_
    return both_nan | both_inf | close


def assert_agree(y, y_ref, bound, what: str = "", rel: float = REL, abs_: float = ABS) -> None:
    ok = agree_mask(y, y_ref, bound, rel, abs_)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        yv = np.asarray(y, dtype=np.float64)[i]
        rv = np.asarray(y_ref, dtype=np.float64)[i]
        bv = np.asarray(bound, dtype=np.float64)[i]
        raise AssertionError(
            f"{what}: {len(bad)} of {ok.size} outputs out of tolerance; first at {i}: "
            f"got {yv!r}, want {rv!r}, |diff| {abs(yv - rv)!r}, allowed {rel * bv + abs_!r}")
