"""Host-side checks of the quantiser's scale arithmetic (no GPU).

The int4 quantiser forms its scale s = fp16(fl32(amax / 7)) without a divide:
q0 = fl(amax * fl(1/7)), then one correction q1 = fma(fma(-q0, 7, amax),
fl(1/7), q0).  These tests emulate that sequence exactly in binary64 (the
residual amax - 7 q0 is exact in binary32; the final fma is one rounding of
q0 + r * fl(1/7), formed in binary64 and rounded to binary32, with any result
that lands on a binary32 midpoint redone in rationals) and compare it with the
correctly rounded quotient.  The default sample covers every binade with
random and boundary significands; PALU_EXHAUSTIVE=1 walks all non-negative
finite binary32 values (about two minutes).
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest

C7 = np.float32(1.0) / np.float32(7.0)


def _rn32_exact(fr: Fraction) -> np.float32:
    """Round a non-negative rational to binary32, ties to even."""
    f = np.float32(float(fr))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    ds = [abs(Fraction(float(x)) - fr) for x in cands]
    best = min(ds)
    ties = [x for x, d in zip(cands, ds) if d == best]
    if len(ties) == 1:
        return ties[0]
    return [x for x in ties if int(np.array(x).view(np.uint32)) % 2 == 0][0]


def _on_midpoint(x64: np.ndarray) -> np.ndarray:
    f = x64.astype(np.float32)
    lo = np.where(f.astype(np.float64) <= x64, f, np.nextafter(f, np.float32(-np.inf)))
    hi = np.nextafter(lo, np.float32(np.inf))
    return (lo.astype(np.float64) + hi.astype(np.float64)) / 2 == x64


def _div7_both(a: np.ndarray):
    """(the corrected product, the correctly rounded a / 7), both binary32."""
    q0 = a * C7
    r64 = a.astype(np.float64) - q0.astype(np.float64) * 7.0
    r = r64.astype(np.float32)
    assert np.all(r.astype(np.float64) == r64), "residual not exact in binary32"
    s64 = q0.astype(np.float64) + r.astype(np.float64) * np.float64(C7)
    q1 = s64.astype(np.float32)
    ref64 = a.astype(np.float64) / 7.0
    ref = ref64.astype(np.float32)
    for i in np.nonzero(_on_midpoint(s64) | _on_midpoint(ref64))[0]:
        A, Q0 = Fraction(float(a[i])), Fraction(float(q0[i]))
        q1[i] = _rn32_exact(Q0 + (A - 7 * Q0) * Fraction(float(C7)))
        ref[i] = _rn32_exact(A / 7)
    return q1, ref


def _sample() -> np.ndarray:
    rng = np.random.default_rng(7)
    exps = np.arange(0, 255, dtype=np.uint32) << 23            # every binade, subnormals included
    mant = np.concatenate([
        rng.integers(0, 1 << 23, size=4096, dtype=np.uint32),
        np.array([0, 1, 2, 3, (1 << 23) - 1, (1 << 23) - 2, 1 << 22, (1 << 22) + 1], dtype=np.uint32),
        np.arange(0, 1 << 23, 1 << 11, dtype=np.uint32),       # a regular grid of significands
    ])
    return (exps[:, None] | mant[None, :]).ravel().view(np.float32)


def test_div7_matches_correctly_rounded_quotient():
    a = _sample()
    q1, ref = _div7_both(a)
    bad = np.nonzero(q1.view(np.uint32) != ref.view(np.uint32))[0]
    assert bad.size == 0, [(float(a[i]), float(q1[i]), float(ref[i])) for i in bad[:5]]


def test_div7_scale_examples():
    # hand values: 7 -> 1, 3.5 -> 0.5, 0 -> 0, 1 -> fl(1/7), the largest finite value
    a = np.array([7.0, 3.5, 0.0, 1.0, np.finfo(np.float32).max], dtype=np.float32)
    q1, ref = _div7_both(a)
    assert q1[0] == 1.0 and q1[1] == 0.5 and q1[2] == 0.0 and q1[3] == C7
    assert np.array_equal(q1.view(np.uint32), ref.view(np.uint32))


@pytest.mark.skipif(os.environ.get("PALU_EXHAUSTIVE") != "1", reason="set PALU_EXHAUSTIVE=1 (about two minutes)")
def test_div7_exhaustive():
    step = 1 << 24
    for start in range(0, 0x7F800000, step):
        a = np.arange(start, min(start + step, 0x7F800000), dtype=np.uint32).view(np.float32)
        q1, ref = _div7_both(a)
        assert np.array_equal(q1.view(np.uint32), ref.view(np.uint32)), hex(start)
