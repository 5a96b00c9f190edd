"""The FP4 scale search's rounding argument, checked on the CPU ("Search Your Block
Floating Point Scales!", ScaleSearch: every candidate scale's E2M1 codes and errors).

The append kernel does not compare |y| with the thresholds m * S of the definition.  It
forms the quotient x * rcp(S), refines it once with the exact residual (fma(-t, S, x), then
fma(e, r, t)) and rounds the result to the nearest E2M1 value, ties to the even code (the
hardware conversion with scale 1).  That equals the definition whenever the refined
quotient lies on the same side of every grid midpoint as the exact one.  This test emulates
those fp32 steps (products of fp32 values are exact in fp64, the residual is exact, each
step is rounded to fp32 once) with a reciprocal off by -1, 0 or +1 ulp, on values within 4
ulp of every midpoint times every E4M3 scale and on random values, and compares the codes
with the oracle's threshold rounding of the exact quotient.
"""
import numpy as np
import pytest

from oracle import numerics as nx


def _e4m3_positive():
    v = []
    for c in range(1, 0x7F):
        e, m = c >> 3, c & 7
        v.append(m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(v, np.float32)


def _refined_quotient(x, S, ulps):
    f64 = np.float64
    r = (1.0 / S.astype(f64)).astype(np.float32)
    if ulps > 0:
        r = np.nextafter(r, np.float32(np.inf))
    elif ulps < 0:
        r = np.nextafter(r, np.float32(0))
    t = (x.astype(f64) * r.astype(f64)).astype(np.float32)
    e = (x.astype(f64) - t.astype(f64) * S.astype(f64)).astype(np.float32)  # exact residual, rounded once
    return (e.astype(f64) * r.astype(f64) + t.astype(f64)).astype(np.float32)


@pytest.mark.parametrize("ulps", [-1, 0, 1])
def test_refined_quotient_rounds_like_the_thresholds(ulps):
    rng = np.random.default_rng(7)
    S_all = _e4m3_positive()
    n = 400_000
    S = S_all[rng.integers(0, len(S_all), n)]
    mids = (nx.E2M1_MAG[:-1] + nx.E2M1_MAG[1:]) / 2.0
    base = (mids[rng.integers(0, len(mids), n)] * S.astype(np.float64)).astype(np.float32)  # exact products
    k = rng.integers(-4, 5, n)
    near = base.copy()
    for step in range(4):
        near = np.where(k > step, np.nextafter(near, np.float32(np.inf)), near)
        near = np.where(k < -step, np.nextafter(near, np.float32(0)), near)
    anywhere = (rng.random(n) * 7.0 * S).astype(np.float32)
    for x in (near, anywhere):
        u = _refined_quotient(x, S, ulps)
        got = nx.e2m1_quantize(u, np.ones_like(S))
        want = nx.e2m1_quantize(x, S)
        assert np.array_equal(got, want), f"{int((got != want).sum())} codes differ"
    # the exact midpoints themselves: the refined quotient is the midpoint, and the tie goes
    # to the even code as in the definition
    u = _refined_quotient(base, S, ulps)
    assert np.array_equal(u.astype(np.float64), (base.astype(np.float64) / S.astype(np.float64)))
