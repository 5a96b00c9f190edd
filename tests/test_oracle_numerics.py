"""Pins for oracle/numerics.py: number formats checked against spec points and brute force."""
import os

import numpy as np
import pytest

from oracle import numerics as nx

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


def test_e4m3_spec_points():
    for code, val in _rows("e4m3_points.txt"):
        got = nx.e4m3_value(int(code, 16))
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val), code


def test_e4m3_table_shape():
    t = nx.e4m3_table()
    assert np.isnan(t).sum() == 2  # 0x7F and 0xFF
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)  # codes 0x00..0x7E increase
    assert pos.max() == 448.0
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])


def test_e4m3_encode_brute_force():
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.uniform(0, 500, 4000), 2.0 ** rng.uniform(-14, 9, 4000),
                        nx.e4m3_table()[:0x7F],  # exact points
                        (nx.e4m3_table()[:0x7E] + nx.e4m3_table()[1:0x7F]) / 2])  # exact ties
    codes = nx.e4m3_encode_nonneg(v)
    table = nx.e4m3_table()[:0x7F]
    for x, c in zip(v, codes):
        if x >= 448:
            assert c == 0x7E
            continue
        d = np.abs(table - x)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert c == want, (x, c, want)


def test_e2m1_values():
    for code, val in _rows("e2m1_values.txt"):
        assert nx.e2m1_value(int(code, 16)) == float(val)
    assert list(nx.E2M1_MAG) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_e2m1_quantize_brute_force():
    rng = np.random.default_rng(8)
    s = np.float64(2.0 ** -3 * 1.375)
    y = np.concatenate([rng.uniform(-8, 8, 5000) * s,
                        np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0]) * s]).astype(np.float32)
    codes = nx.e2m1_quantize(y, s)
    mags = nx.E2M1_MAG
    for x, c in zip(y, codes):
        q = abs(float(x)) / s
        d = np.abs(mags - q)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert (c & 7) == want, (x, c, want)
        assert (c >> 3) == (1 if np.signbit(x) else 0)


def test_f16_sat_is_nearest_even():
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.uniform(-6, 4, 3000),
                        [65504.0, 65519.0, 65520.0, 1e6, -1e6]]).astype(np.float32)
    h = nx.f16_sat(x)
    for xi, hi in zip(x.astype(np.float64), h):
        if abs(xi) >= 65504:
            assert float(hi) == np.copysign(65504.0, xi)
            continue
        up = float(np.nextafter(hi, np.float16(np.inf)))
        dn = float(np.nextafter(hi, np.float16(-np.inf)))
        e = abs(xi - float(hi))
        assert e <= abs(xi - up) and e <= abs(xi - dn)
        if e == abs(xi - up) or e == abs(xi - dn):  # a tie: the kept value has an even mantissa
            assert int(np.float16(hi).view(np.uint16)) & 1 == 0


def test_rne_quotient_brute_force():
    rng = np.random.default_rng(10)
    s = np.float16(0.0371).astype(np.float64)
    y = np.concatenate([rng.uniform(-8, 8, 3000) * s, (np.arange(-15, 16) + 0.5) * s]).astype(np.float32)
    c = nx.rne_quotient(y, s)
    for yi, ci in zip(y.astype(np.float64), c):
        cand = np.arange(-20, 21)
        d = np.abs(yi - cand * s)
        best = cand[d == d.min()]
        want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
        assert ci == want


def test_bf16_widen_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F], dtype=np.uint16)
    got = nx.bf16_bits_to_f32(bits)
    want = np.array([1.0, -1.0, 3.140625, 2.0 ** -133, 3.3895313892515355e38], dtype=np.float32)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("v", [0.0, 448.0, 1000.0])
def test_e4m3_saturates(v):
    assert nx.e4m3_value(nx.e4m3_encode_nonneg(np.array([v]))[0]) == min(v, 448.0)
