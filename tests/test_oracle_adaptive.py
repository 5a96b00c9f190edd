"""Pins for oracle/adaptive.py (adaptive precision of "Runtime-Certified
Bounded-Error Quantized Attention", Methodology section 3).

The block mass is pinned by closed forms (identical keys give each block its
share of the tokens; two key values give the two-level softmax), by the sum over
blocks and by zeros past the sequence; the top-K* choice by brute force over all
subsets of small block sets with exactly representable masses; the union over a
kv head's query heads and the fallback by hand-made cases.
"""
import itertools

import numpy as np
import pytest

import synth
from oracle import adaptive, codec, numerics as nx, rotation as rot


def _cache(k, v, fmt="int8", group=128, rotation="sign_fwht", signs=None, Tmax=None):
    B, H, T, _ = k.shape
    c = codec.Cache(B, H, Tmax or T, fmt, "int4", group, 32)
    codec.append(c, synth.to_bits(k, "f16"), synth.to_bits(v, "f16"), np.zeros(B, int), "f16", rotation, signs)
    return c


def test_block_mass_sums_to_one_and_is_zero_past_the_sequence():
    rng = np.random.default_rng(30)
    s = np.where(rng.integers(0, 2, 128) == 1, 1, -1)
    k = rng.standard_normal((2, 2, 320, 128))
    c = _cache(k, k, signs=s)
    q = synth.to_bits(rng.standard_normal((2, 4, 128)), "f16")
    P = adaptive.block_mass(c, q, "f16", np.array([320, 130]), "sign_fwht", s)
    assert np.allclose(P[0].sum(axis=-1), 1.0) and np.allclose(P[1].sum(axis=-1), 1.0)
    assert not P[1, :, 3:].any() and (P[1, :, :3] > 0).all()
    P0, = [adaptive.block_mass(c, q, "f16", np.array([0, 40]), "sign_fwht", s)]
    assert not P0[0].any() and np.allclose(P0[1, :, 0], 1.0) and not P0[1, :, 1:].any()


def test_block_mass_identical_keys_is_the_token_share():
    rng = np.random.default_rng(31)
    k = np.repeat(rng.standard_normal((1, 1, 1, 128)), 200, axis=2)
    c = _cache(k, rng.standard_normal((1, 1, 200, 128)), rotation="none", Tmax=256)
    q = synth.to_bits(rng.standard_normal((1, 2, 128)), "f16")
    P = adaptive.block_mass(c, q, "f16", np.array([200]), "none")
    assert np.allclose(P[0, :, :4], np.array([64, 64, 64, 8]) / 200.0, rtol=1e-13)


def test_block_mass_two_key_values_closed_form():
    # tokens of block 1 carry key a, all others key b: block 1 holds n1 e^la / (n1 e^la + n2 e^lb)
    rng = np.random.default_rng(32)
    a, b = rng.standard_normal(128), rng.standard_normal(128)
    k = np.tile(b, (1, 1, 256, 1))
    k[0, 0, 64:128] = a
    c = _cache(k, k, fmt="int4", group=32, rotation="none")
    q = synth.to_bits(rng.standard_normal((1, 1, 128)), "f16")
    P = adaptive.block_mass(c, q, "f16", np.array([256]), "none")
    qf = nx.widen_input(q, "f16").astype(np.float64)[0, 0]
    ka, kb = codec.decode_k(c, 0, 0, 64, 65)[0], codec.decode_k(c, 0, 0, 0, 1)[0]
    la, lb = ka @ qf / np.sqrt(128), kb @ qf / np.sqrt(128)
    m = max(la, lb)
    want = 64 * np.exp(la - m) / (64 * np.exp(la - m) + 192 * np.exp(lb - m))
    assert np.isclose(P[0, 0, 1], want, rtol=1e-12)
    assert np.allclose(P[0, 0, [0, 2, 3]], (1 - want) / 3, rtol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_top_blocks_is_the_smallest_covering_set(seed):
    rng = np.random.default_rng(40 + seed)
    n = int(rng.integers(1, 8))
    parts = rng.multinomial(64, rng.dirichlet(np.ones(n)))  # masses k/64: exact in fp32
    m = (parts / 64.0).astype(np.float32)
    for tau in (0.5, 0.75, 0.9, 0.995, 1.0):
        got = adaptive.top_blocks(m, n, tau)
        need = next(k for k in range(1, n + 1)
                    if any(sum(parts[list(s)]) >= tau * 64 for s in itertools.combinations(range(n), k)))
        assert len(got) == need, (parts, tau, got)
        # the k largest, equal masses by lower index
        want = sorted(range(n), key=lambda i: (-parts[i], i))[:need]
        assert got == want


def test_top_blocks_when_the_sum_falls_short_takes_all():
    m = np.array([0.3, 0.3, 0.3], np.float32)
    assert adaptive.top_blocks(m, 3, 0.995) == [0, 1, 2]


def test_select_blocks_unions_query_heads_and_keeps_bound_flags():
    mass = np.zeros((1, 4, 4), np.float32)
    mass[0, 0] = [1.0, 0, 0, 0]          # kv head 0, query head 0 -> block 0
    mass[0, 1] = [0, 0, 1.0, 0]          # kv head 0, query head 1 -> block 2
    mass[0, 2] = [0.5, 0.5, 0, 0]        # kv head 1, query head 2 -> blocks 0, 1 (tau 0.9)
    mass[0, 3] = [0, 0, 0, 1.0]          # kv head 1, query head 3 -> block 3
    fl_in = np.zeros((1, 2, 4), np.uint8)
    fl_in[0, 0, 3] = 1
    got = adaptive.select_blocks(mass, np.array([256]), 0.9, 2, fl_in)
    assert got[0].tolist() == [[1, 0, 1, 1], [1, 1, 0, 1]]
    short = adaptive.select_blocks(mass, np.array([64]), 0.9, 2)  # one block only
    assert short[0].tolist() == [[1, 0, 0, 0], [1, 0, 0, 0]]


def test_dense_fallback_replaces_rows_over_eps():
    out = np.ones((1, 3, 2))
    dense = np.full((1, 3, 2), 7.0)
    cert = np.array([[0.1, 0.5, 0.2]])
    o, c, redo = adaptive.dense_fallback(out, cert, 0.3, dense)
    assert redo.tolist() == [[False, True, False]]
    assert o[0, 1].tolist() == [7.0, 7.0] and o[0, 0].tolist() == [1.0, 1.0]
    assert c.tolist() == [[0.1, 0.0, 0.2]]


def test_top_blocks_tau_zero_and_above_one():
    # tau_cov = 0: the shortest prefix reaching 0 is one block, the largest mass (lowest
    # index among equal masses); tau_cov > 1: coverage is never reached, every block is kept
    rng = np.random.default_rng(31)
    for n in (1, 2, 7, 33):
        m = rng.random(n).astype(np.float32)
        m = (m / m.sum()).astype(np.float32)
        assert adaptive.top_blocks(m, n, 0.0) == [int(np.argmax(m))]
        assert sorted(adaptive.top_blocks(m, n, 2.0)) == list(range(n))
    tie = np.array([0.25, 0.25, 0.5, 0.5], np.float32)[::-1].copy()  # masses 0.5, 0.5, 0.25, 0.25
    assert adaptive.top_blocks(tie, 4, 0.0) == [0]
    assert adaptive.top_blocks(tie, 4, 0.75) == [0, 1]
