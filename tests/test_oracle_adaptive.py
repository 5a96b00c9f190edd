"""Pins for oracle/adaptive.py (adaptive precision of "Runtime-Certified
Bounded-Error Quantized Attention", Methodology section 3).

The block mass is pinned by closed forms (identical keys give each block its
share of the tokens; two key values give the two-level softmax), by the sum over
blocks and by zeros past the sequence; the top-K* choice by brute force over all
subsets of small block sets with exactly representable masses; the union over a
kv head's query heads and the fallback by hand-made cases.  Rung 2 (value
promotion) and the ranking-consistency check are pinned by hand cases with
exactly representable products and scores, the inverted-pair count by the
discordant pairs of scipy's Kendall tau, and the fp16 block scores by a closed
form (constant keys per block) and by scipy's logsumexp.
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


# ---------------------------------------------------------------- rung 2 and the ranking check
def test_promote_values_hand_case():
    # kv head 0 has query heads 0, 1; kv head 1 has query heads 2, 3.  Products mass * ev
    # (fp32, exact here: powers of two): block 0 of kv head 0 reaches 0.25 through query
    # head 1 only, block 1 is already exact (bit 0) and stays 1, block 2 equals tau_v (not
    # above it), block 3 lies past the sequence.
    mass = np.zeros((1, 4, 4), np.float32)
    mass[0, 0] = [0.125, 0.5, 0.25, 0.5]
    mass[0, 1] = [0.5, 0.5, 0.25, 0.5]
    mass[0, 2] = [0.0, 0.25, 0.0, 0.0]
    mass[0, 3] = [0.0, 0.0, 0.0, 0.0]
    ev = np.zeros((1, 2, 4), np.float32)
    ev[0, 0] = [0.5, 1.0, 0.5, 1.0]
    ev[0, 1] = [1.0, 1.0, 1.0, 1.0]
    fl = np.zeros((1, 2, 4), np.uint8)
    fl[0, 0, 1] = 1
    got = adaptive.promote_values(mass, ev, np.array([192]), 0.125, 2, fl)
    assert got[0].tolist() == [[2, 1, 0, 0], [0, 2, 0, 0]]
    assert fl[0].tolist() == [[0, 1, 0, 0], [0, 0, 0, 0]]  # the input is not modified
    # threshold above every product: nothing added
    assert np.array_equal(adaptive.promote_values(mass, ev, np.array([192]), 0.5, 2, fl), fl)


def test_inverted_pairs_hand_cases():
    s = np.array([0.0, 1.0, 0.5])
    assert adaptive.inverted_pairs([0, 1, 2], s, 0.0) == 2   # (0,1) and (0,2)
    assert adaptive.inverted_pairs([0, 1, 2], s, 0.6) == 1   # only (0,1) by more than 0.6
    assert adaptive.inverted_pairs([1, 2, 0], s, 0.0) == 0   # already in decreasing order
    assert adaptive.inverted_pairs([2, 0, 1], s, 0.0) == 2   # (2,1) and (0,1)
    assert adaptive.inverted_pairs([], s, 0.0) == 0
    assert adaptive.inverted_pairs([1], s, 0.0) == 0
    # equal scores are never inverted, at any margin >= 0
    assert adaptive.inverted_pairs([0, 1], np.array([0.5, 0.5]), 0.0) == 0


@pytest.mark.parametrize("seed", range(4))
def test_inverted_pairs_is_the_discordant_count_of_kendalls_tau(seed):
    # with distinct scores and margin 0 the inverted pairs are the discordant pairs between
    # the order and the scores ranked decreasingly: D = (1 - tau) / 2 * n (n - 1) / 2
    from scipy.stats import kendalltau
    rng = np.random.default_rng(70 + seed)
    n = int(rng.integers(5, 40))
    order = list(rng.permutation(n))
    score = rng.standard_normal(n)
    pos = np.empty(n)
    pos[order] = np.arange(n)
    tau = kendalltau(pos, -score).statistic
    want = round((1.0 - tau) / 2.0 * n * (n - 1) / 2.0)
    assert adaptive.inverted_pairs(order, score, 0.0) == want


def test_block_scores_fp16_closed_form():
    # block j holds the key c_j e_0 on all its tokens and q = a e_0: its score is
    # log(n_j) + sigma a c_j with n_j its token count (the last block is partial)
    T, Tmax = 200, 256
    c = np.array([1.0, -2.0, 0.5, 3.0])
    k = np.zeros((1, 1, Tmax, 128))
    for j in range(4):
        k[0, 0, 64 * j:64 * (j + 1), 0] = c[j]
    q = np.zeros((1, 2, 128))
    q[0, 0, 0], q[0, 1, 0] = 2.0, -0.25
    s = adaptive.block_scores_fp16(synth.to_bits(k, "f16"), synth.to_bits(q, "f16"), "f16", np.array([T]))
    n = np.array([64, 64, 64, 8])
    for hq, a in enumerate((2.0, -0.25)):
        want = np.log(n) + a * c / np.sqrt(128)
        assert np.allclose(s[0, hq], want, rtol=0, atol=1e-13)
    s0 = adaptive.block_scores_fp16(synth.to_bits(k, "f16"), synth.to_bits(q, "f16"), "f16", np.array([64]))
    assert np.isneginf(s0[0, :, 1:]).all() and np.isfinite(s0[0, :, 0]).all()


def test_block_scores_fp16_matches_scipy_logsumexp():
    from scipy.special import logsumexp
    rng = np.random.default_rng(71)
    kb = synth.to_bits(rng.standard_normal((2, 2, 192, 128)), "bf16")
    qb = synth.to_bits(rng.standard_normal((2, 4, 128)), "bf16")
    seq = np.array([192, 100])
    s = adaptive.block_scores_fp16(kb, qb, "bf16", seq, softmax_scale=0.3)
    k = nx.widen_input(kb, "bf16").astype(np.float64)
    q = nx.widen_input(qb, "bf16").astype(np.float64)
    for b in range(2):
        for hq in range(4):
            lg = 0.3 * k[b, hq // 2, :seq[b]] @ q[b, hq]
            for j in range((seq[b] + 63) // 64):
                assert abs(s[b, hq, j] - logsumexp(lg[64 * j:64 * (j + 1)])) < 1e-12


def test_ranking_inversions_hand_case():
    # one query head, four blocks; the masses rank them 2, 0, 3, 1
    mass = np.array([[[0.25, 0.0625, 0.5, 0.1875]]], np.float32)  # order 2, 0, 3, 1
    score = np.array([[[1.0, 9.0, 2.0, 1.5]]])
    seq = np.array([256])
    # tau_cov 0.9: 0.5, 0.75, 0.9375 -> K* = 3, promoted in order [2, 0, 3]
    # pairs: (2,0): 1.0 > 2.0? no; (2,3): 1.5 > 2.0? no; (0,3): 1.5 > 1.0: yes -> 1
    lo, hi = adaptive.ranking_inversions(mass, score, seq, 0.9, 0.0)
    assert lo.tolist() == hi.tolist() == [[1]]
    # margin 0.5: 1.5 > 1.0 + 0.5 is false -> 0; window 0.01 around it: lo 0, hi 1
    lo, hi = adaptive.ranking_inversions(mass, score, seq, 0.9, 0.5)
    assert lo.tolist() == hi.tolist() == [[0]]
    lo, hi = adaptive.ranking_inversions(mass, score, seq, 0.9, 0.5, window=0.01)
    assert (lo.tolist(), hi.tolist()) == ([[0]], [[1]])
    # tau_cov 1.0 promotes block 1 as well, ranked last: it scores above all three -> 3 more
    lo, _ = adaptive.ranking_inversions(mass, score, seq, 1.0, 0.0)
    assert lo.tolist() == [[4]]
    # an empty sequence has no promoted blocks
    lo, hi = adaptive.ranking_inversions(mass, score, np.array([0]), 1.0, 0.0)
    assert lo.tolist() == hi.tolist() == [[0]]


def test_dense_fallback_takes_failed_heads_too():
    out = np.ones((1, 3, 2))
    dense = np.full((1, 3, 2), 7.0)
    cert = np.array([[0.1, 0.5, 0.2]])
    fail = np.array([[1, 0, 0]], np.uint8)
    o, c, redo = adaptive.dense_fallback(out, cert, 0.3, dense, fail)
    assert redo.tolist() == [[True, True, False]]
    assert o[0, 0].tolist() == [7.0, 7.0] and o[0, 2].tolist() == [1.0, 1.0]
    assert c.tolist() == [[0.0, 0.0, 0.2]]


def test_select_blocks_keeps_value_bits_of_the_given_flags():
    # a value-promoted block (2) that the top-K* then promotes becomes 3; others keep theirs
    mass = np.zeros((1, 1, 3), np.float32)
    mass[0, 0] = [1.0, 0.0, 0.0]
    fl_in = np.array([[[2, 2, 1]]], np.uint8)
    got = adaptive.select_blocks(mass, np.array([192]), 0.5, 1, fl_in)
    assert got.tolist() == [[[3, 2, 1]]]
