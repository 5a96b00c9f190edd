"""Pins of the output certificate (oracle/bound.py, certificate) that do not retype it.

"Runtime-Certified Bounded-Error Quantized Attention", Methodology section 2: the
attention error splits into a key term (total-variation distance between exact and
approximate softmax, bounded through the per-token score perturbation Delta) and a
value term (per-block reconstruction errors weighted by the blocks' attention mass).

Besides a hand-computed golden, each test builds an attention instance by hand in
which the error actually reaches the certificate (the worst case the tracked
quantities allow) and computes that error by brute force (explicit softmax and
weighted sums in fp64 over explicit key/value vectors).  The certificate must
bound it (E >= err) and be attained (E <= err (1 + 1e-12)): a dropped factor, a
looser total-variation bound, a maximum over flagged blocks or a value error summed
over flagged blocks each break one of the two.
"""
import math
import os

import numpy as np
import pytest

from oracle import bound

HERE = os.path.dirname(os.path.abspath(__file__))
D = 128


def _q_bits():
    q = np.zeros((1, 1, D), dtype=np.float16)
    q[0, 0, 0] = 2.0  # ||q|| = 2; with sigma = 0.5 every unit of key error moves a logit by 1
    return q.view(np.uint16)


def _attend(logits, values):
    """Brute-force softmax attention of one query: sum_i softmax(l)_i v_i (fp64)."""
    l = np.asarray(logits, np.float64)
    w = np.exp(l - l.max())
    w /= w.sum()
    return w @ np.asarray(values, np.float64), w


def _cert(desc_rows, flags, mass, T):
    desc = np.asarray(desc_rows, np.float64)[None, None]
    fl = np.asarray(flags, np.uint8)[None, None]
    m = np.asarray(mass, np.float64)[None, None]
    return float(bound.certificate(desc, _q_bits(), "f16", np.array([T]), fl, m, softmax_scale=0.5)[0, 0])


def test_golden_three_blocks():
    rows, flags, mass, want = [], [], [], None
    for line in open(os.path.join(HERE, "golden", "certificate_blocks.txt")):
        if line.startswith("block"):
            _, _, ek, ev, vn, m, f = line.split()
            rows.append((float(ek), float(ev), float(vn)))
            mass.append(float(m))
            flags.append(int(f))
        elif line.startswith("expected_E"):
            want = float(line.split()[1])
    assert abs(rows[0][0] - math.log(3.0)) < 1e-15
    E = _cert(rows, flags, mass, 192)
    assert abs(E - want) <= 1e-12 * want, (E, want)


@pytest.mark.parametrize("delta", [0.05, 0.3, math.log(3.0), 2.0, 6.0])
def test_key_term_is_attained(delta):
    # Two tokens in one block.  Keys k0 = 0, k1 = delta e0 give logits (0, delta) with
    # q = 2 e0 and sigma = 0.5; the quantized keys k0 + delta e0, k1 - delta e0 (error
    # norm ek = delta each, along q) move them to (delta, 0): the largest total-variation
    # change, since p(token 0) = 1 / (1 + e^delta).  Values +vn u and -vn u are exact.
    vn = 3.0
    u = np.zeros(D)
    u[5] = 1.0
    q = 2.0 * np.eye(D)[0]
    k = np.stack([np.zeros(D), delta * np.eye(D)[0]])
    kh = k + np.stack([delta * np.eye(D)[0], -delta * np.eye(D)[0]])
    v = np.stack([vn * u, -vn * u])
    o, _ = _attend(0.5 * k @ q, v)
    oh, ph = _attend(0.5 * kh @ q, v)
    err = np.linalg.norm(o - oh)
    ek = np.linalg.norm(k - kh, axis=1).max()
    E = _cert([(ek, 0.0, vn)], [0], [ph.sum()], 2)
    assert err <= E * (1 + 1e-12)
    assert E <= err * (1 + 1e-12), (E, err)


def test_value_term_is_attained_and_skips_flagged_blocks():
    # Three blocks of 64 identical tokens; keys exact in blocks 0 and 1 (ek = 0), block 2
    # flagged with large ek and ev: it is recomputed exactly, so neither may enter.
    # Value errors of the unflagged blocks point the same way, so they add up in full.
    T = 192
    u = np.zeros(D)
    u[7] = 1.0
    logits = np.repeat([0.0, 1.0, 0.5], 64)
    vals = np.repeat(np.stack([np.eye(D)[1] * 2.0, -np.eye(D)[2] * 1.5, np.eye(D)[3] * 4.0]), 64, axis=0)
    ev = [0.25, 0.625, 2.0]
    vh = vals.copy()
    vh[:64] -= ev[0] * u
    vh[64:128] -= ev[1] * u
    o, p = _attend(logits, vals)
    oh, ph = _attend(logits, vh)  # block 2 exact in the pass
    err = np.linalg.norm(o - oh)
    mass = [ph[:64].sum(), ph[64:128].sum(), ph[128:].sum()]
    vn = [2.0, 1.5, 4.0]
    E = _cert([(0.0, ev[0], vn[0]), (0.0, ev[1], vn[1]), (5.0, ev[2], vn[2])], [0, 0, 1], mass, T)
    assert err <= E * (1 + 1e-12)
    assert E <= err * (1 + 1e-12), (E, err)


@pytest.mark.parametrize("delta,ev", [(0.2, 0.05), (math.log(3.0), 0.5), (1.5, 2.0)])
def test_both_terms_are_attained(delta, ev):
    # Two blocks of 64 tokens: block 0 keys 0 -> quantized delta e0, values +vn u; block 1
    # keys delta e0 -> quantized 0, values -vn u; every value error is +ev u.  The key part
    # of o - o_hat and the value part then point the same way: |o - o_hat| = E exactly.
    vn = 2.5
    u = np.zeros(D)
    u[9] = 1.0
    q = 2.0 * np.eye(D)[0]
    k = np.concatenate([np.zeros((64, D)), np.tile(delta * np.eye(D)[0], (64, 1))])
    kh = np.concatenate([np.tile(delta * np.eye(D)[0], (64, 1)), np.zeros((64, D))])
    v = np.concatenate([np.tile(vn * u, (64, 1)), np.tile(-vn * u, (64, 1))])
    vh = v + ev * u
    o, _ = _attend(0.5 * k @ q, v)
    oh, ph = _attend(0.5 * kh @ q, vh)
    err = np.linalg.norm(o - oh)
    ek = np.linalg.norm(k - kh, axis=1)
    E = _cert([(ek[:64].max(), ev, vn), (ek[64:].max(), ev, vn)], [0, 0], [ph[:64].sum(), ph[64:].sum()], 128)
    assert err <= E * (1 + 1e-12)
    assert E <= err * (1 + 1e-12), (E, err)


def test_value_promoted_block_counts_in_the_key_term_only():
    # Blocks (ek, ev, vn, mass, flag): block 1 is value-promoted (flag 2), block 2 exact
    # (flag 1).  With ||q|| sigma = 1 the key term takes ek over the blocks whose keys are
    # quantized, blocks 0 and 1: Delta* = max(0.5, ln 3) = ln 3, and 2 tanh(ln 3 / 2) = 1,
    # so the key term is max vn = 4.  The value sum takes block 0 only: 0.5 * 0.25.
    # E = 4 + 0.125.  Dropping block 1 from Delta* gives 2 tanh(0.25) 4 + 0.125 = 2.0747...;
    # counting its value error gives 4 + 0.125 + 0.25 * 10 = 6.625.
    rows = [(0.5, 0.25, 1.0), (math.log(3.0), 10.0, 2.0), (5.0, 10.0, 4.0)]
    E = _cert(rows, [0, 2, 1], [0.5, 0.25, 0.25], 192)
    assert abs(E - 4.125) <= 1e-12 * 4.125, E
    # bit 0 takes precedence: flag 3 is a fully exact block
    assert _cert(rows, [0, 2, 3], [0.5, 0.25, 0.25], 192) == E
