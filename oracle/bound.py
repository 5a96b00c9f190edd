"""Per-block error descriptors, the certified block bound, and the output certificate.

Test infrastructure only: see the package docstring for who may import it.

"Runtime-Certified Bounded-Error Quantized Attention" keeps, next to the
quantized keys and values, per-block error descriptors (Methodology section 1),
and splits the attention error into a key term (the total-variation distance
between exact and approximate softmax, bounded through the per-token score
perturbation) and a value term (per-block reconstruction errors weighted by the
attention mass of each block) (Methodology section 2).  Both are computed from
tracked quantities, without touching the fp16 originals.  The page prints no
formula; the reading taken here:

Descriptors of block b (64 tokens), computed at append time:
    ek_b = max_t ||R k_t - k_hat_t||      key reconstruction error
    ev_b = max_t ||R v_t - v_hat_t||      value reconstruction error
    vn_b = max_t ||v_t||                  value norm (original basis)
(R orthogonal, so these are also the original-basis errors.)

Block bound for kv head h, with the largest query norm of its GQA group:
    Delta_b = max_{hq in group} ||q_hq|| * sigma * ek_b   (Cauchy-Schwarz: every
              logit of block b moves by at most Delta_b)
    bound_b = Delta_b + ev_b;  block flagged for exact recompute iff bound_b > tau.

Certificate for query head hq after a pass in which flagged blocks were exact:
    Delta*  = ||q_hq|| * sigma * max_{b: keys quantized} ek_b
    E       = 2 tanh(Delta* / 2) max_b vn_b + sum_{b: values quantized} P_b ev_b
with P_b the block's softmax mass in that pass.  A flag with bit 0 makes a
block's keys and values exact; bit 1 alone makes only its values exact (value
promotion), so such a block still counts in Delta* but not in the value sum.
Why it holds:
o - o_hat = sum_i (p_i - p_hat_i) v_i + sum_i p_hat_i (v_i - v_hat_i).  The second
sum is at most sum_b P_b ev_b (flagged blocks use exact values).  In the first,
||.|| <= sum_i |p_i - p_hat_i| ||v_i|| <= 2 TV(p, p_hat) max ||v||, and with every
logit moved by some delta_i, |delta_i| <= Delta* (flagged keys exact: delta = 0), the
total-variation distance is at most tanh(Delta* / 2): for any token set A,
p_hat(A) is largest when delta = +Delta* on A and -Delta* elsewhere, which gives
p_hat(A) - p(A) = x a / (1 + (a - 1) x) - x with x = p(A), a = exp(2 Delta*),
whose maximum over x (at x = 1 / (1 + sqrt a)) is (sqrt a - 1) / (sqrt a + 1) =
tanh(Delta* / 2).  Both steps are attained (two tokens with p(A) = 1 / (1 + e^Delta*),
logits moved by +-Delta*, values +-max||v|| along one direction, value errors
along the same direction), so the certificate is the smallest bound these tracked
quantities allow.
"""

import numpy as np

from . import numerics as nx
from .codec import decode_k, decode_v, TILE
from .rotation import rotation_matrix_f64, D


def block_descriptors(cache, dtype, rotation, signs=None, r16=None, seq_len=None):
    """fp64 descriptors [B, H, nblk, 3] = (ek, ev, vn) from the fp16 originals.

    Blocks (or parts of blocks) at or beyond seq_len[b] are ignored (zero).
    """
    if not cache.keep:
        raise ValueError("descriptors need the fp16 originals")
    R = rotation_matrix_f64(rotation, signs, r16)
    nblk = cache.Tmax // TILE
    desc = np.zeros((cache.B, cache.H, nblk, 3))
    for b in range(cache.B):
        T = cache.Tmax if seq_len is None else int(seq_len[b])
        if T <= 0:
            continue
        for h in range(cache.H):
            k = nx.widen_input(cache.k_orig[b, h, :T], dtype).astype(np.float64)
            v = nx.widen_input(cache.v_orig[b, h, :T], dtype).astype(np.float64)
            ek = np.linalg.norm(k @ R.T - decode_k(cache, b, h, 0, T), axis=-1)
            ev = np.linalg.norm(v @ R.T - decode_v(cache, b, h, 0, T), axis=-1)
            vn = np.linalg.norm(v, axis=-1)
            for blk in range((T + TILE - 1) // TILE):
                sl = slice(blk * TILE, min(T, (blk + 1) * TILE))
                desc[b, h, blk] = (ek[sl].max(), ev[sl].max(), vn[sl].max())
    return desc


def error_bound(desc, q_bits, dtype, seq_len, tau, softmax_scale=None):
    """Per-block bound and flags: returns (bound fp64 [B,H,nblk], flags uint8 [B,H,nblk])."""
    B, H, nblk, _ = desc.shape
    Hq = q_bits.shape[1]
    G = Hq // H
    sigma = 1.0 / np.sqrt(D) if not softmax_scale else float(softmax_scale)
    q = nx.widen_input(q_bits, dtype).astype(np.float64)
    qn = np.linalg.norm(q, axis=-1).reshape(B, H, G).max(axis=-1)  # group max
    bound = qn[..., None] * sigma * desc[..., 0] + desc[..., 1]
    for b in range(B):
        nb = (int(seq_len[b]) + TILE - 1) // TILE
        bound[b, :, nb:] = 0.0
    flags = (bound > tau).astype(np.uint8)
    return bound, flags


def certificate(desc, q_bits, dtype, seq_len, flags, mass, softmax_scale=None):
    """Output error certificate E [B, Hq] (see module docstring)."""
    B, H, nblk, _ = desc.shape
    Hq = q_bits.shape[1]
    G = Hq // H
    sigma = 1.0 / np.sqrt(D) if not softmax_scale else float(softmax_scale)
    q = nx.widen_input(q_bits, dtype).astype(np.float64)
    E = np.zeros((B, Hq))
    for b in range(B):
        nb = (int(seq_len[b]) + TILE - 1) // TILE
        for hq in range(Hq):
            h = hq // G
            f = flags[b, h, :nb] if flags is not None else np.zeros(nb, np.uint8)
            kq = (f & 1) == 0        # keys quantized
            vq = (f & 3) == 0        # values quantized
            ekmax = desc[b, h, :nb, 0][kq].max() if kq.any() else 0.0
            dstar = np.linalg.norm(q[b, hq]) * sigma * ekmax
            vnmax = desc[b, h, :nb, 2].max() if nb else 0.0
            val = np.sum(mass[b, hq, :nb][vq] * desc[b, h, :nb, 1][vq])
            E[b, hq] = 2.0 * np.tanh(0.5 * dstar) * vnmax + val
    return E
