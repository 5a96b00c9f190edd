"""Adaptive precision and the dense fallback of a head.

Test infrastructure only: see the package docstring for who may import it.

"Runtime-Certified Bounded-Error Quantized Attention", Methodology section 3
(adaptive precision and the fallback ladder):

* a light scoring pass over the quantized keys estimates the attention mass of
  every block;
* the K* blocks with the largest estimated mass that together cover a fraction
  tau_cov of it (the page's example: 99.5 %) are promoted to the full-precision
  originals; the rest stays quantized;
* values whose reconstruction error is large for their estimated contribution
  are promoted too, and a head that still cannot be certified is recomputed with
  dense attention over the originals (the page's rungs 2 and 3).

Readings taken here (the page gives no formulas):

* Blocks are 64 tokens.  The estimated mass of block b for query head hq is the
  softmax mass of its tokens under the quantized keys,
      P_b = sum_{t in b} softmax_t(sigma * q_rot . k_hat_t),
  i.e. the attention the quantized cache itself would give the block.
* Top-K*: blocks in decreasing P_b (equal masses: lower block index first); K*
  is the smallest k whose running sum of the first k masses reaches tau_cov
  (all blocks if the sum never does).  The running sum is accumulated in fp32
  in that order from the fp32 masses the scoring pass produced, so the choice
  is a deterministic function of those masses.
* Promotion granularity: the decode pass recomputes a block exactly for all
  query heads that share its kv head, so the promoted set of a (sequence, kv
  head) is the union over its query heads.  Promotion flags are a byte per
  block: bit 0 = keys and values from the originals (top-K* blocks, and the
  blocks the certified bound flags), bit 1 alone = values from the originals,
  keys still quantized (rung 2).
* Rung 2, value promotion: a block's estimated contribution to the value error
  is its estimated mass times its value reconstruction error, P_b * ev_b (the
  block's term of the certificate's value sum).  A block not already promoted
  takes its values from the originals when that product, for any query head of
  its kv head, exceeds a threshold tau_v.  The product is taken in fp32 from the
  fp32 masses and descriptors, so the choice is a deterministic function of them.
* Ranking-consistency check: for a query head, the blocks it promoted (its own
  top-K*, in selection order = the ranking by quantized-key mass) are scored
  again from the fp16 originals: the block's log-sum-exp of sigma q . k_t over
  its tokens (the log of its unnormalised attention mass; the ranking ignores
  the common normaliser).  A pair of promoted blocks is inverted when the block
  ranked lower by the quantized keys scores more than a margin delta >= 0 above
  the block ranked higher.  The head fails the check, and is recomputed with
  dense attention over the originals (rung 3), when its number of inverted pairs
  exceeds r >= 0.  The page prints no criterion: delta = 0, r = 0 is its strict
  reading (any disagreement in order); delta and r are the caller's.
* Rung 3 is also triggered by the certificate: a query head whose certificate
  after the promoted pass exceeds eps falls back as well (an addition to the
  page's trigger; the certificate bounds the same failure, quantization noise
  distorting the attention distribution, with a proof).
* Rung 4 (the whole layer densely) is every head falling back; it is not a
  separate step here.
"""

import numpy as np

from . import numerics as nx
from .codec import decode_k, TILE
from .rotation import rotation_matrix_f64, D


def block_mass(cache, q_bits, dtype, seq_len, rotation, signs=None, r16=None, softmax_scale=None):
    """Estimated attention mass per block from the quantized keys (fp64).

    Returns P [B, Hq, Tmax // 64]; blocks at or past seq_len are 0; a row with
    seq_len 0 is all 0.
    """
    B, Hq, _ = q_bits.shape
    H = cache.H
    G = Hq // H
    sigma = 1.0 / np.sqrt(D) if not softmax_scale else float(softmax_scale)
    R = rotation_matrix_f64(rotation, signs, r16)
    q = nx.widen_input(q_bits, dtype).astype(np.float64)
    out = np.zeros((B, Hq, cache.Tmax // TILE))
    for b in range(B):
        T = int(seq_len[b])
        if T <= 0:
            continue
        nb = (T + TILE - 1) // TILE
        for h in range(H):
            kh = decode_k(cache, b, h, 0, T)
            for hq in range(h * G, (h + 1) * G):
                logits = (kh @ (R @ q[b, hq])) * sigma
                w = np.exp(logits - logits.max())
                p = w / w.sum()
                out[b, hq, :nb] = np.add.reduceat(p, np.arange(0, T, TILE))
    return out


def top_blocks(mass_f32, n_blocks, tau_cov):
    """Indices of the top-K* blocks of one query head (reading above).

    mass_f32: fp32 masses of blocks [0, n_blocks); returns the selected indices
    in selection order.
    """
    m = np.asarray(mass_f32[:n_blocks], np.float32)
    order = sorted(range(n_blocks), key=lambda i: (-float(m[i]), i))
    run = np.float32(0.0)
    tau = np.float32(tau_cov)
    for k, i in enumerate(order):
        run = np.float32(run + m[i])
        if run >= tau:
            return order[:k + 1]
    return order


def select_blocks(mass_f32, seq_len, tau_cov, n_kv_heads, flags_in=None):
    """Promotion flags uint8 [B, Hkv, nblk]: the given flags (e.g. the bound's; zeros
    if None) with bit 0 set on the union over each kv head's query heads of their
    top-K* blocks."""
    B, Hq, nblk = mass_f32.shape
    G = Hq // n_kv_heads
    out = np.zeros((B, n_kv_heads, nblk), np.uint8) if flags_in is None else np.array(flags_in, np.uint8, copy=True)
    for b in range(B):
        nb = (int(seq_len[b]) + TILE - 1) // TILE
        if nb == 0:
            continue
        for hq in range(Hq):
            for i in top_blocks(mass_f32[b, hq], nb, tau_cov):
                out[b, hq // G, i] |= 1
    return out


def promote_values(mass_f32, ev_f32, seq_len, tau_v, n_kv_heads, flags):
    """Rung 2 (reading above): flags uint8 [B, Hkv, nblk] with 2 set on the blocks
    without bit 0 whose fp32 product mass * ev exceeds tau_v for some query head of
    the kv head.  mass_f32 [B, Hq, nblk], ev_f32 [B, Hkv, nblk]."""
    B, Hq, nblk = mass_f32.shape
    G = Hq // n_kv_heads
    out = np.array(flags, np.uint8, copy=True)
    tau = np.float32(tau_v)
    for b in range(B):
        nb = (int(seq_len[b]) + TILE - 1) // TILE
        for hq in range(Hq):
            h = hq // G
            for j in range(nb):
                if out[b, h, j] & 1:
                    continue
                if np.float32(mass_f32[b, hq, j]) * np.float32(ev_f32[b, h, j]) > tau:
                    out[b, h, j] |= 2
    return out


def block_scores_fp16(k_orig_bits, q_bits, dtype, seq_len, softmax_scale=None):
    """Block scores from the originals (fp64): s[b, hq, j] = log sum_{t in block j}
    exp(sigma q . k_t) over the positions below seq_len (original basis, no
    rotation); -inf for blocks past the sequence.  k_orig_bits [B, Hkv, Tmax, 128]."""
    B, Hq, _ = q_bits.shape
    H, Tmax = k_orig_bits.shape[1], k_orig_bits.shape[2]
    G = Hq // H
    sigma = 1.0 / np.sqrt(D) if not softmax_scale else float(softmax_scale)
    q = nx.widen_input(q_bits, dtype).astype(np.float64)
    out = np.full((B, Hq, Tmax // TILE), -np.inf)
    for b in range(B):
        T = int(seq_len[b])
        if T <= 0:
            continue
        for h in range(H):
            k = nx.widen_input(k_orig_bits[b, h, :T], dtype).astype(np.float64)
            for hq in range(h * G, (h + 1) * G):
                lg = (k @ q[b, hq]) * sigma
                for j in range((T + TILE - 1) // TILE):
                    x = lg[j * TILE:min(T, (j + 1) * TILE)]
                    mx = x.max()
                    out[b, hq, j] = mx + np.log(np.sum(np.exp(x - mx)))
    return out


def inverted_pairs(order, score, margin):
    """Pairs (i, j), i before j in order, with score[order[j]] > score[order[i]] + margin."""
    n = 0
    for a in range(len(order)):
        for c in range(a + 1, len(order)):
            if score[order[c]] > score[order[a]] + margin:
                n += 1
    return n


def ranking_inversions(mass_f32, score16, seq_len, tau_cov, margin, window=0.0):
    """Inverted pairs among each query head's promoted blocks (reading above).

    Returns (lo, hi), int64 [B, Hq]: the count with the margin raised, and lowered,
    by window (window = 0: lo == hi, the count itself).  A computation of the
    scores that is accurate to window/2 counts a number in [lo, hi].
    """
    B, Hq, _ = mass_f32.shape
    lo = np.zeros((B, Hq), np.int64)
    hi = np.zeros((B, Hq), np.int64)
    for b in range(B):
        nb = (int(seq_len[b]) + TILE - 1) // TILE
        if nb == 0:
            continue
        for hq in range(Hq):
            order = top_blocks(mass_f32[b, hq], nb, tau_cov)
            lo[b, hq] = inverted_pairs(order, score16[b, hq], margin + window)
            hi[b, hq] = inverted_pairs(order, score16[b, hq], margin - window)
    return lo, hi


def dense_fallback(out, certificate, eps, dense_out, fail=None):
    """Rows whose certificate exceeds eps, or that failed the ranking check (fail
    [B, Hq] nonzero), take the dense result (and certificate 0)."""
    out = np.array(out, np.float64, copy=True)
    cert = np.array(certificate, np.float64, copy=True)
    redo = cert > eps
    if fail is not None:
        redo = redo | (np.asarray(fail) != 0)
    out[redo] = dense_out[redo]
    cert[redo] = 0.0
    return out, cert, redo
