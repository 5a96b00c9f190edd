"""Single-token decode attention over the packed cache, in fp64.

Test infrastructure only: see the package docstring for who may import it.

The read side streams the quantized K/V and computes softmax(q k^T / sqrt(d)) V
for the newest query token.  The plain definition is evaluated directly:

* the query is rotated once by the same operator as the cache (q_rot = R q),
  so scores are preserved ("Search Your Block Floating Point Scales!",
  incoherence processing);
* K and V are decoded exactly (codes x scales, fp64) from the packed bytes;
* logits l_i = (q_rot . k_hat_i) * sigma, sigma = 1/sqrt(128) unless given
  (the dense fallback on "Runtime-Certified Bounded-Error Quantized Attention",
  Methodology section 1, is scaled_dot_product_attention, whose default scale
  is 1/sqrt(d));
* softmax with the maximum subtracted, o_rot = sum_i p_i v_hat_i, and the output
  is brought back to the original basis, o = R^T o_rot ("OSCAR", section 2.2B:
  unpack, dequantize, inverse rotation, attention);
* for blocks flagged for exact recompute (64 tokens each), the fp16 originals
  are used instead, in the original basis, for both the logits and the values
  ("Runtime-Certified ...", Methodology sections 1 and 3: fetch the fp16 data
  and compute exact dense attention for what the bound does not cover); a
  block whose flag has bit 0 clear and bit 1 set takes only its values from the
  originals, its logits from the quantized keys (the same page, section 3,
  rung 2: value promotion);
* with a full-precision window, the first n_sink and the last n_recent 64-token
  blocks of the sequence are likewise taken from the full-precision originals,
  in the original basis ("OSCAR", section 2.2B: sink and recent tokens kept in
  BF16, the historical middle in INT2; "Search Your Block Floating Point
  Scales!", attention-sink-aware mixed-precision caching: the first and last
  blocks at full precision, the middle blocks in NVFP4).  Reading: "blocks" are
  the 64-token blocks of the position grid, and "last" counts back from the block
  holding the newest token, so with T tokens the window is the blocks j with
  j < n_sink or j >= ceil(T / 64) - n_recent.

Grouped-query attention: query head hq reads kv head hq // (Hq / Hkv).
No mask: the query attends to positions [0, seq_len), which include the token
appended last.
"""

import numpy as np

from . import numerics as nx
from .codec import decode_k, decode_v, TILE
from .rotation import rotation_matrix_f64, D


def window_blocks(T, n_sink, n_recent):
    """Boolean mask over the ceil(T / 64) blocks of a T-token sequence: True for
    the blocks kept at full precision (the first n_sink, the last n_recent)."""
    nb = (int(T) + TILE - 1) // TILE
    j = np.arange(nb)
    return (j < n_sink) | (j >= nb - n_recent)


def decode_attention(cache, q_bits, dtype, seq_len, rotation, signs=None, r16=None,
                     flags=None, softmax_scale=None, rows=None, window=None, originals=None):
    """Decode attention for every (b, hq) (or the given (b, hq) rows).

    q_bits: uint16 [B, Hq, 128] (fp16/bf16 bit patterns); seq_len: [B];
    flags: uint8 [B, Hkv, nblk] or None (bit 0: exact block; bit 1 alone: exact values).
    window: (n_sink, n_recent) blocks kept at full precision, or None; then
    originals = (k_bits, v_bits), uint16 [B, Hkv, >= T, 128], the appended inputs.
    Returns (out fp64 [B, Hq, 128], block_mass fp64 [B, Hq, nblk]); rows that
    were not requested are left zero.
    """
    B, Hq, _ = q_bits.shape
    H = cache.H
    G = Hq // H
    sigma = 1.0 / np.sqrt(D) if not softmax_scale else float(softmax_scale)
    R = rotation_matrix_f64(rotation, signs, r16)
    q = nx.widen_input(q_bits, dtype).astype(np.float64)
    nblk = cache.Tmax // TILE
    out = np.zeros((B, Hq, D))
    mass = np.zeros((B, Hq, nblk))
    if rows is None:
        rows = [(b, hq) for b in range(B) for hq in range(Hq)]
    by_stream = {}
    for b, hq in rows:
        by_stream.setdefault((b, hq // G), []).append(hq)
    for (b, h), hqs in by_stream.items():
        T = int(seq_len[b])
        if T <= 0:
            continue
        kh = decode_k(cache, b, h, 0, T)
        vh = decode_v(cache, b, h, 0, T)
        exact = np.zeros(T, dtype=bool)   # keys and values from the originals
        exact_v = np.zeros(T, dtype=bool)  # values from the originals
        if flags is not None:
            for blk in range((T + TILE - 1) // TILE):
                sl = slice(blk * TILE, min(T, (blk + 1) * TILE))
                if flags[b, h, blk] & 1:
                    exact[sl] = True
                elif flags[b, h, blk] & 2:
                    exact_v[sl] = True
        if window is not None:
            for blk in np.nonzero(window_blocks(T, *window))[0]:
                exact[blk * TILE:min(T, (blk + 1) * TILE)] = True
        exact_v |= exact
        if exact_v.any():
            # the originals: the kept copy, or the inputs (identical where both exist)
            src_k, src_v = (cache.k_orig, cache.v_orig) if originals is None else originals
            ko = nx.widen_input(src_k[b, h, :T], dtype).astype(np.float64)
            vo = nx.widen_input(src_v[b, h, :T], dtype).astype(np.float64)
        for hq in hqs:
            qr = R @ q[b, hq]
            logits = (kh @ qr) * sigma
            if exact.any():
                logits[exact] = (ko[exact] @ q[b, hq]) * sigma
            m = np.max(logits)
            w = np.exp(logits - m)
            p = w / np.sum(w)
            o_rot = p[~exact_v] @ vh[~exact_v]
            o = R.T @ o_rot
            if exact_v.any():
                o = o + p[exact_v] @ vo[exact_v]
            out[b, hq] = o
            for blk in range((T + TILE - 1) // TILE):
                mass[b, hq, blk] = np.sum(p[blk * TILE:min(T, (blk + 1) * TILE)])
    return out, mass


def dense_attention(k_orig_bits, v_orig_bits, q_bits, dtype, seq_len, softmax_scale=None):
    """Exact fp64 attention over fp16/bf16 originals (no quantization, no rotation).

    k/v: uint16 [B, Hkv, Tmax, 128]; q: uint16 [B, Hq, 128].
    """
    B, Hq, _ = q_bits.shape
    H = k_orig_bits.shape[1]
    G = Hq // H
    sigma = 1.0 / np.sqrt(D) if not softmax_scale else float(softmax_scale)
    q = nx.widen_input(q_bits, dtype).astype(np.float64)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        T = int(seq_len[b])
        for h in range(H):
            k = nx.widen_input(k_orig_bits[b, h, :T], dtype).astype(np.float64)
            v = nx.widen_input(v_orig_bits[b, h, :T], dtype).astype(np.float64)
            for g in range(G):
                hq = h * G + g
                lg = (k @ q[b, hq]) * sigma
                w = np.exp(lg - lg.max())
                out[b, hq] = (w / w.sum()) @ v
    return out


def row_rel_err(got, ref):
    """Per-row max_j |got_j - ref_j| / max_j |ref_j| (the attention parity metric)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return num / np.where(den == 0, 1.0, den)
