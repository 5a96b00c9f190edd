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
  head) is the union over its query heads; promotion takes keys and values
  together (this also covers the page's value promotion for those blocks).
  Blocks the certified bound flags (error bound > tau) are promoted as well:
  that is the value-error rung, with the bound as the contribution estimate.
* The per-head fallback is triggered by the certificate: a query head whose
  certificate after the promoted pass exceeds eps is recomputed with dense
  attention over the originals, which returns the dense result exactly.  (The
  page's trigger is a ranking-consistency check between quantized and
  full-precision block scores, for which it prints no criterion; the
  certificate bounds the same failure - quantization noise distorting the
  attention distribution - with a proof.)
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
    """Promotion flags uint8 [B, Hkv, nblk]: the union over each kv head's query
    heads of their top-K* blocks, OR the bound's flags (if given)."""
    B, Hq, nblk = mass_f32.shape
    G = Hq // n_kv_heads
    out = np.zeros((B, n_kv_heads, nblk), np.uint8) if flags_in is None else (np.asarray(flags_in) != 0).astype(np.uint8)
    for b in range(B):
        nb = (int(seq_len[b]) + TILE - 1) // TILE
        if nb == 0:
            continue
        for hq in range(Hq):
            for i in top_blocks(mass_f32[b, hq], nb, tau_cov):
                out[b, hq // G, i] = 1
    return out


def dense_fallback(out, certificate, eps, dense_out):
    """Rows whose certificate exceeds eps take the dense result (and certificate 0)."""
    out = np.array(out, np.float64, copy=True)
    cert = np.array(certificate, np.float64, copy=True)
    redo = cert > eps
    out[redo] = dense_out[redo]
    cert[redo] = 0.0
    return out, cert, redo
