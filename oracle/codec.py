"""Per-group scales, codes, and the packed cache layout (write side and its inverse).

Test infrastructure only: see the package docstring for who may import it.

Formats (d = 128 channels per head vector, y = the fp32 rotated vector):

int4 / int8 symmetric, group G in {32, 128} (int4 also 16)
    "When Quantization Is Free", Methodology section 2 (per-group absmax, round to
    signed int4/int8, two int4 per byte) and "Runtime-Certified Bounded-Error
    Quantized Attention", Methodology section 1 (INT8 keys, INT4 values).
    a = max|y| over the group; s = fp16(fl32(a / qmax)) with qmax = 7 or 127;
    code = clamp(rne(y / s), -qmax, qmax) with rne the round-half-to-even of the
    exact quotient by the *stored* fp16 scale; s == 0 gives all-zero codes.
    Readings: qmax = 2^(b-1)-1 (symmetric, -8/-128 unused); dividing by the
    stored scale makes |y - c*s| <= s/2 hold against the metadata.
    Groups of 16 (int4): "When Quantization Is Free", Methodology section 3
    (per-channel scaling combined with groups of 16 for d = 128).

int2 asymmetric with clipping, group 32
    "OSCAR", section 2.2A (clipping thresholds from rotated calibration
    activations) and 2.2B (INT2 history).  y is first clamped to [-t_c, t_c]
    per channel; lo/hi = min/max of the group; s = fp16(fl32(fl32(hi-lo)/3));
    z = fp16(lo); code = clamp(rne(fl32(y - z) / s), 0, 3); value = c*s + z.
    Reading: the zero point is stored as an fp16 offset value (scale/offset
    metadata, "Runtime-Certified ..." Methodology section 1).

fp4 E2M1 with an E4M3 scale per 16, absmax or searched
    "Search Your Block Floating Point Scales!", Methodology (ScaleSearch).
    t = fl32(a / 6); candidates S_k = E4M3(fl32(t * m_k)) for
    m_k in {0.900, 0.925, ..., 1.100} (9 values) or m = 1 only (absmax);
    codes = nearest E2M1 to y / S_k; err_k = sum of fl32(d_j^2),
    d_j = fl32(y_j - e_j * S_k), summed sequentially over j = 0..7 and 8..15
    separately, then the two halves added; the first k with the smallest err
    is kept.  Readings: the multiplicative grid stands in for the page's
    bit-offset search (the configured workload asks for it); 9 points so that
    x1.00 is a candidate; candidates are rounded to E4M3 before their error is
    measured, since the stored scale is what dequantization uses.
    Mode "offsets" is the search as the page states it: the candidates are the
    E4M3 bit patterns c0 + f of the absmax scale c0 = E4M3(t), for the integer
    offsets f = -2, ..., 6 in that order (the page's reinterpret-add-reinterpret),
    keeping only non-negative finite patterns 0x00..0x7E.  The range is the
    page's own example (f in [-2, 6]); it covers the ~1.5x larger scales the page
    finds optimal for many blocks (absmax mapped to 4 instead of 6) plus two
    smaller ones.

Layout of the cache buffers (bytes; little-endian; B batch, H kv heads,
Tmax positions, a multiple of 64):

    k_codes[B][H][Tmax][KB]      K code row of each token, channel order
    k_meta [B][H][Tmax][KM]      its scales (int2: 4 scales then 4 offsets)
    v_codes[B][H][Tmax/64][128][CB]
                                 V codes per 64-token tile, channel-major: the
                                 64 codes of channel c are packed consecutively
                                 along the token axis
    v_meta [B][H][Tmax/64][NM][64]  V metadata per tile, element-major

Packing inside a byte: int4/fp4 element e at nibble e % 2 of byte e // 2 (even
element in the low nibble); int2 element e at bits 2*(e%4) of byte e // 4; int8
one byte per element (two's complement).  For K the element index is the
channel; for V tiles it is the token within the tile.
"""

import numpy as np

from . import numerics as nx
from .rotation import rotate_input_f32, D

FORMATS = ("int4", "int8", "int2", "fp4")
SEARCH_M = np.array([0.9, 0.925, 0.95, 0.975, 1.0, 1.025, 1.05, 1.075, 1.1], dtype=np.float32)
SEARCH_OFFSETS = tuple(range(-2, 7))  # f in the page's s(f) = reinterpret(reinterpret(s, int8) + f)
SCALE_MODES = ("absmax", "search9", "offsets")
TILE = 64


def qmax_of(fmt):
    return {"int4": 7, "int8": 127}[fmt]


def bits_of(fmt):
    return {"int4": 4, "int8": 8, "int2": 2, "fp4": 4}[fmt]


def group_of(fmt, group):
    if fmt == "int2":
        return 32
    if fmt == "fp4":
        return 16
    if group in (32, 128) or (fmt == "int4" and group == 16):
        return group
    raise ValueError("int4 groups are 16, 32 or 128; int8 groups 32 or 128")


def row_bytes(fmt):
    """KB: packed code bytes per 128-channel vector."""
    return D * bits_of(fmt) // 8


def meta_elems(fmt, group):
    """(NM, ES): metadata elements per vector and bytes per element."""
    g = group_of(fmt, group)
    if fmt in ("int4", "int8"):
        return D // g, 2
    if fmt == "int2":
        return 2 * (D // 32), 2
    return D // 16, 1


def chan_bytes(fmt):
    """CB: bytes holding one channel's 64 tokens in a V tile."""
    return TILE * bits_of(fmt) // 8


# ------------------------------------------------------------------ quantizers
def quantize_sym(y, fmt, group):
    """Symmetric absmax quantization of fp32 vectors y [..., 128].

    Returns (codes int16 [..., 128], scales float16 [..., 128/G]).
    """
    qmax = qmax_of(fmt)
    g = group_of(fmt, group)
    y = np.asarray(y, dtype=np.float32)
    yg = y.reshape(y.shape[:-1] + (D // g, g))
    a = np.max(np.abs(yg), axis=-1)  # exact
    s = nx.f16_sat(nx.f32(a) / np.float32(qmax))  # fl32 divide, then fp16 RNE
    sf = s.astype(np.float64)[..., None]
    safe = np.where(sf == 0, 1.0, sf)
    c = np.clip(nx.rne_quotient(yg, safe), -qmax, qmax)
    c = np.where(sf == 0, 0, c)
    return c.reshape(y.shape).astype(np.int16), s


def dequant_sym(codes, scales, fmt, group):
    g = group_of(fmt, group)
    c = np.asarray(codes, dtype=np.float64)
    cg = c.reshape(c.shape[:-1] + (D // g, g))
    return (cg * np.asarray(scales, dtype=np.float64)[..., None]).reshape(c.shape)


def clip_f32(y, t):
    """y_c <- min(max(y_c, -t_c), t_c) with per-channel fp32 thresholds t."""
    y = np.asarray(y, dtype=np.float32)
    t = np.asarray(t, dtype=np.float32)
    return np.minimum(np.maximum(y, -t), t)


def quantize_asym2(y, clip_t=None):
    """Asymmetric 2-bit quantization, group 32, optional per-channel clipping.

    Returns (codes int16 [..., 128], scales f16 [..., 4], offsets f16 [..., 4]).
    """
    y = np.asarray(y, dtype=np.float32)
    if clip_t is not None:
        y = clip_f32(y, clip_t)
    yg = y.reshape(y.shape[:-1] + (4, 32))
    lo = np.min(yg, axis=-1)
    hi = np.max(yg, axis=-1)
    s = nx.f16_sat(nx.f32(nx.f32(hi - lo) / np.float32(3.0)))
    z = nx.f16_sat(lo)
    sf = s.astype(np.float64)[..., None]
    zf32 = z.astype(np.float32)[..., None]
    r = nx.f32(yg - zf32)  # fl32(y - z)
    safe = np.where(sf == 0, 1.0, sf)
    c = np.clip(nx.rne_quotient(r, safe), 0, 3)
    c = np.where(sf == 0, 0, c)
    return c.reshape(y.shape).astype(np.int16), s, z


def dequant_asym2(codes, scales, offsets):
    c = np.asarray(codes, dtype=np.float64)
    cg = c.reshape(c.shape[:-1] + (4, 32))
    v = cg * np.asarray(scales, np.float64)[..., None] + np.asarray(offsets, np.float64)[..., None]
    return v.reshape(c.shape)


def _fp4_block_error(yb, codes, S):
    """err = fl32(seqsum_{j<8} fl32(d_j^2) + seqsum_{8<=j<16} fl32(d_j^2)), d = fl32(y - e*S).

    The page defines the error as the sum of squared residuals over the block, not an
    order of summation; the reading taken is two sequential fp32 partial sums (elements
    0..7 and 8..15) added at the end, which halves the dependent-add chain per
    candidate in a write kernel.  The order decides the choice on near ties, so it is
    part of the bit-exact contract (pinned by tests/golden/fp4_sum_order.txt).
    """
    e = nx.e2m1_value(codes)
    prod = nx.f32(e * np.asarray(S, np.float64)[..., None])  # exact: <= 6 significant bits
    d = nx.f32(yb - prod)
    sq = nx.f32(d * d)
    lo = np.zeros(yb.shape[:-1], dtype=np.float32)
    hi = np.zeros(yb.shape[:-1], dtype=np.float32)
    for j in range(8):
        lo = nx.f32(lo + sq[..., j])
        hi = nx.f32(hi + sq[..., 8 + j])
    return nx.f32(lo + hi)


def quantize_fp4(y, scale_mode="search9"):
    """FP4 E2M1 codes with E4M3 block scales (16 elements), absmax or searched.

    Returns (codes uint8 nibbles [..., 128], scale codes uint8 [..., 8]).
    """
    if scale_mode not in SCALE_MODES:
        raise ValueError(scale_mode)
    y = np.asarray(y, dtype=np.float32)
    yb = y.reshape(y.shape[:-1] + (8, 16))
    a = np.max(np.abs(yb), axis=-1)
    t = nx.f32(nx.f32(a) / np.float32(6.0))
    if scale_mode == "offsets":
        c0 = nx.e4m3_encode_nonneg(t).astype(np.int64)
        # patterns outside 0x00..0x7E are not candidates: clamping them onto the ends repeats
        # a candidate already tried (same error), so the first-smallest choice is unchanged
        cands = [np.clip(c0 + f, 0, 0x7E).astype(np.uint8) for f in SEARCH_OFFSETS]
    else:
        mults = SEARCH_M if scale_mode == "search9" else np.array([1.0], dtype=np.float32)
        cands = [nx.e4m3_encode_nonneg(nx.f32(t * m)) for m in mults]
    best_err = None
    best_codes = None
    best_sc = None
    for sc in cands:
        S = nx.e4m3_value(sc)
        Ssafe = np.where(S == 0, 1.0, S)
        codes = nx.e2m1_quantize(yb, Ssafe[..., None])
        codes = np.where((S == 0)[..., None], np.uint8(0), codes).astype(np.uint8)
        err = _fp4_block_error(yb, codes, np.where(S == 0, 0.0, S))
        if best_err is None:
            best_err, best_codes, best_sc = err, codes, sc
        else:
            better = err < best_err  # strict: the first k with the smallest error wins
            best_err = np.where(better, err, best_err)
            best_codes = np.where(better[..., None], codes, best_codes)
            best_sc = np.where(better, sc, best_sc)
    return best_codes.reshape(y.shape).astype(np.uint8), best_sc.astype(np.uint8)


def dequant_fp4(codes, scale_codes):
    v = nx.e2m1_value(codes)
    vb = v.reshape(v.shape[:-1] + (8, 16))
    return (vb * nx.e4m3_value(scale_codes)[..., None]).reshape(v.shape)


def quantize(y, fmt, group=32, scale_mode="search9", clip_t=None):
    """Dispatch: returns (codes [..., 128] as small ints, meta elements [..., NM]).

    Meta elements: fp16 scales (int4/int8), fp16 [s0..s3, z0..z3] (int2), or
    E4M3 codes (fp4).  Clipping applies to int2 only.
    """
    if fmt in ("int4", "int8"):
        c, s = quantize_sym(y, fmt, group)
        return c, s
    if fmt == "int2":
        c, s, z = quantize_asym2(y, clip_t)
        return c, np.concatenate([s, z], axis=-1)
    if fmt == "fp4":
        return quantize_fp4(y, scale_mode)
    raise ValueError(fmt)


def dequantize(codes, meta, fmt, group=32):
    """Exact fp64 values of codes + metadata (rotated basis)."""
    if fmt in ("int4", "int8"):
        return dequant_sym(codes, meta, fmt, group)
    if fmt == "int2":
        return dequant_asym2(codes, meta[..., :4], meta[..., 4:])
    if fmt == "fp4":
        return dequant_fp4(codes, meta)
    raise ValueError(fmt)


# ------------------------------------------------------------------ packing
def pack_elems(codes, fmt):
    """Pack small integer codes along the last axis into bytes (see module doc)."""
    c = np.asarray(codes).astype(np.int64)
    bits = bits_of(fmt)
    mask = (1 << bits) - 1
    per = 8 // bits
    cg = (c & mask).reshape(c.shape[:-1] + (c.shape[-1] // per, per))
    out = np.zeros(cg.shape[:-1], dtype=np.int64)
    for e in range(per):
        out |= cg[..., e] << (bits * e)
    return out.astype(np.uint8)


def unpack_elems(packed, fmt, signed):
    """Inverse of pack_elems; signed=True sign-extends (int4/int8 two's complement)."""
    p = np.asarray(packed, dtype=np.int64)
    bits = bits_of(fmt)
    mask = (1 << bits) - 1
    per = 8 // bits
    out = np.stack([(p >> (bits * e)) & mask for e in range(per)], axis=-1)
    out = out.reshape(p.shape[:-1] + (p.shape[-1] * per,))
    if signed:
        out = np.where(out >= (1 << (bits - 1)), out - (1 << bits), out)
    return out


def meta_to_bytes(meta, fmt):
    """Metadata elements -> little-endian bytes (fp16 -> 2 bytes, E4M3 -> 1)."""
    if fmt == "fp4":
        return np.asarray(meta, dtype=np.uint8)
    m = np.ascontiguousarray(np.asarray(meta, dtype=np.float16))
    return m.view(np.uint8).reshape(m.shape[:-1] + (m.shape[-1] * 2,))


def bytes_to_meta(b, fmt):
    if fmt == "fp4":
        return np.asarray(b, dtype=np.uint8)
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint8))
    return b.view(np.float16).reshape(b.shape[:-1] + (b.shape[-1] // 2,))


# ------------------------------------------------------------------ cache
class Cache:
    """Host mirror of the cache buffers, with the byte layout in the module doc."""

    def __init__(self, B, H, Tmax, k_fmt, v_fmt, k_group=32, v_group=32, keep_fp16_copy=False, lam_k=None,
                 lam_v=None):
        if Tmax % TILE:
            raise ValueError("Tmax must be a multiple of 64")
        # per-channel rescale factors [H, 128] (fp32) of K and V, or None
        self.lam_k = None if lam_k is None else np.asarray(lam_k, np.float32)
        self.lam_v = None if lam_v is None else np.asarray(lam_v, np.float32)
        self.B, self.H, self.Tmax = B, H, Tmax
        self.k_fmt, self.v_fmt, self.k_group, self.v_group = k_fmt, v_fmt, k_group, v_group
        nt = Tmax // TILE
        self.k_codes = np.zeros((B, H, Tmax, row_bytes(k_fmt)), np.uint8)
        nmk, esk = meta_elems(k_fmt, k_group)
        self.k_meta = np.zeros((B, H, Tmax, nmk * esk), np.uint8)
        self.v_codes = np.zeros((B, H, nt, D, chan_bytes(v_fmt)), np.uint8)
        nmv, esv = meta_elems(v_fmt, v_group)
        self.v_meta = np.zeros((B, H, nt, nmv, TILE * esv), np.uint8)
        self.keep = keep_fp16_copy
        if keep_fp16_copy:
            self.k_orig = np.zeros((B, H, Tmax, D), np.uint16)
            self.v_orig = np.zeros((B, H, Tmax, D), np.uint16)

    # --- V tile helpers (token-major codes <-> channel-major packed tile bytes)
    def _v_store(self, b, h, t, codes, meta):
        """Write codes [n,128] / meta [n,NM] of tokens t..t+n-1 into the V tiles.

        Each touched tile is decoded to token-major codes, the new rows are
        overwritten, and the tile is packed again (so earlier tokens sharing a
        byte are preserved).
        """
        fmt = self.v_fmt
        n = codes.shape[0]
        _, es = meta_elems(fmt, self.v_group)
        mb = meta_to_bytes(meta, fmt)  # [n, NM*ES]
        for tile in range(t // TILE, (t + n - 1) // TILE + 1):
            tok = self.v_tile_codes(b, h, tile)  # [64, 128]
            lo = max(t, tile * TILE)
            hi = min(t + n, (tile + 1) * TILE)
            tok[lo - tile * TILE:hi - tile * TILE] = codes[lo - t:hi - t]
            self.v_codes[b, h, tile] = pack_elems(tok.T, fmt)
            for pos in range(lo, hi):
                tau = pos - tile * TILE
                elems = mb[pos - t].reshape(-1, es)
                self.v_meta[b, h, tile][:, tau * es:(tau + 1) * es] = elems

    def v_tile_codes(self, b, h, tile):
        """Codes [64 tokens, 128 channels] of one V tile, decoded from bytes."""
        signed = self.v_fmt in ("int4", "int8")
        raw = unpack_elems(self.v_codes[b, h, tile], self.v_fmt, signed)  # [128, 64]
        return raw.T.copy()

    def v_tile_meta(self, b, h, tile):
        """Metadata elements [64 tokens, NM] of one V tile."""
        _, es = meta_elems(self.v_fmt, self.v_group)
        m = self.v_meta[b, h, tile]  # [NM, 64*ES]
        nm = m.shape[0]
        per_tok = m.reshape(nm, TILE, es).transpose(1, 0, 2).reshape(TILE, nm * es)
        return bytes_to_meta(per_tok, self.v_fmt)


def append(cache, k_bits, v_bits, start_pos, dtype, rotation, signs=None, r16=None,
           clip_k=None, clip_v=None, scale_mode="search9"):
    """Rotate, quantize and pack new K/V vectors into the cache.

    k_bits, v_bits: uint16 input bit patterns [B, H, n, 128] (fp16 or bf16);
    start_pos: [B] first position written per sequence.  Follows the write-side
    order of "When Quantization Is Free", Methodology section 2: widen, sign flip,
    transform, per-group scale, round, pack.  clip_k/clip_v: per (kv head,
    channel) fp32 thresholds for int2 ("OSCAR", section 2.2A).
    With per-channel rescale factors on the cache ("When Quantization Is Free",
    Methodology sections 2 and 3: one scale per coordinate, then the per-group
    scales), the rotated vectors are multiplied by them in fp32 before clipping
    and quantization: y'_c = fl32(y_c * lambda_c).
    Returns the fp32 rotated (and rescaled) vectors (yk, yv) for the caller's checks.
    """
    B, H, n, _ = k_bits.shape
    xk = nx.widen_input(k_bits, dtype)
    xv = nx.widen_input(v_bits, dtype)
    yk = rotate_input_f32(xk, rotation, signs, r16)
    yv = rotate_input_f32(xv, rotation, signs, r16)
    if cache.lam_k is not None:
        yk = nx.f32(yk * cache.lam_k[None, :, None, :])
    if cache.lam_v is not None:
        yv = nx.f32(yv * cache.lam_v[None, :, None, :])
    for b in range(B):
        t0 = int(start_pos[b])
        if t0 < 0 or t0 + n > cache.Tmax:
            raise ValueError("append out of range")
        for h in range(H):
            ck = None if clip_k is None else clip_k[h]
            cv = None if clip_v is None else clip_v[h]
            kc, km = quantize(yk[b, h], cache.k_fmt, cache.k_group, scale_mode, ck)
            vc, vm = quantize(yv[b, h], cache.v_fmt, cache.v_group, scale_mode, cv)
            cache.k_codes[b, h, t0:t0 + n] = pack_elems(kc, cache.k_fmt)
            cache.k_meta[b, h, t0:t0 + n] = meta_to_bytes(km, cache.k_fmt)
            cache._v_store(b, h, t0, vc, vm)
            if cache.keep:
                cache.k_orig[b, h, t0:t0 + n] = k_bits[b, h]
                cache.v_orig[b, h, t0:t0 + n] = v_bits[b, h]
    return yk, yv


def decode_k(cache, b, h, t0, t1):
    """Dequantized K (rotated basis, fp64) for positions [t0, t1) of stream (b, h);
    with per-channel rescale factors, the dequantized values divided by them."""
    signed = cache.k_fmt in ("int4", "int8")
    codes = unpack_elems(cache.k_codes[b, h, t0:t1], cache.k_fmt, signed)
    meta = bytes_to_meta(cache.k_meta[b, h, t0:t1], cache.k_fmt)
    out = dequantize(codes, meta, cache.k_fmt, cache.k_group)
    if cache.lam_k is not None:
        out = out / cache.lam_k[h].astype(np.float64)
    return out


def decode_v(cache, b, h, t0, t1):
    """Dequantized V (rotated basis, fp64) for positions [t0, t1) of stream (b, h)."""
    out = np.zeros((t1 - t0, D))
    for tile in range(t0 // TILE, (t1 - 1) // TILE + 1 if t1 > t0 else t0 // TILE):
        codes = cache.v_tile_codes(b, h, tile)
        meta = cache.v_tile_meta(b, h, tile)
        vals = dequantize(codes, meta, cache.v_fmt, cache.v_group)
        lo = max(t0, tile * TILE)
        hi = min(t1, (tile + 1) * TILE)
        out[lo - t0:hi - t0] = vals[lo - tile * TILE:hi - tile * TILE]
    if cache.lam_v is not None:
        out = out / cache.lam_v[h].astype(np.float64)
    return out


def calibrate_clip(calib_bits, dtype, rotation, signs=None, r16=None, ratio=0.9, lam=None):
    """Per-channel clipping thresholds from rotated calibration vectors.

    "OSCAR", section 2.2A: thresholds are estimated from the *rotated*
    calibration activations.  Reading taken: t_c = fl32(ratio * max_t |y_t,c|)
    per (kv head, channel), with y the same fp32 write-side rotation as append
    and ratio = fl32(0.9) for the configured workload; with per-channel rescale
    factors lam [H, 128], y is rescaled first (the vectors as the quantizer sees them).
    calib_bits: uint16 [H, n, 128]; returns float32 [H, 128].
    """
    x = nx.widen_input(calib_bits, dtype)
    y = rotate_input_f32(x, rotation, signs, r16)
    if lam is not None:
        y = nx.f32(y * np.asarray(lam, np.float32)[:, None, :])
    a = np.max(np.abs(y), axis=-2)
    return nx.f32(np.float32(ratio) * a)


def calibrate_lambda(calib_bits, dtype, rotation, signs=None, r16=None):
    """Per-channel rescale factors from rotated calibration vectors.

    "When Quantization Is Free", Methodology section 2 (a per-channel rescale,
    learned or calibrated, before the per-group absmax) and section 3 (one scale
    per coordinate combined with per-group scales).  Reading taken (calibrated):
    lambda_c = fl32(1 / max_t |y_t,c|) per (kv head, channel), 1 where the maximum
    is 0, so every channel spans [-1, 1] before the group scales.
    calib_bits: uint16 [H, n, 128]; returns float32 [H, 128].
    """
    x = nx.widen_input(calib_bits, dtype)
    y = rotate_input_f32(x, rotation, signs, r16)
    a = np.max(np.abs(y), axis=-2)
    one = np.float32(1.0)
    return np.where(a > 0, nx.f32(one / np.where(a > 0, a, one)), one).astype(np.float32)
