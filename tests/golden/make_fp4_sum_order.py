"""Writes fp4_sum_order.txt: FP4 blocks on which the order of the fp32 error sum decides
which E4M3 scale the 9-point search picks ("Search Your Block Floating Point Scales!",
Methodology, ScaleSearch: the block scale is the candidate with the smallest squared
error).  The page defines the error as a sum, not an order; the reading fixes it as two
fp32 partial sums (elements 0..7 and 8..15, each sequential) added at the end.

This script does not use oracle/: it re-derives E4M3 and E2M1 rounding by enumerating
the value sets and evaluates every candidate with fp32 arithmetic in both orders.  A tie
is built on purpose: elements 0..14 are seeded draws (element 0 the block's absmax), and
element 15 is solved so that two candidate scales have equal exact error (the difference
is linear in it while its codes stay fixed); fp32 neighbours of that root are then
scanned for values where the halves order and the sequential order (j = 0..15) choose
different scales.

    python tests/golden/make_fp4_sum_order.py
"""
import os

import numpy as np

F = np.float32
MULT = np.array([0x3F666666, 0x3F6CCCCD, 0x3F733333, 0x3F79999A, 0x3F800000, 0x3F833333, 0x3F866666,
                 0x3F89999A, 0x3F8CCCCD], np.uint32).view(np.float32)  # fl32(0.900), ..., fl32(1.100)
# E4M3FN non-negative values by code (bias 7, subnormal step 2^-9, 0x7F is NaN)
E4M3 = np.array([(c & 7) * 2.0 ** -9 if c < 8 else (1 + (c & 7) / 8) * 2.0 ** ((c >> 3) - 7) for c in range(127)])
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e4m3(x):
    """Round a non-negative fp32 to E4M3 (nearest, ties to the even code, saturating at 448)."""
    x = float(x)
    if x >= 448.0:
        return 126
    return min(range(127), key=lambda c: (abs(E4M3[c] - x), c & 1))


def e2m1_signed(y, S):
    """Signed E2M1 values nearest to y / S (ties to the even code, magnitudes above 6 -> 6)."""
    r = np.abs(y.astype(np.float64)) / S
    dist = np.abs(r[..., None] - E2M1)
    key = dist * 4 + (np.arange(8) & 1) * 1e-300  # exact distances; equal -> even code first
    idx = np.argmin(np.where(dist == dist.min(-1, keepdims=True), np.arange(8) & 1, 9), axis=-1)
    return np.copysign(E2M1[idx], y)


def candidate_codes(absmax):
    t = F(F(absmax) / F(6.0))
    return [e4m3(F(t * m)) for m in MULT]


def errors(y, codes, order):
    """fp32 error of every candidate for blocks y [N, 16] -> [N, 9]."""
    out = np.empty((y.shape[0], len(codes)), np.float32)
    for k, c in enumerate(codes):
        S = E4M3[c]
        d = y if S == 0.0 else (y - (e2m1_signed(y, S) * S).astype(np.float32)).astype(np.float32)
        sq = (d * d).astype(np.float32)
        if order == "halves":
            lo = np.zeros(y.shape[0], np.float32)
            hi = np.zeros(y.shape[0], np.float32)
            for j in range(8):
                lo = (lo + sq[:, j]).astype(np.float32)
                hi = (hi + sq[:, 8 + j]).astype(np.float32)
            out[:, k] = (lo + hi).astype(np.float32)
        else:
            e = np.zeros(y.shape[0], np.float32)
            for j in range(16):
                e = (e + sq[:, j]).astype(np.float32)
            out[:, k] = e
    return out


def choice(err):
    """First candidate with the strictly smallest error."""
    return np.argmin(err, axis=1)


def search(rng, n_want):
    found = []
    for attempt in range(2000):
        head = (rng.standard_normal(15) / np.sqrt(rng.chisquare(4, 15) / 4)).astype(np.float32)
        head[0] = F(np.abs(head).max() * 1.25 + 0.01)  # element 0 is the absmax
        a = float(head[0])
        codes = candidate_codes(a)
        uniq = sorted(set(codes), key=codes.index)
        for i in range(len(uniq) - 1):
            S1, S2 = E4M3[uniq[i]], E4M3[uniq[i + 1]]
            r1 = head.astype(np.float64) - e2m1_signed(head, S1) * S1
            r2 = head.astype(np.float64) - e2m1_signed(head, S2) * S2
            C = float(np.sum(r1 * r1) - np.sum(r2 * r2))
            for v1 in np.concatenate([E2M1, -E2M1[1:]]):
                for v2 in np.concatenate([E2M1, -E2M1[1:]]):
                    den = 2.0 * (v1 * S1 - v2 * S2)
                    if den == 0.0:
                        continue
                    ys = (C + (v1 * S1) ** 2 - (v2 * S2) ** 2) / den
                    if not abs(ys) < a:
                        continue
                    y0 = np.float32(ys)
                    if e2m1_signed(np.array([y0]), S1)[0] != v1 or e2m1_signed(np.array([y0]), S2)[0] != v2:
                        continue
                    # fp32 neighbours of the root
                    bits = np.int64(np.array([y0], np.float32).view(np.int32)[0])
                    scan = (bits + np.arange(-3000, 3001)).astype(np.int32).view(np.float32)
                    ys16 = np.concatenate([np.tile(head, (scan.size, 1)), scan[:, None]], axis=1).astype(np.float32)
                    ok = np.abs(scan) < a
                    kh = choice(errors(ys16, codes, "halves"))
                    ks = choice(errors(ys16, codes, "seq"))
                    ch = np.array(codes)[kh]
                    cs = np.array(codes)[ks]
                    hit = np.nonzero(ok & (ch != cs))[0]
                    for h in hit[:1]:
                        found.append((ys16[h], ch[h], cs[h]))
                    if len(found) >= n_want:
                        return found, attempt + 1
    return found, 2000


def main(n_want=3, seed=20261203):
    rng = np.random.default_rng(seed)
    found, attempts = search(rng, n_want)
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "fp4_sum_order.txt"), "w") as f:
        f.write("# Written by make_fp4_sum_order.py (standalone fp32 emulation; no oracle, no GPU).\n")
        f.write("# FP4 blocks (16 fp32 inputs to the quantizer) on which the order of the fp32 error sum\n")
        f.write("# changes the 9-point ScaleSearch choice.  Reading: error = fl32(s_lo + s_hi), s_lo and\n")
        f.write("# s_hi the sequential fp32 sums of the squared residuals of elements 0..7 and 8..15.\n")
        f.write(f"# {len(found)} blocks, {attempts} seeded draws of elements 0..14 (seed {seed}).\n")
        for y, ch, cs in found:
            f.write("block " + " ".join(f"0x{b:08X}" for b in y.view(np.uint32)) + "\n")
            f.write(f"halves_code 0x{int(ch):02X} sequential_code 0x{int(cs):02X}\n")
    print(f"{len(found)} blocks from {attempts} draws")


if __name__ == "__main__":
    main()
