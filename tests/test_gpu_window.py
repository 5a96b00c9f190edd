"""GPU parity of the full-precision window: the first sink_blocks and the last
recent_blocks 64-token blocks of each sequence attended from their originals,
the middle from the codes ("OSCAR", section 2.2B, mixed-precision layout;
"Search Your Block Floating Point Scales!", attention-sink-aware mixed-precision
caching).

Checked through the C ABI:
* the window buffers equal, byte for byte, a host model of the copy rule (every
  call copies the rows it writes in sink blocks and in its own last recent_blocks
  blocks; sink block j goes to slot j, any other block j to slot sink + j % recent),
  including single-token steps that wrap the ring;
* decode attention equals the oracle's fp64 attention with the same window, over
  the library's own codes (decoded by the oracle's unpacker), per output row
  max |out - ref| / max |ref| <= 2e-3;
* with the certified cache, flagged blocks and window blocks together, and the
  certificate agrees with the oracle's (window blocks count as exact).
"""
import numpy as np
import pytest
import torch

import bit_kv_cache_append_amd as kvq
import synth
from oracle import attention, bound
from gpu_harness import dev_bits, make_gpu_cache, oracle_view_of_gpu, setup_rotation

pytestmark = pytest.mark.gpu
TOL = 2e-3


class Windowed:
    """A GPU cache with a window, filled by appends of per-sequence position ranges."""

    def __init__(self, c):
        self.c = c
        self.s, self.r16, s_dev, r_dev = setup_rotation(c)
        self.p, self.g = make_gpu_cache(c, s_dev, r_dev)
        if c["k_fmt"] == "int2" or c["v_fmt"] == "int2":
            ck = np.stack([synth.calibration(c, 0, h) for h in range(c["Hkv"])])
            cv = np.stack([synth.calibration(c, 1, h) for h in range(c["Hkv"])])
            self.g.clip_k, self.g.clip_v = kvq.calibrate_clip(self.p, self.g, dev_bits(ck), dev_bits(cv),
                                                              ratio=c.get("clip_ratio", 0.9))
        self.len = [0] * c["B"]
        ns, nr = c["sink_blocks"], c["recent_blocks"]
        self.model = {t: np.zeros((c["B"], c["Hkv"], (ns + nr) * 64, 128), np.uint16) for t in "kv"}
        # synth values depend on the position only, so rewriting a position rewrites the same bits
        self.x = {"k": synth.kv_all(c, 0, 0, c["T"]), "v": synth.kv_all(c, 1, 0, c["T"])}
        self.k, self.v = self.x["k"], self.x["v"]

    def append(self, starts, n):
        k = np.stack([self.k[b, :, st:st + n] for b, st in enumerate(starts)])
        v = np.stack([self.v[b, :, st:st + n] for b, st in enumerate(starts)])
        kvq.append(self.p, self.g, dev_bits(k), dev_bits(v), starts)
        self.len = [st + n for st in starts]
        ns, nr = self.c["sink_blocks"], self.c["recent_blocks"]
        for b, st in enumerate(starts):
            end = st + n
            jlast = (end - 1) // 64
            for j in range(st // 64, jlast + 1):
                if j < ns or j > jlast - nr:
                    slot = j if j < ns else ns + j % nr
                    lo, hi = max(st, 64 * j), min(end, 64 * j + 64)
                    r0 = slot * 64 + lo - 64 * j
                    for t in "kv":
                        self.model[t][b, :, r0:r0 + hi - lo] = self.x[t][b, :, lo:hi]

    def check_window_bytes(self):
        c = self.c
        ns, nr = c["sink_blocks"], c["recent_blocks"]
        for t in "kv":
            got = self.g.bufs[t + "_win"].cpu().numpy().view(np.uint16).reshape(self.model[t].shape)
            assert np.array_equal(got, self.model[t]), f"{t}_win differs from the copy rule"
        # the scenario keeps the contract: every window row of the current lengths holds its original
        for b, T in enumerate(self.len):
            for j in np.nonzero(attention.window_blocks(T, ns, nr))[0]:
                slot = j if j < ns else ns + j % nr
                lo, hi = j * 64, min(T, j * 64 + 64)
                for t in "kv":
                    assert np.array_equal(self.model[t][b, :, slot * 64:slot * 64 + hi - lo], self.x[t][b, :, lo:hi])

    def decode_and_check(self, q, tag, flags=None, certificate=False):
        c = self.c
        seq = list(self.len)
        fl = None if flags is None else flags
        out = kvq.decode_attn(self.p, self.g, dev_bits(q), seq, flags=fl, certificate=certificate)
        cert = None
        if certificate:
            out, cert = out
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        oc = oracle_view_of_gpu(c, self.g)
        fln = None if fl is None else fl.cpu().numpy()
        ref, mass = attention.decode_attention(oc, q, c["dtype"], np.array(seq), c["rotation"], self.s, self.r16,
                                               flags=fln, window=(c["sink_blocks"], c["recent_blocks"]),
                                               originals=(self.k, self.v))
        rows = [(b, hq) for b in range(c["B"]) for hq in range(c["Hq"]) if seq[b] > 0]
        err = attention.row_rel_err(got, ref)
        worst = max(err[b, hq] for b, hq in rows)
        print(f"[window] {tag} seq={seq}: max row rel err {worst:.3e}", flush=True)
        assert worst <= TOL, f"{tag}: max row rel err {worst:.3e}"
        return got, ref, mass, cert, fln


def test_ring_through_single_token_steps():
    """Prefill (sequence 1 rewriting a stretch it already holds, so the lengths are
    ragged), then one token per call across two block boundaries: the ring wraps."""
    c = synth.config(2, B=2, T=1152, sink_blocks=1, recent_blocks=2)
    print("[window] int4 ring", flush=True)
    w = Windowed(c)
    w.append([0, 0], 900)
    w.append([900, 836], 100)
    w.check_window_bytes()
    q = synth.queries(c)
    w.decode_and_check(q, "int4 after prefill")
    for i in range(100):
        w.append([1000 + i, 936 + i], 1)
        if i in (23, 87, 99):
            w.check_window_bytes()
            w.decode_and_check(synth.queries(c, step=i + 1), f"int4 step {i}")


CASES = {
    # "OSCAR": sink and recent tokens in BF16, the middle INT2 after the dense rotation and clipping
    "int2-dense-bf16": (synth.config(4, B=2, T=1024, dtype="bf16", sink_blocks=1, recent_blocks=2),
                        [([0, 0], 700), ([700, 600], 100)]),
    # "Search Your Block Floating Point Scales!": first and last blocks full precision, middle NVFP4
    "fp4-search": (synth.config(5, B=2, T=1024, sink_blocks=2, recent_blocks=2), [([0, 0], 1024)]),
    "fp4-ragged-short": (synth.config(5, B=3, Hq=8, Hkv=2, T=512, sink_blocks=1, recent_blocks=1),
                         [([0, 0, 0], 100), ([100, 1, 30], 29)]),
    "int4-recent-only-g128": (synth.config(1, B=2, Hq=8, Hkv=2, T=512, k_group=128, v_group=128,
                                           sink_blocks=0, recent_blocks=3), [([0, 0], 300), ([300, 200], 150)]),
    "int4-sink-only": (synth.config(2, B=1, T=640, sink_blocks=2, recent_blocks=0), [([0], 640)]),
    "int4-g16-ragged": (synth.config(2, B=2, Hq=8, Hkv=2, T=512, k_group=16, v_group=16, sink_blocks=1,
                                     recent_blocks=1), [([0, 0], 400), ([400, 300], 50)]),
    "int8k-int4v-window-no-copy": (synth.config(3, B=2, T=1024, keep=False, sink_blocks=1, recent_blocks=1),
                                   [([0, 0], 1024), ([1000, 896], 24)]),
    "whole-sequence-in-window": (synth.config(2, B=2, T=256, sink_blocks=2, recent_blocks=2),
                                 [([0, 0], 200), ([200, 1], 1)]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_window_decode_matches_oracle(name):
    c, appends = CASES[name]
    print(f"[window] case {name}", flush=True)
    w = Windowed(c)
    for starts, n in appends:
        w.append(starts, n)
    w.check_window_bytes()
    w.decode_and_check(synth.queries(c), name)


def test_window_covering_sequence_is_dense_attention():
    c = synth.config(2, B=2, T=256, sink_blocks=4, recent_blocks=0)
    print("[window] dense", flush=True)
    w = Windowed(c)
    w.append([0, 0], 256)
    w.append([256 - 56, 77], 56)  # lengths 256 and 133
    w.check_window_bytes()
    q = synth.queries(c)
    got, _, _, _, _ = w.decode_and_check(q, "all-window")
    dense = attention.dense_attention(w.k, w.v, q, c["dtype"], np.array(w.len))
    assert attention.row_rel_err(got, dense).max() <= TOL


def test_certified_with_window():
    c = synth.config(3, B=2, T=2048, sink_blocks=1, recent_blocks=1)
    print("[window] certified", flush=True)
    w = Windowed(c)
    w.append([0, 0], 2048)
    w.append([2048 - 64, 1900], 64)  # lengths 2048 and 1964
    w.check_window_bytes()
    q = synth.queries(c)
    _, fl = kvq.error_bound(w.p, w.g, dev_bits(q), w.len, c["tau"])
    got, ref, mass, cert, fln = w.decode_and_check(q, "cert+window", flags=fl, certificate=True)
    oc = oracle_view_of_gpu(c, w.g)
    seq = np.array(w.len)
    dense = attention.dense_attention(oc.k_orig, oc.v_orig, q, c["dtype"], seq)
    E = cert.cpu().numpy()
    assert np.all(np.linalg.norm(ref - dense, axis=-1) <= E), "certificate must bound the error"
    # window blocks are exact: for the oracle's certificate they count as flagged
    exact = fln.copy()
    for b, T in enumerate(w.len):
        nb = (T + 63) // 64
        exact[b, :, :nb] |= attention.window_blocks(T, c["sink_blocks"], c["recent_blocks"]).astype(np.uint8)
    desc = bound.block_descriptors(oc, c["dtype"], c["rotation"], w.s)
    E_or = bound.certificate(desc, q, c["dtype"], seq, exact, mass)
    assert np.all(E >= E_or * (1 - 1e-5)), "certificate below the oracle's"
    assert np.all(E <= E_or * (1 + 2.0 ** -7) + 1e-9), "certificate far above the oracle's"
