"""GPU parity of kvq_decode_attn / kvq_error_bound / kvq_decode_attn_dense.

Attention is compared with the oracle's fp64 attention over the same decoded
cache (the library's own packed bytes, decoded by the oracle's unpacker, after
the append test has shown those bytes equal the oracle's): per output row,
max |out - ref| / max |ref| <= 2e-3.
"""
import numpy as np
import pytest
import torch

import bit_kv_cache_append_amd as kvq
import synth
from oracle import attention, bound, codec
from gpu_harness import (dev_bits, make_gpu_cache, oracle_view_of_gpu, setup_rotation)

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _filled(c, seq):
    """A GPU cache holding tokens [0, seq[b]) of every sequence, plus inputs for the oracle."""
    s, r16, s_dev, r_dev = setup_rotation(c)
    p, gcache = make_gpu_cache(c, s_dev, r_dev)
    if c["k_fmt"] == "int2" or c["v_fmt"] == "int2":
        ck = np.stack([synth.calibration(c, 0, h) for h in range(c["Hkv"])])
        cv = np.stack([synth.calibration(c, 1, h) for h in range(c["Hkv"])])
        tk, tv = kvq.calibrate_clip(p, gcache, dev_bits(ck), dev_bits(cv), ratio=c.get("clip_ratio", 0.9))
        gcache.clip_k, gcache.clip_v = tk, tv
    T = c["T"]
    k = synth.kv_all(c, 0, 0, T)
    v = synth.kv_all(c, 1, 0, T)
    kvq.append(p, gcache, dev_bits(k), dev_bits(v), [0] * c["B"])
    torch.cuda.synchronize()
    return s, r16, p, gcache, k, v


def _check_rows(got, ref, rows, tag):
    err = attention.row_rel_err(got, ref)
    worst = max(err[b, hq] for b, hq in rows)
    print(f"[decode] {tag}: max row rel err {worst:.3e}", flush=True)
    assert worst <= TOL, f"{tag}: max row rel err {worst:.3e}"
    return worst


CASES = {
    "c1-tiny-int4": (synth.config(1), [1024]),
    "c2-gqa-int4": (synth.config(2, B=3, T=1088), [1088, 1000, 65]),
    "c2-short-and-empty": (synth.config(2, B=4, T=256), [1, 63, 0, 64]),
    "int4-g128-none": (synth.config(1, B=2, Hq=8, Hkv=2, T=512, rotation="none", k_group=128, v_group=128), [512, 300]),
    "c3-int8k-int4v": (synth.config(3, B=2, T=2048), [2048, 1500]),
    "c4-int2-dense": (synth.config(4, B=2, T=1024), [1024, 777]),
    "g1-and-g2": (synth.config(2, B=2, Hq=4, Hkv=2, T=512), [512, 333]),
    "c5-fp4-search-bf16": (synth.config(5, B=2, T=1024), [1024, 701]),
    "fp4-absmax-f16-ragged": (synth.config(5, B=3, Hq=8, Hkv=2, T=512, dtype="f16", scale_mode="absmax"), [512, 129, 1]),
    "fp4-offsets-search": (synth.config(5, B=2, Hq=8, Hkv=2, T=512, scale_mode="offsets"), [512, 300]),
    "gqa8-two-head-groups": (synth.config(2, B=2, Hq=16, Hkv=2, T=640), [640, 513]),
    "gqa6-partial-group-bf16": (synth.config(2, B=1, Hq=12, Hkv=2, T=384, dtype="bf16"), [384]),
    "c2-int4-srft": (synth.config(2, B=2, T=640, rotation="srft"), [640, 333]),
    "int4-g16-gqa": (synth.config(2, B=3, T=640, k_group=16, v_group=16), [640, 577, 1]),
    "int4-g16-certified": (synth.config(3, B=2, T=1024, k_fmt="int4", k_group=16, v_group=16), [1024, 700]),
    "int4-g16-none-bf16": (synth.config(1, B=2, Hq=8, Hkv=2, T=384, rotation="none", k_group=16, v_group=16,
                                        dtype="bf16"), [384, 200]),
    "c3-int8k-int4v-srft": (synth.config(3, B=2, T=1024, rotation="srft"), [1024, 700]),
    "c4-int2-srft": (synth.config(4, B=2, T=512, rotation="srft"), [512, 65]),
    "c5-fp4-srft-bf16": (synth.config(5, B=2, T=512, rotation="srft"), [512, 129]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_decode_matches_oracle(name):
    c, seq = CASES[name]
    print(f"[decode] case {name}", flush=True)
    s, r16, p, gcache, k, v = _filled(c, seq)
    q = synth.queries(c)
    out = kvq.decode_attn(p, gcache, dev_bits(q), seq)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    oc = oracle_view_of_gpu(c, gcache)
    ref, _ = attention.decode_attention(oc, q, c["dtype"], np.array(seq), c["rotation"], s, r16)
    rows = [(b, hq) for b in range(c["B"]) for hq in range(c["Hq"]) if seq[b] > 0]
    _check_rows(got, ref, rows, name)
    for b in range(c["B"]):
        if seq[b] == 0:
            assert not got[b].any()


def test_dense_baseline_matches_oracle():
    c = synth.config(2, B=2, T=640, keep=True)
    seq = [640, 400]
    print("[decode-dense]", flush=True)
    k = synth.kv_all(c, 0, 0, c["T"])
    v = synth.kv_all(c, 1, 0, c["T"])
    q = synth.queries(c)
    p = kvq.params_from_config(c)
    out = kvq.decode_attn_dense(p, dev_bits(k), dev_bits(v), dev_bits(q), seq)
    torch.cuda.synchronize()
    ref = attention.dense_attention(k, v, q, "f16", np.array(seq))
    rows = [(b, hq) for b in range(c["B"]) for hq in range(c["Hq"])]
    _check_rows(out.cpu().numpy(), ref, rows, "dense")


@pytest.fixture(scope="module")
def certified():
    c = synth.config(3, B=2, T=4096)
    seq = [4096, 4019]
    s, r16, p, gcache, k, v = _filled(c, seq)
    q = synth.queries(c)
    return c, seq, s, p, gcache, q


def test_error_bound_flags(certified):
    c, seq, s, p, gcache, q = certified
    print("[bound]", flush=True)
    bnd, fl = kvq.error_bound(p, gcache, dev_bits(q), seq, c["tau"])
    torch.cuda.synchronize()
    oc = oracle_view_of_gpu(c, gcache)
    # descriptors describe every appended token (all T of them), the bound uses seq_len
    desc = bound.block_descriptors(oc, c["dtype"], c["rotation"], s)
    ob, of = bound.error_bound(desc, q, c["dtype"], np.array(seq), c["tau"])
    assert np.array_equal(fl.cpu().numpy(), of), "flags differ from the oracle's"
    gb = bnd.cpu().numpy()
    assert np.all(gb >= ob * (1 - 1e-6)) and np.all(gb <= ob * (1 + 2.0 ** -8) + 1e-7)
    planted = set()
    for b in range(c["B"]):
        for h in range(c["Hkv"]):
            for blk, off in synth.planted(c, b, h):
                if blk * 64 + off < seq[b]:
                    planted.add((b, h, blk))
    assert set(map(tuple, np.argwhere(fl.cpu().numpy()))) == planted


@pytest.mark.parametrize("mode", ["flags", "none", "all"])
def test_certified_decode(certified, mode):
    c, seq, s, p, gcache, q = certified
    print(f"[cert] {mode}", flush=True)
    qd = dev_bits(q)
    if mode == "flags":
        _, fl = kvq.error_bound(p, gcache, qd, seq, c["tau"])
    elif mode == "all":
        _, fl = kvq.error_bound(p, gcache, qd, seq, 0.0)
    else:
        fl = None
    out, cert = kvq.decode_attn(p, gcache, qd, seq, flags=fl, certificate=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    oc = oracle_view_of_gpu(c, gcache)
    fln = None if fl is None else fl.cpu().numpy()
    ref, mass = attention.decode_attention(oc, q, c["dtype"], np.array(seq), c["rotation"], s, flags=fln)
    rows = [(b, hq) for b in range(c["B"]) for hq in range(c["Hq"])]
    _check_rows(got, ref, rows, f"cert-{mode}")
    dense = attention.dense_attention(oc.k_orig, oc.v_orig, q, c["dtype"], np.array(seq))
    # the certificate bounds the quantization error: exact attention over the quantized
    # cache (flagged blocks exact) vs dense attention over the originals
    err = np.linalg.norm(ref - dense, axis=-1)
    E = cert.cpu().numpy()
    assert np.all(err <= E), "certificate must bound the error to dense attention"
    desc = bound.block_descriptors(oc, c["dtype"], c["rotation"], s)
    E_or = bound.certificate(desc, q, c["dtype"], np.array(seq), fln, mass)
    # the library rounds its descriptors outward (x(1 + 2^-10) plus a rotation slack), so its
    # certificate sits just above the oracle's exact one
    assert np.all(E >= E_or * (1 - 1e-5)), "certificate below the oracle's"
    assert np.all(E <= E_or * (1 + 2.0 ** -7) + 1e-9), "certificate far above the oracle's"
    if mode == "all":
        assert not E.any()
        assert attention.row_rel_err(got, dense).max() <= TOL


@pytest.mark.parametrize("B,T", [(1, 16384), (2, 8192)])
def test_split_merge_repeatable(B, T):
    """Many splits, many calls on one workspace, alternating between two queries: the last
    split workgroup must see every other split's record of *this* call (a record left from
    the previous call, made with the other query, would show as a gross error) and must
    leave the arrival counters at zero (the next call merges again).  Chunks are shared out
    at run time, so calls differ at the level of the fp16 probabilities, within the bar."""
    c = synth.config(2, B=B, T=T)
    seq = [T] * B
    print(f"[decode] merge repeatable B={B} T={T}", flush=True)
    s, r16, p, gcache, k, v = _filled(c, seq)
    qs = [synth.queries(c), synth.queries(synth.config(1, B=B, Hq=c["Hq"]))]
    ws = kvq.workspace(p)
    assert kvq.decode_splits(p, seq) >= 4
    oc = oracle_view_of_gpu(c, gcache)
    refs = [attention.decode_attention(oc, q, c["dtype"], np.array(seq), c["rotation"], s, r16)[0] for q in qs]
    qd = [dev_bits(q) for q in qs]
    outs = [torch.empty((B, c["Hq"], 128), dtype=torch.float32, device="cuda") for _ in range(100)]
    for i in range(100):
        kvq.decode_attn(p, gcache, qd[i % 2], seq, ws=ws, out=outs[i])
    torch.cuda.synchronize()
    worst = max(float(attention.row_rel_err(outs[i].cpu().numpy(), refs[i % 2]).max()) for i in range(100))
    print(f"[decode] merge repeatable: worst row rel err over 100 alternating calls {worst:.2e}", flush=True)
    assert worst <= TOL


def _prefix_view(p_small, big):
    """A cache object for the first sequences of `big`: every buffer is laid out
    [stream][...] with stream = b * Hkv + h, so the first B' sequences are each buffer's
    prefix, and the view's buffers are prefixes of the big cache's (no copy)."""
    v = kvq.Cache(p_small, signs=big.signs, rot_f16=big.rot_f16)
    for n, t in v.bufs.items():
        if t is not None:
            v.bufs[n] = big.bufs[n][: t.numel()]
    return v


@pytest.mark.parametrize("cfg", [2, 3])
def test_split_count_invariance(cfg):
    """One sequence decoded alone (8 splits per unit) and as the first of 16 (2 splits):
    the split count changes only the fp32 order of the merge, so the two outputs agree far
    inside the bar, both meet the oracle, and the certified cache's flags and certificates
    agree too.  The data is appended once, through the one-sequence view."""
    T = 8192
    c1 = synth.config(cfg, B=1, T=T)
    c16 = synth.config(cfg, B=16, T=T)
    print(f"[decode] split-count invariance, config {cfg}", flush=True)
    s, r16, s_dev, r_dev = setup_rotation(c1)
    p16, g16 = make_gpu_cache(c16, s_dev, r_dev)
    p1 = kvq.params_from_config(c1)
    g1 = _prefix_view(p1, g16)
    k = synth.kv_all(c1, 0, 0, T)
    v = synth.kv_all(c1, 1, 0, T)
    kvq.append(p1, g1, dev_bits(k), dev_bits(v), [0])
    seq1, seq16 = [T], [T] + [0] * 15
    assert kvq.decode_splits(p1, seq1) == 8 and kvq.decode_splits(p16, seq16) == 2
    q1 = synth.queries(c1)
    q16 = np.zeros((16,) + q1.shape[1:], dtype=q1.dtype)
    q16[0] = q1[0]
    cert = cfg == 3
    if cert:
        _, f1 = kvq.error_bound(p1, g1, dev_bits(q1), seq1, c1["tau"])
        _, f16 = kvq.error_bound(p16, g16, dev_bits(q16), seq16, c1["tau"])
        o1, e1 = kvq.decode_attn(p1, g1, dev_bits(q1), seq1, flags=f1, certificate=True)
        o16, e16 = kvq.decode_attn(p16, g16, dev_bits(q16), seq16, flags=f16, certificate=True)
    else:
        o1 = kvq.decode_attn(p1, g1, dev_bits(q1), seq1)
        o16 = kvq.decode_attn(p16, g16, dev_bits(q16), seq16)
    torch.cuda.synchronize()
    a1, a16 = o1.cpu().numpy()[0], o16.cpu().numpy()[0]
    diff = float(attention.row_rel_err(a16[None], a1[None]).max())
    print(f"[decode] 8 vs 2 splits: max row rel difference {diff:.2e}", flush=True)
    assert diff <= 1e-4
    assert not o16.cpu().numpy()[1:].any(), "empty sequences give zero rows"
    oc = oracle_view_of_gpu(c1, g1)
    fln = None
    if cert:
        fln = f1.cpu().numpy()
        assert np.array_equal(fln[0], f16.cpu().numpy()[0])
    ref, _ = attention.decode_attention(oc, q1, c1["dtype"], np.array(seq1), c1["rotation"], s, r16, flags=fln)
    rows = [(0, hq) for hq in range(c1["Hq"])]
    _check_rows(o1.cpu().numpy(), ref, rows, "8 splits")
    _check_rows(o16.cpu().numpy()[:1], ref, rows, "2 splits")
    if cert:
        E1, E16 = e1.cpu().numpy()[0], e16.cpu().numpy()[0]
        assert np.allclose(E1, E16, rtol=1e-5, atol=1e-9), "certificates differ between split counts"
        assert not e16.cpu().numpy()[1:].any()


def test_fp4_every_scale_code():
    """FP4 keys and values over every E4M3 scale code 0x00..0x7E (subnormal, normal, the largest,
    448) and random E2M1 nibbles, written straight into the cache bytes: the decode reads the
    scales through the hardware fp8 conversion (keys) and the fp16 bit form (values), the oracle
    by the E4M3 definition; attention over the same bytes within the bar."""
    c = synth.config(5, B=2, Hq=4, Hkv=1, T=1024, dtype="f16")
    s, r16, s_dev, r_dev = setup_rotation(c)
    p, gcache = make_gpu_cache(c, s_dev, r_dev)
    oc = codec.Cache(c["B"], c["Hkv"], c["T"], "fp4", "fp4", c["k_group"], c["v_group"])
    rng = np.random.default_rng(2024)
    oc.k_codes[...] = rng.integers(0, 256, size=oc.k_codes.shape, dtype=np.uint8)
    oc.v_codes[...] = rng.integers(0, 256, size=oc.v_codes.shape, dtype=np.uint8)
    oc.k_meta[...] = (np.arange(oc.k_meta.size) % 0x7F).reshape(oc.k_meta.shape).astype(np.uint8)
    oc.v_meta[...] = ((np.arange(oc.v_meta.size) * 5) % 0x7F).reshape(oc.v_meta.shape).astype(np.uint8)
    assert set(np.unique(oc.k_meta)) == set(range(0x7F)) and set(np.unique(oc.v_meta)) == set(range(0x7F))
    for name in ("k_codes", "k_meta", "v_codes", "v_meta"):
        gcache.bufs[name].copy_(torch.from_numpy(getattr(oc, name).reshape(-1)))
    # a small query keeps the logits moderate (keys reach 6 x 448 per channel)
    q = synth.to_f16_bits(0.02 * rng.standard_normal((c["B"], c["Hq"], 128)))
    seq = [1024, 777]
    out = kvq.decode_attn(p, gcache, dev_bits(q), seq)
    torch.cuda.synchronize()
    ref, _ = attention.decode_attention(oc, q, "f16", np.array(seq), c["rotation"], s, r16)
    rows = [(b, hq) for b in range(c["B"]) for hq in range(c["Hq"])]
    _check_rows(out.cpu().numpy(), ref, rows, "fp4-every-scale-code")
