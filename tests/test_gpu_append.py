"""GPU parity of kvq_append: packed codes and scales bit-exact against the oracle.

Covers every format, both rotations and none, fp16 and bf16 inputs, ragged
starts and lengths, appends split across calls, single-token appends, the fp16
copy and the per-block descriptors.
"""
import numpy as np
import pytest
import torch

import bit_kv_cache_append_amd as kvq
import synth
from oracle import bound, codec
from gpu_harness import (assert_bytes_equal, dev_bits, make_gpu_cache, make_oracle_cache, setup_rotation)

pytestmark = pytest.mark.gpu

CASES = {
    "int4-fwht-f16": synth.config(1, B=2, Hq=2, Hkv=2, T=256),
    "int4-g32-gqa": synth.config(2, B=2, Hq=8, Hkv=2, T=320),
    "int8k-int4v-cert": synth.config(3, B=2, Hq=8, Hkv=2, T=256, n_plant=2),
    "int2-dense": synth.config(4, B=2, Hq=8, Hkv=2, T=256),
    "int2-dense-bf16": synth.config(4, B=3, Hq=8, Hkv=2, T=320, dtype="bf16"),
    "int2-dense-noclip": synth.config(4, B=1, Hq=4, Hkv=2, T=192, no_clip=True),
    "fp4-search-bf16": synth.config(5, B=2, Hq=8, Hkv=2, T=256),
    "fp4-absmax": synth.config(5, B=2, Hq=8, Hkv=2, T=192, scale_mode="absmax"),
    "int4-g128-none": synth.config(1, B=2, Hq=2, Hkv=2, T=192, rotation="none", k_group=128, v_group=128),
    "int8-g32-int2-fwht": synth.config(2, B=1, Hq=4, Hkv=2, T=192, k_fmt="int8", v_fmt="int2"),
    "int4-bf16": synth.config(2, B=1, Hq=4, Hkv=2, T=128, dtype="bf16"),
    "fp4-f16-absmax": synth.config(5, B=1, Hq=4, Hkv=2, T=128, dtype="f16", scale_mode="absmax"),
    "fp4-f16-search": synth.config(5, B=1, Hq=4, Hkv=2, T=128, dtype="f16"),
    "fp4-offsets-bf16": synth.config(5, B=2, Hq=8, Hkv=2, T=256, scale_mode="offsets"),
    "fp4-offsets-dense-f16": synth.config(5, B=1, Hq=4, Hkv=2, T=192, dtype="f16", scale_mode="offsets",
                                          rotation="dense"),
    # SRFT ("When Quantization Is Free", Methodology sections 1-2): the Stockham FFT write side
    "int4-srft-f16": synth.config(1, B=2, Hq=2, Hkv=2, T=256, rotation="srft"),
    "int4-g16-fwht": synth.config(2, B=2, Hq=8, Hkv=2, T=256, k_group=16, v_group=16),
    "int4-g16-srft-bf16-cert": synth.config(2, B=2, Hq=8, Hkv=2, T=192, k_group=16, v_group=16, rotation="srft",
                                            dtype="bf16", keep=True),
    "int8k-int4v-srft-cert": synth.config(3, B=2, Hq=8, Hkv=2, T=256, n_plant=2, rotation="srft"),
    "int2-srft-bf16": synth.config(4, B=2, Hq=8, Hkv=2, T=256, dtype="bf16", rotation="srft"),
    "fp4-srft": synth.config(5, B=2, Hq=8, Hkv=2, T=192, rotation="srft"),
}


def _clip(c, p, gcache, s, r16):
    if (c["k_fmt"] != "int2" and c["v_fmt"] != "int2") or c.get("no_clip"):
        return None, None
    ck = np.stack([synth.calibration(c, 0, h) for h in range(c["Hkv"])])
    cv = np.stack([synth.calibration(c, 1, h) for h in range(c["Hkv"])])
    tk, tv = kvq.calibrate_clip(p, gcache, dev_bits(ck), dev_bits(cv), ratio=0.9)
    torch.cuda.synchronize()
    ok = codec.calibrate_clip(ck, c["dtype"], c["rotation"], s, r16, 0.9)
    ov = codec.calibrate_clip(cv, c["dtype"], c["rotation"], s, r16, 0.9)
    assert np.array_equal(tk.cpu().numpy(), ok), "clip thresholds (K) differ"
    assert np.array_equal(tv.cpu().numpy(), ov), "clip thresholds (V) differ"
    return (tk, tv), (ok, ov)


def _run(c, pieces):
    """Append the workload in `pieces` = [(start offsets per b, n)], on GPU and oracle."""
    s, r16, s_dev, r_dev = setup_rotation(c)
    p, gcache = make_gpu_cache(c, s_dev, r_dev)
    dev_clip, host_clip = _clip(c, p, gcache, s, r16)
    if dev_clip is not None:
        gcache.clip_k, gcache.clip_v = dev_clip if c["k_fmt"] == "int2" or c["v_fmt"] == "int2" else (None, None)
    oc = make_oracle_cache(c)
    for starts, n in pieces:
        k = np.stack([np.stack([synth.kv_slice(c, 0, b, h, starts[b], n) for h in range(c["Hkv"])])
                      for b in range(c["B"])])
        v = np.stack([np.stack([synth.kv_slice(c, 1, b, h, starts[b], n) for h in range(c["Hkv"])])
                      for b in range(c["B"])])
        kvq.append(p, gcache, dev_bits(k), dev_bits(v), starts)
        codec.append(oc, k, v, np.array(starts), c["dtype"], c["rotation"], s, r16,
                     None if host_clip is None or c["k_fmt"] != "int2" else host_clip[0],
                     None if host_clip is None or c["v_fmt"] != "int2" else host_clip[1], c["scale_mode"])
    torch.cuda.synchronize()
    return s, r16, p, gcache, oc


@pytest.mark.parametrize("name", list(CASES))
def test_append_full_bit_exact(name):
    c = CASES[name]
    print(f"[append] case {name}", flush=True)
    T = c["T"]
    s, r16, p, gcache, oc = _run(c, [([0] * c["B"], T)])
    assert_bytes_equal(oc, gcache, name)
    if c["keep"]:
        ko = gcache.bufs["k_orig"].cpu().numpy().view(np.uint16).reshape(oc.k_orig.shape)
        vo = gcache.bufs["v_orig"].cpu().numpy().view(np.uint16).reshape(oc.v_orig.shape)
        assert np.array_equal(ko, oc.k_orig) and np.array_equal(vo, oc.v_orig)
        seq = np.full(c["B"], T)
        want = bound.block_descriptors(oc, c["dtype"], c["rotation"], s, r16, seq_len=seq)
        got = gcache.bufs["blk_desc"].cpu().numpy().reshape(want.shape)
        assert np.all(got >= want), "descriptors must bound the exact errors"
        assert np.all(got <= want * (1 + 2.0 ** -8) + 1e-6 * np.abs(want).max()), "descriptors too loose"


@pytest.mark.parametrize("name", ["int4-g32-gqa", "int8k-int4v-cert", "fp4-search-bf16", "int2-dense",
                                  "int2-dense-bf16", "int4-srft-f16"])
def test_append_ragged_pieces(name):
    c = CASES[name]
    print(f"[append-ragged] case {name}", flush=True)
    B = c["B"]
    # sequences start at different offsets; pieces of 37, 100, 1 and 1 tokens
    base = [3, 64][:B] + [0] * max(0, B - 2)
    pieces, off = [], 0
    for n in (37, 100, 1, 1):
        pieces.append(([b0 + off for b0 in base], n))
        off += n
    s, r16, p, gcache, oc = _run(c, pieces)
    assert_bytes_equal(oc, gcache, name)


def test_append_rejects_out_of_range():
    c = CASES["int4-fwht-f16"]
    s, r16, s_dev, r_dev = setup_rotation(c)
    p, gcache = make_gpu_cache(c, s_dev, r_dev)
    k = torch.zeros((c["B"], c["Hkv"], 10, 128), dtype=torch.int16, device="cuda")
    with pytest.raises(kvq.KvqError):
        kvq.append(p, gcache, k, k, [c["T"] - 5, 0])
    assert not gcache.bufs["k_codes"].any()


def _edge_bits(shape, seed):
    """fp16 bit patterns mixing ordinary values with edge cases: subnormals, signed zeros,
    the largest finite values, all-zero vectors and vectors of one repeated value."""
    rng = np.random.default_rng(seed)
    x = synth.to_f16_bits(rng.standard_normal(shape))
    flat = x.reshape(-1, shape[-1])
    n = flat.shape[0]
    pick = lambda frac: rng.random(flat.shape) < frac
    sub = pick(0.05)  # subnormals of either sign
    flat[sub] = (rng.integers(1, 0x400, size=int(sub.sum())) | (rng.integers(0, 2, size=int(sub.sum())) << 15)).astype(np.uint16)
    big = pick(0.002)  # +-65504
    flat[big] = np.where(rng.random(int(big.sum())) < 0.5, 0x7BFF, 0xFBFF).astype(np.uint16)
    nz = pick(0.02)
    flat[nz] = 0x8000  # negative zero
    flat[rng.choice(n, size=max(1, n // 50), replace=False)] = 0  # whole zero vectors
    rows = rng.choice(n, size=max(1, n // 50), replace=False)
    flat[rows] = flat[rows, :1]  # one value repeated over the vector
    tiny = rng.choice(n, size=max(1, n // 50), replace=False)
    flat[tiny] = (rng.integers(1, 0x400, size=(len(tiny), shape[-1]))).astype(np.uint16)  # subnormal vectors
    return x


@pytest.mark.parametrize("name", ["int4-g32-gqa", "int8k-int4v-cert", "int4-g16-fwht", "fp4-f16-search",
                                  "int4-srft-f16"])
def test_append_edge_values_bit_exact(name):
    """fp16 edge cases (subnormals, signed zeros, +-65504, zero and constant vectors, vectors
    of subnormals) through the fast and generic append paths: codes, metadata, originals and
    descriptors as the oracle's."""
    c = CASES[name]
    print(f"[append] edge values {name}", flush=True)
    B, H, T = c["B"], c["Hkv"], c["T"]
    k = _edge_bits((B, H, T, 128), 11)
    v = _edge_bits((B, H, T, 128), 12)
    s, r16, s_dev, r_dev = setup_rotation(c)
    p, gcache = make_gpu_cache(c, s_dev, r_dev)
    oc = make_oracle_cache(c)
    kvq.append(p, gcache, dev_bits(k), dev_bits(v), [0] * B)
    torch.cuda.synchronize()
    codec.append(oc, k, v, np.zeros(B, int), c["dtype"], c["rotation"], s, r16, None, None, c["scale_mode"])
    assert_bytes_equal(oc, gcache, f"edge-{name}")
    if c["keep"]:
        want = bound.block_descriptors(oc, c["dtype"], c["rotation"], s, r16)
        got = gcache.bufs["blk_desc"].cpu().numpy().reshape(want.shape)
        assert np.all(got >= want) and np.all(got <= want * (1 + 2.0 ** -8) + 1e-6 * np.abs(want).max())
