"""Shared setup for the GPU parity tests: run a workload through libkvq and the oracle.

Inputs come from synth (seeded).  The library path runs only through the C ABI
(bit_kv_cache_append_amd); the oracle side never sees a library output except
where a test explicitly decodes the library's own packed bytes with the
oracle's unpacker (attention parity judged separately from code parity).
"""
import numpy as np
import torch

import bit_kv_cache_append_amd as kvq
import synth
from oracle import codec

FMT_ROW = {"int4": 64, "int8": 128, "int2": 32, "fp4": 64}


def dev_bits(a):
    return kvq.to_device_bits(a)


def setup_rotation(c):
    """(signs numpy, R16 as numpy float16 for the oracle, signs device, rot bits device)."""
    s = synth.signs(c)
    bits = synth.dense_rotation_f16(c) if c["rotation"] == "dense" else None
    s_dev = torch.from_numpy(s.copy()).cuda()
    r_dev = dev_bits(bits) if bits is not None else None
    r16 = bits.view(np.float16) if bits is not None else None
    return s, r16, s_dev, r_dev


def make_gpu_cache(c, s_dev, r_dev, clip=None):
    p = kvq.params_from_config(c)
    cache = kvq.Cache(p, signs=s_dev, rot_f16=r_dev,
                      clip_k=None if clip is None else clip[0], clip_v=None if clip is None else clip[1])
    return p, cache


def make_oracle_cache(c):
    return codec.Cache(c["B"], c["Hkv"], c["T"], c["k_fmt"], c["v_fmt"], c["k_group"], c["v_group"],
                       keep_fp16_copy=c["keep"])


def gpu_bytes(cache, name, shape):
    return cache.bufs[name].cpu().numpy().reshape(shape)


def oracle_view_of_gpu(c, gcache):
    """An oracle Cache object holding the library's bytes (for decoding them on the CPU)."""
    oc = make_oracle_cache(c)
    oc.k_codes[...] = gpu_bytes(gcache, "k_codes", oc.k_codes.shape)
    oc.k_meta[...] = gpu_bytes(gcache, "k_meta", oc.k_meta.shape)
    oc.v_codes[...] = gpu_bytes(gcache, "v_codes", oc.v_codes.shape)
    oc.v_meta[...] = gpu_bytes(gcache, "v_meta", oc.v_meta.shape)
    if c["keep"]:
        oc.k_orig[...] = gpu_bytes(gcache, "k_orig", (c["B"], c["Hkv"], c["T"], 128 * 2)).view(np.uint16)
        oc.v_orig[...] = gpu_bytes(gcache, "v_orig", (c["B"], c["Hkv"], c["T"], 128 * 2)).view(np.uint16)
    return oc


def assert_bytes_equal(oc, gcache, tag=""):
    for name in ("k_codes", "k_meta", "v_codes", "v_meta"):
        want = getattr(oc, name)
        got = gpu_bytes(gcache, name, want.shape)
        if not np.array_equal(got, want):
            bad = np.argwhere(got != want)
            i0 = tuple(bad[0][:-1])
            print(f"{tag} {name} first bad row {i0}:\n got  {got[i0].tolist()}\n want {want[i0].tolist()}", flush=True)
            raise AssertionError(f"{tag} {name}: {len(bad)} bytes differ, first at {bad[:5].tolist()} "
                                 f"got {got[tuple(bad[0])]} want {want[tuple(bad[0])]}")
