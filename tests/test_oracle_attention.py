"""Pins for oracle/attention.py and oracle/bound.py.

Attention is checked against torch's scaled_dot_product_attention (a library
routine) on the decoded cache, against rotation invariance, and against the
special cases T = 1, identical keys and tau = 0.  The bound is checked to bound
what it claims to bound, on the certified synthetic workload.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import attention, bound, codec, numerics as nx, rotation as rot


def _cache(fk, fv, B=2, H=2, T=256, gk=32, gv=32, keep=False):
    return codec.Cache(B, H, T, fk, fv, gk, gv, keep_fp16_copy=keep)


def _fill(cache, rng, dtype="f16", rotation="sign_fwht", signs=None, n=None, scale=1.0):
    n = cache.Tmax if n is None else n
    k = (rng.standard_normal((cache.B, cache.H, n, 128)) * scale).astype(np.float32)
    v = (rng.standard_normal((cache.B, cache.H, n, 128)) * scale).astype(np.float32)
    kb, vb = synth.to_bits(k, dtype), synth.to_bits(v, dtype)
    codec.append(cache, kb, vb, np.zeros(cache.B, int), dtype, rotation, signs)
    return kb, vb


def _sdpa(q, k, v, G):
    """torch SDPA in fp64 with GQA by repeating kv heads; q [Hq,d], k/v [H,T,d]."""
    kq = torch.from_numpy(np.repeat(k, G, axis=0))
    vq = torch.from_numpy(np.repeat(v, G, axis=0))
    qq = torch.from_numpy(q)[:, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qq, kq, vq)
    return o[:, 0, :].numpy()


@pytest.mark.parametrize("fk,fv,rotation", [("int8", "int4", "none"), ("int4", "int4", "sign_fwht"),
                                            ("fp4", "int2", "sign_fwht")])
def test_decode_matches_sdpa_on_decoded_cache(fk, fv, rotation):
    rng = np.random.default_rng(20)
    s = np.where(rng.integers(0, 2, 128) == 1, 1, -1)
    cache = _cache(fk, fv, B=2, H=2, T=256)
    _fill(cache, rng, rotation=rotation, signs=s)
    Hq = 8
    q = synth.to_bits(rng.standard_normal((2, Hq, 128)), "f16")
    seq = np.array([256, 131])
    out, _ = attention.decode_attention(cache, q, "f16", seq, rotation, s)
    R = rot.rotation_matrix_f64(rotation, s)
    qf = q.view(np.float16).astype(np.float64)
    for b in range(2):
        T = seq[b]
        kh = np.stack([codec.decode_k(cache, b, h, 0, T) @ R for h in range(2)])  # back to original basis
        vh = np.stack([codec.decode_v(cache, b, h, 0, T) @ R for h in range(2)])
        ref = _sdpa(qf[b], kh, vh, Hq // 2)
        assert np.allclose(out[b], ref, rtol=1e-10, atol=1e-12)


def test_single_token_returns_value():
    rng = np.random.default_rng(21)
    s = np.where(rng.integers(0, 2, 128) == 1, 1, -1)
    cache = _cache("int4", "int4", B=1, H=1, T=64)
    _fill(cache, rng, signs=s, n=1)
    q = synth.to_bits(rng.standard_normal((1, 2, 128)), "f16")
    out, mass = attention.decode_attention(cache, q, "f16", np.array([1]), "sign_fwht", s)
    R = rot.rotation_matrix_f64("sign_fwht", s)
    v0 = R.T @ codec.decode_v(cache, 0, 0, 0, 1)[0]
    assert np.allclose(out[0, 0], v0) and np.allclose(out[0, 1], v0)
    assert np.allclose(mass[0, :, 0], 1.0)


def test_identical_keys_average_values():
    rng = np.random.default_rng(22)
    s = np.where(rng.integers(0, 2, 128) == 1, 1, -1)
    cache = _cache("int8", "int4", B=1, H=1, T=128)
    k = np.repeat(rng.standard_normal((1, 1, 1, 128)), 100, axis=2)
    v = rng.standard_normal((1, 1, 100, 128))
    codec.append(cache, synth.to_bits(k, "f16"), synth.to_bits(v, "f16"), np.array([0]), "f16", "sign_fwht", s)
    q = synth.to_bits(rng.standard_normal((1, 1, 128)), "f16")
    out, _ = attention.decode_attention(cache, q, "f16", np.array([100]), "sign_fwht", s)
    R = rot.rotation_matrix_f64("sign_fwht", s)
    assert np.allclose(out[0, 0], R.T @ codec.decode_v(cache, 0, 0, 0, 100).mean(axis=0))


def test_all_flagged_is_dense_attention():
    # "Runtime-Certified ...", Contributions: the fallback returns the dense result exactly
    rng = np.random.default_rng(23)
    s = np.where(rng.integers(0, 2, 128) == 1, 1, -1)
    cache = _cache("int8", "int4", B=2, H=2, T=192, gk=128, gv=128, keep=True)
    _fill(cache, rng, signs=s)
    q = synth.to_bits(rng.standard_normal((2, 4, 128)), "f16")
    seq = np.array([192, 100])
    flags = np.ones((2, 2, 3), np.uint8)
    out, _ = attention.decode_attention(cache, q, "f16", seq, "sign_fwht", s, flags=flags)
    dense = attention.dense_attention(cache.k_orig, cache.v_orig, q, "f16", seq)
    assert np.allclose(out, dense, rtol=1e-12, atol=1e-14)
    qf = q.view(np.float16).astype(np.float64)
    for b in range(2):
        T = seq[b]
        k = cache.k_orig[b, :, :T].view(np.float16).astype(np.float64)
        v = cache.v_orig[b, :, :T].view(np.float16).astype(np.float64)
        assert np.allclose(dense[b], _sdpa(qf[b], k, v, 2), rtol=1e-10, atol=1e-12)


def test_value_only_flags_take_the_original_values():
    # "Runtime-Certified ...", Methodology section 3, rung 2: a value-promoted block (flag 2)
    # reads its values from the originals.  Every token carries the same value vector, so
    # the output is that vector whatever the logits: the original with flag 2, its int4
    # reconstruction without.
    rng = np.random.default_rng(24)
    T = 192
    cache = _cache("int8", "int4", B=1, H=1, T=T, gk=128, gv=32, keep=True)
    k = rng.standard_normal((1, 1, T, 128))
    v = np.repeat(rng.standard_normal((1, 1, 1, 128)), T, axis=2)
    vb = synth.to_bits(v, "f16")
    codec.append(cache, synth.to_bits(k, "f16"), vb, np.zeros(1, int), "f16", "none")
    q = synth.to_bits(rng.standard_normal((1, 2, 128)), "f16")
    v16 = vb[0, 0, 0].view(np.float16).astype(np.float64)
    out2, _ = attention.decode_attention(cache, q, "f16", np.array([T]), "none", flags=np.full((1, 1, 3), 2, np.uint8))
    out0, _ = attention.decode_attention(cache, q, "f16", np.array([T]), "none")
    assert np.abs(out2[0] - v16).max() <= 1e-12 * np.abs(v16).max()
    assert np.abs(out0[0] - v16).max() > 1e-3  # int4 reconstruction error: the case tells them apart


def test_value_only_flags_keep_the_quantized_logits():
    # Values on the int4 grid (each 32-channel group holds +-7/8, entries k/8): their codes
    # are exact, so a value-promoted block (flag 2) gives the same output as no promotion,
    # while a full promotion (flag 1) also takes exact keys and gives dense attention.
    rng = np.random.default_rng(25)
    T = 192
    cache = _cache("int8", "int4", B=1, H=1, T=T, gk=128, gv=32, keep=True)
    k = rng.standard_normal((1, 1, T, 128))
    v = rng.integers(-7, 8, size=(1, 1, T, 128)) / 8.0
    v[..., ::32] = 7.0 / 8.0
    kb, vb = synth.to_bits(k, "f16"), synth.to_bits(v, "f16")
    codec.append(cache, kb, vb, np.zeros(1, int), "f16", "none")
    assert np.array_equal(codec.decode_v(cache, 0, 0, 0, T), v[0, 0])
    q = synth.to_bits(3.0 * rng.standard_normal((1, 2, 128)), "f16")
    seq = np.array([T])
    flag = lambda f: np.full((1, 1, 3), f, np.uint8)
    out0, _ = attention.decode_attention(cache, q, "f16", seq, "none")
    out1, _ = attention.decode_attention(cache, q, "f16", seq, "none", flags=flag(1))
    out2, _ = attention.decode_attention(cache, q, "f16", seq, "none", flags=flag(2))
    out3, _ = attention.decode_attention(cache, q, "f16", seq, "none", flags=flag(3))
    dense = attention.dense_attention(cache.k_orig, cache.v_orig, q, "f16", seq)
    assert np.allclose(out2, out0, rtol=1e-12, atol=1e-15)
    assert np.allclose(out1, dense, rtol=1e-12, atol=1e-15) and np.array_equal(out3, out1)
    assert np.abs(out2 - dense).max() > 1e-4  # int8 key error moves the logits


@pytest.mark.parametrize("T,window,want", [
    (323, (1, 2), [1, 0, 0, 0, 1, 1]),   # 6 blocks, the last one partial
    (100, (1, 2), [1, 1]),               # window wider than the sequence
    (640, (0, 1), [0] * 9 + [1]),
    (640, (2, 0), [1, 1] + [0] * 8),
    (64, (0, 0), [0]),
    (0, (1, 1), []),
])
def test_window_blocks_examples(T, window, want):
    # "Search Your Block Floating Point Scales!": first and last blocks at full precision
    assert attention.window_blocks(T, *window).astype(int).tolist() == want


def test_window_covering_all_is_dense_attention():
    rng = np.random.default_rng(24)
    s = np.where(rng.integers(0, 2, 128) == 1, 1, -1)
    cache = _cache("int4", "int4", B=2, H=2, T=192)
    kb, vb = _fill(cache, rng, signs=s)
    q = synth.to_bits(rng.standard_normal((2, 4, 128)), "f16")
    seq = np.array([192, 70])
    out, _ = attention.decode_attention(cache, q, "f16", seq, "sign_fwht", s, window=(3, 0), originals=(kb, vb))
    dense = attention.dense_attention(kb, vb, q, "f16", seq)
    assert np.allclose(out, dense, rtol=1e-12, atol=1e-14)
    none, _ = attention.decode_attention(cache, q, "f16", seq, "sign_fwht", s, window=(0, 0), originals=(kb, vb))
    plain, _ = attention.decode_attention(cache, q, "f16", seq, "sign_fwht", s)
    assert np.array_equal(none, plain)


@pytest.mark.parametrize("fk,fv,dtype,rotation", [("int4", "int4", "f16", "sign_fwht"),
                                                  ("fp4", "fp4", "bf16", "sign_fwht"),
                                                  ("int2", "int2", "f16", "none")])
def test_window_matches_mixed_cache_sdpa(fk, fv, dtype, rotation):
    # sink block 0 and the two newest blocks exact, the middle decoded from codes: the same
    # attention as SDPA over one key/value matrix in the original basis that holds the
    # originals at those positions and the derotated decoded rows elsewhere
    rng = np.random.default_rng(25)
    s = np.where(rng.integers(0, 2, 128) == 1, 1, -1)
    cache = _cache(fk, fv, B=2, H=2, T=384)
    kb, vb = _fill(cache, rng, dtype=dtype, rotation=rotation, signs=s)
    Hq = 4
    q = synth.to_bits(rng.standard_normal((2, Hq, 128)), dtype)
    seq = np.array([323, 384])
    exact_ranges = {323: [(0, 64), (256, 323)], 384: [(0, 64), (256, 384)]}
    out, _ = attention.decode_attention(cache, q, dtype, seq, rotation, s, window=(1, 2), originals=(kb, vb))
    R = rot.rotation_matrix_f64(rotation, s)
    qf = nx.widen_input(q, dtype).astype(np.float64)
    for b in range(2):
        T = seq[b]
        k = np.stack([codec.decode_k(cache, b, h, 0, T) @ R for h in range(2)])
        v = np.stack([codec.decode_v(cache, b, h, 0, T) @ R for h in range(2)])
        for lo, hi in exact_ranges[T]:
            k[:, lo:hi] = nx.widen_input(kb[b, :, lo:hi], dtype)
            v[:, lo:hi] = nx.widen_input(vb[b, :, lo:hi], dtype)
        assert np.allclose(out[b], _sdpa(qf[b], k, v, Hq // 2), rtol=1e-10, atol=1e-12)


def test_row_rel_err_metric():
    ref = np.array([[1.0, -2.0, 0.5]])
    got = np.array([[1.0, -2.004, 0.5]])
    assert np.isclose(attention.row_rel_err(got, ref)[0], 0.002)


@pytest.fixture(scope="module")
def certified_small():
    c = synth.config(3, B=2, T=4096)
    k = synth.kv_all(c, 0, 0, c["T"])
    v = synth.kv_all(c, 1, 0, c["T"])
    s = synth.signs(c)
    cache = codec.Cache(c["B"], c["Hkv"], c["T"], c["k_fmt"], c["v_fmt"], c["k_group"], c["v_group"],
                        keep_fp16_copy=True)
    codec.append(cache, k, v, np.zeros(c["B"], int), c["dtype"], c["rotation"], s)
    q = synth.queries(c)
    seq = np.array([c["T"], c["T"] - 77])
    desc = bound.block_descriptors(cache, c["dtype"], c["rotation"], s, seq_len=seq)
    return c, cache, s, q, seq, desc


def test_descriptors_bound_per_token_errors(certified_small):
    c, cache, s, q, seq, desc = certified_small
    R = rot.rotation_matrix_f64("sign_fwht", s)
    for b in range(c["B"]):
        T = seq[b]
        for h in range(c["Hkv"]):
            k = nx.widen_input(cache.k_orig[b, h, :T], "f16").astype(np.float64)
            kh = codec.decode_k(cache, b, h, 0, T) @ R  # original basis
            v = nx.widen_input(cache.v_orig[b, h, :T], "f16").astype(np.float64)
            vh = codec.decode_v(cache, b, h, 0, T) @ R
            ek = np.linalg.norm(k - kh, axis=1)
            ev = np.linalg.norm(v - vh, axis=1)
            blk = np.arange(T) // 64
            assert np.all(ek <= desc[b, h, blk, 0] * (1 + 1e-12))
            assert np.all(ev <= desc[b, h, blk, 1] * (1 + 1e-12))
            assert np.allclose(np.maximum.reduceat(ek, np.arange(0, T, 64)), desc[b, h, :len(range(0, T, 64)), 0])
            # per-token logit error bounded by Delta_b (Cauchy-Schwarz)
            G = c["Hq"] // c["Hkv"]
            for g in range(G):
                qq = q[b, h * G + g].view(np.float16).astype(np.float64)
                dl = np.abs((k - kh) @ qq) / np.sqrt(128)
                assert np.all(dl <= np.linalg.norm(qq) / np.sqrt(128) * desc[b, h, blk, 0] * (1 + 1e-12))


def test_flags_match_planted_blocks(certified_small):
    c, cache, s, q, seq, desc = certified_small
    bd, fl = bound.error_bound(desc, q, "f16", seq, c["tau"])
    planted = set()
    for b in range(c["B"]):
        for h in range(c["Hkv"]):
            for blk, off in synth.planted(c, b, h):
                if blk * 64 + off < seq[b]:
                    planted.add((b, h, blk))
    got = set(map(tuple, np.argwhere(fl)))
    assert got == planted
    unpl = np.array([bd[i] for i in np.ndindex(bd.shape) if i not in planted])
    assert unpl.max() <= 0.7 * c["tau"]
    assert min(bd[i] for i in planted) >= 2 * c["tau"]
    _, none = bound.error_bound(desc, q, "f16", seq, np.inf)
    assert not none.any()
    _, allf = bound.error_bound(desc, q, "f16", seq, 0.0)
    assert allf[0].all() and allf[1, :, :63].all() and not allf[1, :, 63:].any()


@pytest.mark.parametrize("tau", [1e-2, np.inf])
def test_certificate_bounds_error(certified_small, tau):
    c, cache, s, q, seq, desc = certified_small
    _, fl = bound.error_bound(desc, q, "f16", seq, tau)
    out, mass = attention.decode_attention(cache, q, "f16", seq, "sign_fwht", s, flags=fl)
    dense = attention.dense_attention(cache.k_orig, cache.v_orig, q, "f16", seq)
    E = bound.certificate(desc, q, "f16", seq, fl, mass)
    err = np.linalg.norm(out - dense, axis=-1)
    assert np.all(err <= E)
    assert np.all(E > 0)


def test_corrupted_codes_escape_the_stored_certificate(certified_small):
    """What the certificate does not catch ("Runtime-Certified Bounded-Error Quantized
    Attention", Methodology sections 1-2: the descriptors are measured when a block is
    written).  A block's value codes and scales changed after the append leave the stored
    descriptors, hence the flags and the certificate, as they were, while the attention
    moves far beyond the certificate; descriptors measured again from the damaged block
    would flag it."""
    import copy
    c, cache, s, q, seq, desc = certified_small
    tau = 1e-2
    _, fl = bound.error_bound(desc, q, "f16", seq, tau)
    out, mass = attention.decode_attention(cache, q, "f16", seq, "sign_fwht", s, flags=fl)
    E = bound.certificate(desc, q, "f16", seq, fl, mass)
    G = c["Hq"] // c["Hkv"]
    # the unflagged block of (sequence 0, kv head 0) with the most attention mass (its heads summed)
    m0 = mass[0, :G].sum(axis=0)
    m0 = np.where(fl[0, 0] == 0, m0, -1.0)
    blk = int(np.argmax(m0[: seq[0] // 64]))
    bad = copy.deepcopy(cache)
    bad.v_codes[0, 0, blk] = 0x77  # every value code of the block's tile +7 (int4 nibbles) ...
    bad.v_meta[0, 0, blk].view(np.uint16)[...] = 0x3C00  # ... and every value scale 1.0 (fp16)
    _, fl2 = bound.error_bound(desc, q, "f16", seq, tau)
    out2, mass2 = attention.decode_attention(bad, q, "f16", seq, "sign_fwht", s, flags=fl2)
    E2 = bound.certificate(desc, q, "f16", seq, fl2, mass2)
    assert np.array_equal(fl2, fl) and np.array_equal(E2, E), "the stored descriptors decide flags and certificate"
    dense = attention.dense_attention(cache.k_orig, cache.v_orig, q, "f16", seq)
    err = np.linalg.norm(out2 - dense, axis=-1)
    assert np.all(err[0, :G] > 2 * E[0, :G]), "the damaged block's heads: error far beyond the certificate"
    rest = np.ones(err.shape, bool)
    rest[0, :G] = False
    assert np.all(err[rest] <= E[rest]), "every other row keeps its bound"
    # measured again from the damaged codes, the block's value error flags it
    desc2 = bound.block_descriptors(bad, c["dtype"], c["rotation"], s, seq_len=seq)
    assert desc2[0, 0, blk, 1] > 10 * desc[0, 0, blk, 1]
    _, fl3 = bound.error_bound(desc2, q, "f16", seq, tau)
    assert fl3[0, 0, blk] and not fl[0, 0, blk]
