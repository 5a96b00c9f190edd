"""GPU parity at the full sizes of the five workloads, in the launch configuration bench.py uses.

Each test appends the whole cache of one workload through the C ABI (C4 fills a
seeded sample of its 64 sequences with data and leaves the rest zero, so the
launches still cover the full shape while the host only generates what the
oracle checks), then decodes every sequence at full context.  The oracle checks
what it can afford one by one:

* packed codes and metadata, bit for bit, on sampled (sequence, kv head) streams
  (a one-stream oracle cache appended with the same tokens);
* attention rows within 2e-3 (per-row max relative error): all 512 rows of the
  GQA workload, 256 sampled rows of the others, against the oracle's fp64
  attention over the library's own packed bytes;
* for the certified workload, the block flags and the certificate of the
  sampled sequences.
"""
import numpy as np
import pytest
import torch

import bit_kv_cache_append_amd as kvq
import synth
from oracle import attention, bound, codec
from gpu_harness import dev_bits, make_gpu_cache, make_oracle_cache, setup_rotation

pytestmark = pytest.mark.gpu
TOL = 2e-3
WORKERS = 16


def _log(msg):
    print(f"[fullsize] {msg}", flush=True)


def _stream_bytes_match(c, gcache, k, v, b, h, s, r16, clip=None):
    """Oracle append of stream (b, h) alone (all T tokens) vs the library's bytes of that stream."""
    one = synth.config(c["cfg"], **{**c, "B": 1, "Hkv": 1, "Hq": 1})
    oc = make_oracle_cache(one)
    ck = cv = None
    if clip is not None:
        ck, cv = clip[0][h:h + 1], clip[1][h:h + 1]
    codec.append(oc, k[None, None], v[None, None], np.array([0]), c["dtype"], c["rotation"], s, r16,
                 clip_k=ck, clip_v=cv, scale_mode=c["scale_mode"])
    for name in ("k_codes", "k_meta", "v_codes", "v_meta"):
        want = getattr(oc, name)[0, 0]
        got = gcache.bufs[name].view(c["B"], c["Hkv"], -1)[b, h].cpu().numpy().reshape(want.shape)
        if not np.array_equal(got, want):
            bad = np.argwhere(got != want)
            raise AssertionError(f"stream ({b}, {h}) {name}: {len(bad)} bytes differ, first at {bad[:3].tolist()}")


def _oracle_view(c, gcache, bs):
    """An oracle cache holding the library's bytes of sequences bs (all kv heads)."""
    sub = synth.config(c["cfg"], **{**c, "B": len(bs)})
    oc = make_oracle_cache(sub)
    full = make_oracle_cache(synth.config(c["cfg"], **{**c, "B": 1}))  # per-sequence shapes
    for name in ("k_codes", "k_meta", "v_codes", "v_meta"):
        arr = gcache.bufs[name].view(c["B"], -1)
        for i, b in enumerate(bs):
            getattr(oc, name)[i] = arr[b].cpu().numpy().reshape(getattr(full, name).shape[1:])
    if c["keep"]:
        for name in ("k_orig", "v_orig"):
            arr = gcache.bufs[name].view(torch.int16).view(c["B"], c["Hkv"], c["T"], 128)
            for i, b in enumerate(bs):
                getattr(oc, name)[i] = arr[b].cpu().numpy().view(np.uint16)
    return oc


def _rows_check(got, ref, rows, tag):
    err = attention.row_rel_err(got, ref)
    worst = max(err[i, hq] for i, hq in rows)
    _log(f"{tag}: {len(rows)} rows, max row rel err {worst:.3e}")
    assert worst <= TOL, f"{tag}: max row rel err {worst:.3e}"


def test_c2_gqa_int4_bench_shape():
    """B=16 Hq=32 Hkv=8 T=8192: context append, 4096-token prefill append, decode (bench's calls)."""
    c = synth.config(2)
    B, Hq, H, T, P = c["B"], c["Hq"], c["Hkv"], c["T"], c["prefill"]
    _log("c2: generating inputs")
    k = synth.kv_all(c, 0, 0, T, workers=WORKERS, start_method="spawn")
    v = synth.kv_all(c, 1, 0, T, workers=WORKERS, start_method="spawn")
    q = synth.queries(c)
    s, r16, s_dev, r_dev = setup_rotation(c)
    p, gcache = make_gpu_cache(c, s_dev, r_dev)
    kvq.append(p, gcache, dev_bits(k[:, :, :T - P]), dev_bits(v[:, :, :T - P]), [0] * B)
    kvq.append(p, gcache, dev_bits(k[:, :, T - P:]), dev_bits(v[:, :, T - P:]), [T - P] * B)
    ws = kvq.workspace(p)
    out = kvq.decode_attn(p, gcache, dev_bits(q), [T] * B, ws=ws)
    torch.cuda.synchronize()
    # the launch configuration bench.py times: 2 splits x 8 kv heads x 16 sequences = 256 workgroups
    assert kvq.decode_splits(p, [T] * B) == 2
    _log("c2: bytes of sampled streams")
    for b, h in ((0, 0), (5, 3), (10, 7), (15, 4)):
        _stream_bytes_match(c, gcache, k[b, h], v[b, h], b, h, s, r16)
    _log("c2: attention, all rows")
    oc = _oracle_view(c, gcache, list(range(B)))
    ref, _ = attention.decode_attention(oc, q, c["dtype"], np.full(B, T), c["rotation"], s)
    _rows_check(out.cpu().numpy(), ref, [(b, hq) for b in range(B) for hq in range(Hq)], "c2")


def test_c3_certified_full():
    """B=32 T=32768, int8 K / int4 V per token, fp16 copy; bound, flags, certified decode."""
    c = synth.config(3)
    B, Hq, H, T = c["B"], c["Hq"], c["Hkv"], c["T"]
    _log("c3: generating inputs")
    k = synth.kv_all(c, 0, 0, T, workers=WORKERS, start_method="spawn")
    v = synth.kv_all(c, 1, 0, T, workers=WORKERS, start_method="spawn")
    q = synth.queries(c)
    s, r16, s_dev, r_dev = setup_rotation(c)
    p, gcache = make_gpu_cache(c, s_dev, r_dev)
    kvq.append(p, gcache, dev_bits(k), dev_bits(v), [0] * B)
    seq = [T] * B
    qd = dev_bits(q)
    bnd, fl = kvq.error_bound(p, gcache, qd, seq, c["tau"])
    out, cert = kvq.decode_attn(p, gcache, qd, seq, flags=fl, certificate=True)
    torch.cuda.synchronize()
    fl_all = fl.cpu().numpy()
    _log(f"c3: {int(fl_all.sum())} of {fl_all.size} blocks flagged")
    _log("c3: bytes of sampled streams")
    for b, h in ((0, 0), (17, 5), (31, 7)):
        _stream_bytes_match(c, gcache, k[b, h], v[b, h], b, h, s, r16)
    del k, v
    bs = [0, 4, 9, 13, 18, 22, 27, 31]
    oc = _oracle_view(c, gcache, bs)
    qs = q[bs]
    seq_s = np.full(len(bs), T)
    _log("c3: descriptors and flags of sampled sequences")
    desc = bound.block_descriptors(oc, c["dtype"], c["rotation"], s)
    _, of = bound.error_bound(desc, qs, c["dtype"], seq_s, c["tau"])
    assert np.array_equal(fl_all[bs], of), "flags differ from the oracle's"
    planted = {(i, h, blk) for i, b in enumerate(bs) for h in range(H) for blk, _ in synth.planted(c, b, h)}
    assert set(map(tuple, np.argwhere(fl_all[bs]))) == planted
    _log("c3: certified attention of sampled sequences")
    ref, mass = attention.decode_attention(oc, qs, c["dtype"], seq_s, c["rotation"], s, flags=fl_all[bs])
    got = out.cpu().numpy()[bs]
    _rows_check(got, ref, [(i, hq) for i in range(len(bs)) for hq in range(Hq)], "c3")
    E = cert.cpu().numpy()[bs]
    E_or = bound.certificate(desc, qs, c["dtype"], seq_s, fl_all[bs], mass)
    assert np.all(E >= E_or * (1 - 1e-5)) and np.all(E <= E_or * (1 + 2.0 ** -7) + 1e-9)
    dense = attention.dense_attention(oc.k_orig, oc.v_orig, qs, c["dtype"], seq_s)
    assert np.all(np.linalg.norm(ref - dense, axis=-1) <= E), "certificate must bound the error"


def test_c4_int2_dense_full_shape():
    """B=64 T=32768, int2 g32 with dense rotation and clipping; 8 sequences hold data, the rest zeros."""
    c = synth.config(4)
    B, Hq, H, T = c["B"], c["Hq"], c["Hkv"], c["T"]
    bs = [0, 9, 18, 27, 36, 45, 54, 63]
    s, r16, s_dev, r_dev = setup_rotation(c)
    p, gcache = make_gpu_cache(c, s_dev, r_dev)
    ck = np.stack([synth.calibration(c, 0, h) for h in range(H)])
    cv = np.stack([synth.calibration(c, 1, h) for h in range(H)])
    tk, tv = kvq.calibrate_clip(p, gcache, dev_bits(ck), dev_bits(cv), ratio=c["clip_ratio"])
    gcache.clip_k, gcache.clip_v = tk, tv
    host_clip = (codec.calibrate_clip(ck, c["dtype"], c["rotation"], s, r16, c["clip_ratio"]),
                 codec.calibrate_clip(cv, c["dtype"], c["rotation"], s, r16, c["clip_ratio"]))
    torch.cuda.synchronize()
    assert np.array_equal(tk.cpu().numpy(), host_clip[0]) and np.array_equal(tv.cpu().numpy(), host_clip[1])
    _log("c4: generating the sampled sequences")
    kd = torch.zeros((B, H, T, 128), dtype=torch.int16, device="cuda")
    vd = torch.zeros_like(kd)
    ks, vs = {}, {}
    for b in bs:
        ks[b] = np.stack([synth.kv_slice(c, 0, b, h, 0, T) for h in range(H)])
        vs[b] = np.stack([synth.kv_slice(c, 1, b, h, 0, T) for h in range(H)])
        kd[b] = dev_bits(ks[b])
        vd[b] = dev_bits(vs[b])
    kvq.append(p, gcache, kd, vd, [0] * B)
    del kd, vd
    q = synth.queries(c)
    out = kvq.decode_attn(p, gcache, dev_bits(q), [T] * B)
    torch.cuda.synchronize()
    _log("c4: bytes of sampled streams")
    for b, h in ((0, 0), (27, 3), (63, 7)):
        _stream_bytes_match(c, gcache, ks[b][h], vs[b][h], b, h, s, r16, clip=host_clip)
    # an all-zero sequence: zero codes, zero scales and offsets
    for name in ("k_codes", "k_meta", "v_codes", "v_meta"):
        assert not gcache.bufs[name].view(B, -1)[1].any().item(), f"zero sequence {name}"
    _log("c4: attention of sampled sequences")
    oc = _oracle_view(c, gcache, bs)
    ref, _ = attention.decode_attention(oc, q[bs], c["dtype"], np.full(len(bs), T), c["rotation"], s, r16)
    _rows_check(out.cpu().numpy()[bs], ref, [(i, hq) for i in range(len(bs)) for hq in range(Hq)], "c4")


def test_c5_fp4_search_full():
    """B=8 T=131072, FP4 E2M1 with searched E4M3 block scales, bf16 Student-t inputs."""
    c = synth.config(5)
    B, Hq, H, T = c["B"], c["Hq"], c["Hkv"], c["T"]
    _log("c5: generating inputs")
    k = synth.kv_all(c, 0, 0, T, workers=WORKERS, start_method="spawn")
    v = synth.kv_all(c, 1, 0, T, workers=WORKERS, start_method="spawn")
    q = synth.queries(c)
    s, r16, s_dev, r_dev = setup_rotation(c)
    p, gcache = make_gpu_cache(c, s_dev, r_dev)
    kvq.append(p, gcache, dev_bits(k), dev_bits(v), [0] * B)
    out = kvq.decode_attn(p, gcache, dev_bits(q), [T] * B)
    torch.cuda.synchronize()
    _log("c5: bytes of sampled streams")
    for b, h in ((0, 0), (7, 6)):
        _stream_bytes_match(c, gcache, k[b, h], v[b, h], b, h, s, r16)
    del k, v
    _log("c5: attention, all 256 rows")
    oc = _oracle_view(c, gcache, list(range(B)))
    ref, _ = attention.decode_attention(oc, q, c["dtype"], np.full(B, T), c["rotation"], s)
    _rows_check(out.cpu().numpy(), ref, [(b, hq) for b in range(B) for hq in range(Hq)], "c5")
