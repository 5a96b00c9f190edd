"""GPU parity at the full sizes of the five workloads, in the launch configuration bench.py uses.

Each workload's whole cache is appended through the C ABI (every sequence holds
seeded data) and decoded at full context.  The oracle checks what it can afford,
in a pool of worker processes:

* packed codes and metadata, bit for bit: every (sequence, kv head) stream of the
  GQA and certified workloads, the 64 streams of eight sampled sequences of the
  2-bit workload (its other sequences are drawn on the GPU from the same law) and
  all 64 streams of the FP4 workload (a one-stream oracle cache appended with the
  same tokens per worker; SHA-256 digests compared stream by stream);
* attention rows within 2e-3 (per-row max relative error) for three seeded query
  draws: all 512 rows of the GQA workload and all 256 rows of the FP4 workload,
  256 rows of eight sampled sequences of the others, against the oracle's fp64
  attention over the library's own packed bytes;
* for the certified workload, the block flags and the certificate of the sampled
  sequences, for every query draw.
"""
import hashlib
import multiprocessing as mp
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest
import torch

import bit_kv_cache_append_amd as kvq
import synth
from fullsize_oracle import ARRAYS, stream_digests
from oracle import attention, bound, codec
from gpu_harness import dev_bits, make_gpu_cache, make_oracle_cache, setup_rotation

pytestmark = pytest.mark.gpu
TOL = 2e-3
WORKERS = 16
QUERY_DRAWS = (0, 1, 2)


def _log(msg):
    print(f"[fullsize] {msg}", flush=True)


def _pool():
    return ProcessPoolExecutor(max_workers=WORKERS, mp_context=mp.get_context("spawn"),
                               initializer=synth.one_blas_thread)


def _gpu_digests(c, gcache, b, h):
    out = []
    for name in ARRAYS:
        a = gcache.bufs[name].view(c["B"], c["Hkv"], -1)[b, h].cpu().numpy()
        out.append(hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest())
    return tuple(out)


def _check_streams(tag, c, gcache, streams, r16=None, clip=None):
    """Every listed stream's packed bytes equal to the oracle's (digests)."""
    _log(f"{tag}: bytes of {len(streams)} streams")
    with _pool() as ex:
        futs = [ex.submit(stream_digests, c, b, h, r16, clip) for b, h in streams]
        bad = []
        for i, f in enumerate(futs):
            (b, h), want = f.result()
            got = _gpu_digests(c, gcache, b, h)
            bad += [(b, h, n) for n, g, w in zip(ARRAYS, got, want) if g != w]
            if (i + 1) % 16 == 0:
                _log(f"{tag}: {i + 1} of {len(streams)} streams compared")
    assert not bad, f"{tag}: {len(bad)} arrays differ, first {bad[:4]}"
    _log(f"{tag}: {len(streams)} streams bit-identical")


def _oracle_view(c, gcache, bs):
    """An oracle cache holding the library's bytes of sequences bs (all kv heads)."""
    sub = synth.config(c["cfg"], **{**c, "B": len(bs)})
    oc = make_oracle_cache(sub)
    full = make_oracle_cache(synth.config(c["cfg"], **{**c, "B": 1}))  # per-sequence shapes
    for name in ARRAYS:
        arr = gcache.bufs[name].view(c["B"], -1)
        for i, b in enumerate(bs):
            getattr(oc, name)[i] = arr[b].cpu().numpy().reshape(getattr(full, name).shape[1:])
    if c["keep"]:
        for name in ("k_orig", "v_orig"):
            arr = gcache.bufs[name].view(torch.int16).view(c["B"], c["Hkv"], c["T"], 128)
            for i, b in enumerate(bs):
                getattr(oc, name)[i] = arr[b].cpu().numpy().view(np.uint16)
    return oc


def _rows_check(got, ref, tag):
    err = attention.row_rel_err(got, ref)
    worst = float(err.max())
    _log(f"{tag}: {err.size} rows, max row rel err {worst:.3e}")
    assert worst <= TOL, f"{tag}: max row rel err {worst:.3e}"


def _fill(c, gcache, p, B, T):
    k = synth.kv_all(c, 0, 0, T, workers=WORKERS, start_method="spawn")
    v = synth.kv_all(c, 1, 0, T, workers=WORKERS, start_method="spawn")
    kvq.append(p, gcache, dev_bits(k), dev_bits(v), [0] * B)
    torch.cuda.synchronize()


# ---------------------------------------------------------------- GQA int4 (the bench line)
@pytest.fixture(scope="module")
def c2():
    """B=16 Hq=32 Hkv=8 T=8192: context append then the 4096-token prefill append (bench's calls)."""
    c = synth.config(2)
    B, T, P = c["B"], c["T"], c["prefill"]
    _log("c2: generating inputs")
    k = synth.kv_all(c, 0, 0, T, workers=WORKERS, start_method="spawn")
    v = synth.kv_all(c, 1, 0, T, workers=WORKERS, start_method="spawn")
    s, r16, s_dev, r_dev = setup_rotation(c)
    p, gcache = make_gpu_cache(c, s_dev, r_dev)
    kvq.append(p, gcache, dev_bits(k[:, :, :T - P]), dev_bits(v[:, :, :T - P]), [0] * B)
    kvq.append(p, gcache, dev_bits(k[:, :, T - P:]), dev_bits(v[:, :, T - P:]), [T - P] * B)
    torch.cuda.synchronize()
    # the launch configuration bench.py times: 2 splits x 8 kv heads x 16 sequences = 256 workgroups
    assert kvq.decode_splits(p, [T] * B) == 2
    return c, p, gcache, s, r16


def test_c2_bytes_all_streams(c2):
    c, p, gcache, s, r16 = c2
    _check_streams("c2", c, gcache, [(b, h) for b in range(c["B"]) for h in range(c["Hkv"])])


@pytest.mark.parametrize("draw", QUERY_DRAWS)
def test_c2_attention_all_rows(c2, draw):
    c, p, gcache, s, r16 = c2
    B, T = c["B"], c["T"]
    q = synth.queries(c, step=draw)
    out = kvq.decode_attn(p, gcache, dev_bits(q), [T] * B)
    torch.cuda.synchronize()
    oc = _oracle_view(c, gcache, list(range(B)))
    ref, _ = attention.decode_attention(oc, q, c["dtype"], np.full(B, T), c["rotation"], s)
    _rows_check(out.cpu().numpy(), ref, f"c2 query draw {draw}")


# ---------------------------------------------------------------- certified int8 K / int4 V
@pytest.fixture(scope="module")
def c3():
    """B=32 T=32768, int8 K / int4 V per token, fp16 copy and block descriptors."""
    c = synth.config(3)
    _log("c3: generating inputs")
    s, r16, s_dev, r_dev = setup_rotation(c)
    p, gcache = make_gpu_cache(c, s_dev, r_dev)
    _fill(c, gcache, p, c["B"], c["T"])
    bs = [0, 4, 9, 13, 18, 22, 27, 31]
    oc = _oracle_view(c, gcache, bs)
    desc = bound.block_descriptors(oc, c["dtype"], c["rotation"], s)
    return c, p, gcache, s, bs, oc, desc


def test_c3_bytes_all_streams(c3):
    c, p, gcache, s, bs, oc, desc = c3
    _check_streams("c3", c, gcache, [(b, h) for b in range(c["B"]) for h in range(c["Hkv"])])


@pytest.mark.parametrize("draw", QUERY_DRAWS)
def test_c3_certified_attention(c3, draw):
    c, p, gcache, s, bs, oc, desc = c3
    B, H, T = c["B"], c["Hkv"], c["T"]
    q = synth.queries(c, step=draw)
    seq = [T] * B
    qd = dev_bits(q)
    bnd, fl = kvq.error_bound(p, gcache, qd, seq, c["tau"])
    out, cert = kvq.decode_attn(p, gcache, qd, seq, flags=fl, certificate=True)
    torch.cuda.synchronize()
    fl_all = fl.cpu().numpy()
    _log(f"c3 query draw {draw}: {int(fl_all.sum())} of {fl_all.size} blocks flagged")
    qs = q[bs]
    seq_s = np.full(len(bs), T)
    _, of = bound.error_bound(desc, qs, c["dtype"], seq_s, c["tau"])
    assert np.array_equal(fl_all[bs], of), "flags differ from the oracle's"
    planted = {(i, h, blk) for i, b in enumerate(bs) for h in range(H) for blk, _ in synth.planted(c, b, h)}
    assert set(map(tuple, np.argwhere(fl_all[bs]))) == planted
    ref, mass = attention.decode_attention(oc, qs, c["dtype"], seq_s, c["rotation"], s, flags=fl_all[bs])
    _rows_check(out.cpu().numpy()[bs], ref, f"c3 query draw {draw}")
    E = cert.cpu().numpy()[bs]
    E_or = bound.certificate(desc, qs, c["dtype"], seq_s, fl_all[bs], mass)
    assert np.all(E >= E_or * (1 - 1e-5)) and np.all(E <= E_or * (1 + 2.0 ** -7) + 1e-9)
    dense = attention.dense_attention(oc.k_orig, oc.v_orig, qs, c["dtype"], seq_s)
    assert np.all(np.linalg.norm(ref - dense, axis=-1) <= E), "certificate must bound the error"


# ---------------------------------------------------------------- int2 with the dense rotation
@pytest.fixture(scope="module")
def c4():
    """B=64 T=32768, int2 g32 with dense rotation and clipping; every sequence holds data."""
    c = synth.config(4)
    B, H = c["B"], c["Hkv"]
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
    # every sequence holds data of the workload's law: the eight sequences the oracle checks
    # come from the seeded host generator, the others are drawn on the GPU from the same law
    # (the generator's bases, seeded normal draws) to keep the host work small
    T = c["T"]
    bs = [0, 9, 18, 27, 36, 45, 54, 63]
    _log("c4: drawing inputs on the GPU")
    lam = torch.arange(1, 129, device="cuda", dtype=torch.float32).rsqrt()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4004)
    dev = {0: torch.empty((B, H, T, 128), dtype=torch.int16, device="cuda"), 1: None}
    dev[1] = torch.empty_like(dev[0])
    for tensor in (0, 1):
        U = torch.from_numpy(np.stack([synth.anisotropic_basis(c, tensor, h) for h in range(H)])).float().cuda()
        Ut = U.transpose(1, 2).contiguous()
        for b0 in range(0, B, 8):
            z = torch.randn((8, H, T, 128), generator=gen, device="cuda")
            dev[tensor][b0:b0 + 8] = torch.matmul(z * lam, Ut).half().view(torch.int16)
            del z
    _log("c4: generating the checked sequences on the host")
    jobs = [(tensor, b, h) for tensor in (0, 1) for b in bs for h in range(H)]
    with _pool() as ex:
        for (tensor, b, h), x in zip(jobs, ex.map(synth.kv_slice, [c] * len(jobs), *zip(*jobs), [0] * len(jobs),
                                                   [T] * len(jobs))):
            dev[tensor][b, h] = dev_bits(x)
    kvq.append(p, gcache, dev[0], dev[1], [0] * B)
    torch.cuda.synchronize()
    del dev
    return c, p, gcache, s, r16, host_clip, bs


def test_c4_bytes_64_streams(c4):
    c, p, gcache, s, r16, host_clip, bs = c4
    _check_streams("c4", c, gcache, [(b, h) for b in bs for h in range(c["Hkv"])], r16=r16, clip=host_clip)


@pytest.mark.parametrize("draw", QUERY_DRAWS)
def test_c4_attention_sampled(c4, draw):
    c, p, gcache, s, r16, host_clip, bs = c4
    B, T = c["B"], c["T"]
    q = synth.queries(c, step=draw)
    out = kvq.decode_attn(p, gcache, dev_bits(q), [T] * B)
    torch.cuda.synchronize()
    oc = _oracle_view(c, gcache, bs)
    ref, _ = attention.decode_attention(oc, q[bs], c["dtype"], np.full(len(bs), T), c["rotation"], s, r16)
    _rows_check(out.cpu().numpy()[bs], ref, f"c4 query draw {draw}")


# ---------------------------------------------------------------- FP4 with scale search
@pytest.fixture(scope="module")
def c5():
    """B=8 T=131072, FP4 E2M1 with searched E4M3 block scales, bf16 Student-t inputs."""
    c = synth.config(5)
    _log("c5: generating inputs")
    s, r16, s_dev, r_dev = setup_rotation(c)
    p, gcache = make_gpu_cache(c, s_dev, r_dev)
    _fill(c, gcache, p, c["B"], c["T"])
    return c, p, gcache, s


def test_c5_bytes_all_streams(c5):
    c, p, gcache, s = c5
    _check_streams("c5", c, gcache, [(b, h) for b in range(c["B"]) for h in range(c["Hkv"])])


@pytest.mark.parametrize("draw", QUERY_DRAWS)
def test_c5_attention_all_rows(c5, draw):
    c, p, gcache, s = c5
    B, T = c["B"], c["T"]
    q = synth.queries(c, step=draw)
    out = kvq.decode_attn(p, gcache, dev_bits(q), [T] * B)
    torch.cuda.synchronize()
    oc = _oracle_view(c, gcache, list(range(B)))
    ref, _ = attention.decode_attention(oc, q, c["dtype"], np.full(B, T), c["rotation"], s)
    _rows_check(out.cpu().numpy(), ref, f"c5 query draw {draw}")
