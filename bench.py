#!/usr/bin/env python3
"""Decode-attention and append throughput of the int4 KV cache on one MI355X.

Workload (Llama-3-8B-shaped GQA decode): B=16 sequences, 32 query heads over 8
kv heads, head_dim 128, context 8192; fp16 K/V N(0,1) with 10 seeded (head,
channel) pairs x8; sign + Walsh-Hadamard rotation; symmetric int4 with one fp16
scale per 32 channels for K and V.

One step = the whole hot path:
  1. kvq_append of a 4096-token prefill (positions 4096..8191 of all 16
     sequences, 16 x 8 x 4096 K and V vectors) into one cache, then
  2. kvq_decode_attn of one query token per (sequence, query head) over all 8192
     positions of another cache.
Four caches (and four copies of the prefill input) are used in rotation: the
decode of step i reads the cache appended in step i-2, so between two uses of a
cache at least 3 x 144 MiB of other data streams through the 256 MB Infinity
Cache and every timed call reads its inputs from HBM.  Each kernel sequence is
also timed on its own: batches of back-to-back calls over the rotating buffers,
HIP events around each batch on the stream the calls are launched on, the median
of the batch means (decode: 32 batches of 16 calls, after 64 untimed ones); and once more as 50 single
calls, each after a 1 GiB read flush (median; includes one launch).

value = decode effective KV GB/s = packed K/V bytes (codes + scales) / median
decode call time (one launch: the splits are merged by their last workgroup).
The same-shape fp16 decode (kvq_decode_attn_dense) is timed the same way for the
int4-vs-fp16 comparison; append throughput is reported in Mvec/s.  The CPU oracle
is timed as a reported baseline: one process on 4 sequences, and one process per
available core (at most 16) over all 16 sequences.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_F32_PEAK_TFLOPS = 157.3
# VALU issue peak without packed instructions (the build disables packed fp32): 256 CUs x
# 4 SIMDs x 16 lanes per clock (one wave64 instruction per SIMD every 4 cycles) x 2.4 GHz,
# in lane-instructions per second; the published 157.3 TFLOP/s counts packed fp32 FMAs
VALU_PEAK_TLANES = 256 * 4 * 16 * 2.4e9 / 1e12
METRIC = "decode-attn effective KV GB/s & % HBM peak (int4 vs fp16); append Mvec/s"
NROT = 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workers", type=int, default=min(16, os.cpu_count() or 1))
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with one plain 256 MiB device copy (reference for hardware byte counters)")
    ap.add_argument("--workload", type=int, default=2, choices=(2, 3, 4, 5),
                    help="2 (default): the GQA int4 line; 3/4/5: the certified, int2 and FP4 workloads")
    ap.add_argument("--window", type=str, default=None, metavar="SINK,RECENT",
                    help="workloads 3/4/5: keep the first SINK and last RECENT 64-token blocks of every "
                         "sequence at full precision")
    ap.add_argument("--adaptive", type=str, default=None, metavar="TAU_COV,EPS[,TAU_V[,MARGIN[,MAX_INV]]]",
                    help="workload 3 with retrieval needles and queries that seek them: also time the "
                         "adaptive-precision ladder (scoring pass, top-K* promotion covering TAU_COV of the "
                         "estimated mass, value promotion of blocks whose mass times value error exceeds TAU_V "
                         "(default 1e-6), ranking-consistency check with margin MARGIN (default 0) and at most "
                         "MAX_INV inverted pairs (default 0), decode, dense fallback of the heads that fail the "
                         "check or whose certificate exceeds EPS)")
    ap.add_argument("--rotation", default="sign_fwht", choices=("sign_fwht", "srft"),
                    help="workload 2: the rotation applied before quantization (sign + Walsh-Hadamard, or the "
                         "sign + real-packed FFT form)")
    args = ap.parse_args()
    if args.rotation != "sign_fwht" and args.workload != 2:
        ap.error("--rotation applies to workload 2")
    if args.adaptive is not None:
        if args.workload != 3:
            ap.error("--adaptive applies to workload 3 (the certified cache)")
        vals = [float(x) for x in args.adaptive.split(",")]
        if not 2 <= len(vals) <= 5:
            ap.error("--adaptive takes TAU_COV,EPS[,TAU_V[,MARGIN[,MAX_INV]]]")
        vals += [1e-6, 0.0, 0.0][len(vals) - 2:]
        args.adaptive = tuple(vals[:4]) + (int(vals[4]),)
    if args.window is not None:
        if args.workload == 2:
            ap.error("--window applies to workloads 3, 4 and 5")
        args.window = tuple(int(x) for x in args.window.split(","))
        if len(args.window) != 2 or min(args.window) < 0:
            ap.error("--window takes SINK,RECENT (two non-negative block counts)")
    return args


def median_of_batches(batch_time, fn, per, n_batches):
    """(median, min) over n_batches of the mean ms per call of per back-to-back calls of fn(i)
    (HIP events around each batch, on the stream the calls are launched on)."""
    vals = []
    for k in range(n_batches):
        vals.append(batch_time(lambda i, k=k: fn(k * per + i), per))
    return float(np.median(vals)), float(np.min(vals))


def attention_window_tokens(T, n_sink, n_recent):
    """Tokens of a T-token sequence in its first n_sink and last n_recent 64-token blocks."""
    nb = (T + 63) // 64
    blocks = [j for j in range(nb) if j < n_sink or j >= nb - n_recent]
    return sum(min(T, 64 * j + 64) - 64 * j for j in blocks)


def kernel_traffic(roofline_kernel_src):
    """HBM bytes per decode call from the committed counter summary, if it was taken on this kernel source."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    prof = os.path.join(here, "profiles", "decode_int4_c2_traffic.json")
    src = os.path.join(here, roofline_kernel_src)
    try:
        rec = json.load(open(prof))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_call")


def append_valu_roofline(key, app_s):
    """VALU roofline of an append launch: the committed per-launch VALU instruction count of
    this workload (SQ_INSTS_VALU, valid only for the kernel source it was taken on) x 64
    lanes / the launch time measured here, against VALU_PEAK_TLANES; None without a record."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    try:
        rec = json.load(open(os.path.join(here, "profiles", "append_valu.json")))
        sha = hashlib.sha256(open(os.path.join(here, rec["kernel_source"]), "rb").read()).hexdigest()
    except (OSError, ValueError, KeyError):
        return None
    w = rec.get("workloads", {}).get(key)
    if rec.get("kernel_source_sha256") != sha or w is None:
        return None
    achieved = w["valu_wave_instr_per_launch"] * 64 / app_s / 1e12
    return {"bound": "alu", "achieved": round(achieved, 2), "peak": round(VALU_PEAK_TLANES, 2),
            "unit": "T VALU lane-instructions/s", "frac": round(achieved / VALU_PEAK_TLANES, 4),
            "kernel": w["kernel"], "valu_wave_instr_per_launch": w["valu_wave_instr_per_launch"],
            **({"note": w["note"]} if "note" in w else {})}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_seq_setup(c, b):
    """Inputs of sequence b and an oracle cache holding its context before the prefill."""
    import synth
    from oracle import codec
    cs = dict(c, B=1)
    T, P, H = c["T"], c["prefill"], c["Hkv"]
    k = np.stack([synth.kv_slice(c, 0, b, h, 0, T) for h in range(H)])[None]
    v = np.stack([synth.kv_slice(c, 1, b, h, 0, T) for h in range(H)])[None]
    s = synth.signs(c)
    oc = codec.Cache(1, H, T, cs["k_fmt"], cs["v_fmt"], cs["k_group"], cs["v_group"])
    codec.append(oc, k[:, :, :T - P], v[:, :, :T - P], np.zeros(1, int), "f16", cs["rotation"], s,
                 scale_mode=cs["scale_mode"])
    q = synth.queries(c)[b:b + 1]
    return k, v, s, oc, q


def _oracle_seq_run(c, k, v, s, oc, q):
    """Times (append of the prefill, decode over the whole context) of one sequence."""
    from oracle import attention, codec
    T, P = c["T"], c["prefill"]
    t0 = time.perf_counter()
    codec.append(oc, k[:, :, T - P:], v[:, :, T - P:], np.full(1, T - P), "f16", c["rotation"], s,
                 scale_mode=c["scale_mode"])
    t1 = time.perf_counter()
    attention.decode_attention(oc, q, "f16", np.full(1, T), c["rotation"], s)
    t2 = time.perf_counter()
    return t1 - t0, t2 - t1


def _oracle_worker(c, seqs, barrier, out):
    """One process of the N-process baseline: set its sequences up, wait for the others, then
    run the prefill appends of all of them and, after a second barrier, their decodes."""
    os.environ["OMP_NUM_THREADS"] = "1"
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        st = [_oracle_seq_setup(c, b) for b in seqs]
        from oracle import attention, codec
        T, P = c["T"], c["prefill"]
        barrier.wait()
        ta0 = time.time()
        for k, v, s, oc, q in st:
            codec.append(oc, k[:, :, T - P:], v[:, :, T - P:], np.full(1, T - P), "f16", c["rotation"], s,
                         scale_mode=c["scale_mode"])
        ta1 = time.time()
        barrier.wait()
        td0 = time.time()
        for k, v, s, oc, q in st:
            attention.decode_attention(oc, q, "f16", np.full(1, T), c["rotation"], s)
        td1 = time.time()
    out.put((ta0, ta1, td0, td1))


def cpu_baseline(c, sample_b):
    """The oracle timed on the host cores (a reported baseline, not the target).

    One process (one BLAS thread) on sample_b sequences; then N processes (one BLAS thread
    each, N = the cores this process may use, at most 16) over all B sequences, released
    together by a barrier after their set-up, the append and the decode timed separately."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits
    T, P, H, B = c["T"], c["prefill"], c["Hkv"], c["B"]
    bytes_per_seq = H * T * 144
    with threadpool_limits(1):
        app1 = dec1 = 0.0
        for b in range(sample_b):
            st = _oracle_seq_setup(c, b)
            ta, td = _oracle_seq_run(c, *st)
            app1 += ta
            dec1 += td
    cores = len(os.sched_getaffinity(0))
    nproc = max(1, min(16, cores, B))
    ctx = mp.get_context("spawn")  # the parent has initialised the GPU: no fork
    barrier = ctx.Barrier(nproc)
    out = ctx.Queue()
    procs = [ctx.Process(target=_oracle_worker, args=(c, list(range(r, B, nproc)), barrier, out)) for r in range(nproc)]
    for pr in procs:
        pr.start()
    res = [out.get(timeout=600) for _ in procs]
    for pr in procs:
        pr.join(timeout=60)
    app_n = max(r[1] for r in res) - min(r[0] for r in res)
    dec_n = max(r[3] for r in res) - min(r[2] for r in res)
    vecs_seq = H * P * 2
    return {
        "value": round(bytes_per_seq * B / dec_n / 1e9, 4), "unit": "GB/s", "cores": nproc, "kind": "oracle",
        "sample": (f"all {B} sequences in {nproc} processes (one BLAS thread each, released together): decode over "
                   f"{T} tokens of every sequence (all {c['Hq']} q heads) in {dec_n:.2f} s, the {P}-token prefill "
                   f"append ({vecs_seq * B} vectors) in {app_n:.2f} s; one process on {sample_b} sequences: decode "
                   f"{dec1:.2f} s, append {app1:.2f} s"),
        "append_mvec_s": round(vecs_seq * B / app_n / 1e6, 4),
        "single_process": {"value": round(bytes_per_seq * sample_b / dec1 / 1e9, 4),
                           "append_mvec_s": round(vecs_seq * sample_b / app1 / 1e6, 4), "sequences": sample_b},
        "host": {"cpus_available": cores, "cpu_model": _cpu_model()},
    }


def bench_workload(cfg_id, args):
    """Decode and append throughput of workload 3 (certified int8/int4), 4 (int2, dense rotation)
    or 5 (FP4 with scale search) at full shape, same timing method as the default line.

    Inputs are drawn on the GPU from a seeded generator with the workload's law (the host
    generator would take minutes at these sizes; the values only have to have the right
    distribution and structure for timing).  The full context is filled by appending one
    4096-token piece repeatedly; the timed append is a 4096-token prefill at the end of the
    context, as in the default line.
    """
    import torch
    import bit_kv_cache_append_amd as kvq
    import synth

    kvq.lib()
    dev = torch.device("cuda:0")
    c = synth.config(cfg_id)
    if args.window is not None:
        c["sink_blocks"], c["recent_blocks"] = args.window
    if args.adaptive is not None:
        c["needles"] = 4
    B, Hq, H, T, P = c["B"], c["Hq"], c["Hkv"], c["T"], c["prefill"]
    nrot = 4
    g = torch.Generator(device=dev)
    g.manual_seed(1234 + cfg_id)

    def progress(msg):
        print(f"[bench w{cfg_id}] {msg}", file=sys.stderr, flush=True)

    # The certified workload fills its context with T / P distinct pieces (the others reuse nrot
    # pieces): planted tokens (x10 in K and V alike), two in each of the first two pieces and
    # one in each other piece of every (sequence, kv head), so every stream holds 10 planted
    # tokens in 512 blocks (~2%).  With needles, every stream also holds that many retrieval
    # needles at uniform positions: needle i's key is L_i sqrt(128) / a * u for a unit
    # direction u of the stream, L_i = top - i (top uniform in 20 +- 0.5; in one stream of
    # eight, L_1 = L_0 - 0.005), and the queries of the stream's heads are a u + (I - u u^T) z,
    # which gives needle i the logit L_i.
    nfill = T // P if c["data"] == "certified" else nrot
    plant_pos = [torch.randint(0, P, (2 if i < 10 - nfill else 1, B, H), generator=g, device=dev)
                 for i in range(nfill)]
    nn = int(c.get("needles", 0))
    if nn:
        ndir = torch.randn((B, H, 128), generator=g, device=dev, dtype=torch.float64)
        ndir /= ndir.norm(dim=-1, keepdim=True)
        nlog = (c["needle_top"] + torch.rand((B, H, 1), generator=g, device=dev, dtype=torch.float64) - 0.5
                - torch.arange(nn, device=dev, dtype=torch.float64))
        tie = (torch.arange(B * H, device=dev) % c["needle_tie_every"] == 0).view(B, H)
        nlog[..., 1] = torch.where(tie, nlog[..., 0] - 0.005, nlog[..., 1])
        npos = torch.randint(0, T, (B, H, nn), generator=g, device=dev)

    def draw(tensor, piece):
        shape = (B, H, P, 128)
        if c["data"] == "certified":
            x = torch.randn(shape, generator=g, device=dev) * (c["k_sigma"] if tensor == 0 else c["v_sigma"])
            for t in plant_pos[piece]:
                idx = t[..., None, None].expand(B, H, 1, 128)
                x.scatter_(2, idx, x.gather(2, idx) * c["plant_factor"])
            if nn and tensor == 0:
                for i in range(nn):
                    here = (npos[..., i] // P == piece)[..., None, None]
                    idx = (npos[..., i] % P)[..., None, None].expand(B, H, 1, 128)
                    key = (nlog[..., i, None] * math.sqrt(128) / c["needle_q"] * ndir).float()[:, :, None, :]
                    x.scatter_(2, idx, torch.where(here, key, x.gather(2, idx)))
            return x.half().view(torch.int16)
        if c["data"] == "anisotropic":
            z = torch.randn(shape, generator=g, device=dev)
            d = torch.arange(1, 129, device=dev, dtype=torch.float32).rsqrt()
            # Haar bases per kv head from a QR on the host (small), then to the device
            gh = torch.Generator().manual_seed(int(torch.randint(0, 2 ** 31, (1,), generator=g, device=dev).item()))
            u = torch.linalg.qr(torch.randn((H, 128, 128), generator=gh, dtype=torch.float64))[0].float().to(dev)
            x = torch.matmul(z * d, u.transpose(1, 2).contiguous())  # x[b,h,t] = U_h (d * z)
            return x.half().view(torch.int16)
        # Student-t(nu) = N(0,1) / sqrt(chi2(nu) / nu), chi2(nu) = sum of nu squared normals (nu = 4)
        nu = int(c["nu"])
        z = torch.randn(shape, generator=g, device=dev)
        chi = sum(torch.randn(shape, generator=g, device=dev) ** 2 for _ in range(nu))
        x = z / torch.sqrt(chi / nu)
        return x.bfloat16().view(torch.int16)

    s_dev = torch.from_numpy(synth.signs(c).copy()).to(dev)
    r_dev = kvq.to_device_bits(synth.dense_rotation_f16(c)) if c["rotation"] == "dense" else None
    p = kvq.params_from_config(c)
    caches = [kvq.Cache(p, signs=s_dev, rot_f16=r_dev) for _ in range(nrot)]
    if c["k_fmt"] == "int2" or c["v_fmt"] == "int2":
        ck = np.stack([synth.calibration(c, 0, h) for h in range(H)])
        cv = np.stack([synth.calibration(c, 1, h) for h in range(H)])
        tk, tv = kvq.calibrate_clip(p, caches[0], kvq.to_device_bits(ck), kvq.to_device_bits(cv),
                                    ratio=c["clip_ratio"])
        for cc in caches:
            cc.clip_k, cc.clip_v = tk, tv
    kin = [draw(0, i) for i in range(nfill)]
    vin = [draw(1, i) for i in range(nfill)]
    for cc in caches:
        for t0 in range(0, T, P):
            kvq.append(p, cc, kin[(t0 // P) % nfill], vin[(t0 // P) % nfill], [t0] * B)
    torch.cuda.synchronize()
    progress("caches filled")
    q = torch.randn((B, Hq, 128), generator=g, device=dev)
    if nn:
        uq = ndir.float().repeat_interleave(Hq // H, dim=1)
        q = c["needle_q"] * uq + q - (q * uq).sum(-1, keepdim=True) * uq
    q = (q.bfloat16() if c["dtype"] == "bf16" else q.half()).view(torch.int16)
    seq = [T] * B
    ws = kvq.workspace(p)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
    cert = torch.empty((B, Hq), dtype=torch.float32, device=dev) if c["keep"] else None
    nt = T // 64
    bnd = torch.empty((B, H, nt), dtype=torch.float32, device=dev)
    flg = torch.empty((B, H, nt), dtype=torch.uint8, device=dev)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def batch_time(fn, n):
        e0, e1 = ev(), ev()
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def do_decode(i):
        cc = caches[i % nrot]
        if c["keep"]:
            kvq.error_bound(p, cc, q, seq, c["tau"], bound=bnd, flags=flg)
            kvq.decode_attn(p, cc, q, seq, flags=flg, certificate=True, ws=ws, out=out, cert=cert)
        else:
            kvq.decode_attn(p, cc, q, seq, ws=ws, out=out)

    def do_append(i):
        # a 4096-token prefill: the reused pieces go to the last span; the distinct pieces of
        # the certified workload go back to their own spans (among the last nrot), so the
        # cache's contents, planted tokens and needles included, stay as filled
        if nfill == nrot:
            kvq.append(p, caches[i % nrot], kin[i % nrot], vin[i % nrot], [T - P] * B)
        else:
            piece = nfill - nrot + i % nrot
            kvq.append(p, caches[i % nrot], kin[piece], vin[piece], [piece * P] * B)

    n_each = max(args.steps, 4 * nrot)
    for i in range(args.warmup):
        do_append(i)
        do_decode(i + 2)
    torch.cuda.synchronize()
    step_ms = batch_time(lambda i: (do_append(i), do_decode(i + 2)), args.steps)
    progress(f"{args.steps} steps timed")
    batch_time(do_decode, 4 * nrot)  # untimed: the clocks settle under this load first
    dec_ms, dec_min = median_of_batches(batch_time, do_decode, 16, 8)
    batch_time(do_append, nrot)
    app_ms, _ = median_of_batches(batch_time, do_append, 8, 8)
    # the fp16/bf16 same-shape baseline: the certified workload's own originals, else fresh tensors
    if c["keep"]:
        dense = [(caches[i].bufs["k_orig"], caches[i].bufs["v_orig"]) for i in range(2)]
    else:
        dense = []
        for i in range(2):
            kd = torch.empty((B, H, T, 128), dtype=torch.int16, device=dev)
            vd = torch.empty_like(kd)
            for t0 in range(0, T, P):
                kd[:, :, t0:t0 + P] = kin[(t0 // P + i) % nrot]
                vd[:, :, t0:t0 + P] = vin[(t0 // P + i) % nrot]
            dense.append((kd, vd))
    dws = kvq.workspace(p)
    dout = torch.empty_like(out)
    batch_time(lambda i: kvq.decode_attn_dense(p, dense[i % 2][0], dense[i % 2][1], q, seq, ws=dws, out=dout), 8)
    f16_ms, _ = median_of_batches(batch_time, lambda i: kvq.decode_attn_dense(p, dense[i % 2][0], dense[i % 2][1], q,
                                                                              seq, ws=dws, out=dout), 8, 8)
    progress("batches timed")
    sizes = kvq.buffer_bytes(p)
    packed = sizes["k_codes"] + sizes["k_meta"] + sizes["v_codes"] + sizes["v_meta"]
    io = B * Hq * 128 * 2 + B * Hq * 128 * 4
    extra = ""
    if c["keep"]:
        do_decode(0)
        torch.cuda.synchronize()
        nflag = int(flg.sum().item())
        kb_tok = 128 + 2
        vb_tok = 64 + 2
        packed += sizes["blk_desc"] - nflag * 64 * (kb_tok + vb_tok) + nflag * 64 * 512
        io += B * Hq * 4
        extra = f"; {nflag} of {flg.numel()} blocks flagged ({100.0 * nflag / flg.numel():.2f}%), recomputed from fp16"
    if args.window is not None:
        # window blocks are read from the full-precision copy (512 B per token) instead of the codes
        nwin = int(attention_window_tokens(T, *args.window))
        per_tok = (sizes["k_codes"] + sizes["k_meta"] + sizes["v_codes"] + sizes["v_meta"]) // (B * H * T)
        packed += B * H * nwin * (512 - per_tok)
        extra += (f"; window: first {args.window[0]} and last {args.window[1]} blocks of 64 tokens at full "
                  f"precision ({nwin} tokens per sequence and kv head)")
    dense_bytes = 2 * B * H * T * 128 * 2
    vecs = B * H * P * 2
    in_bytes = vecs * 256
    out_bytes = vecs // 2 * (sizes["k_codes"] + sizes["k_meta"] + sizes["v_codes"] + sizes["v_meta"]) // (B * H * T)
    if c["keep"]:
        out_bytes += vecs * 256  # fp16 copies
    app_bytes = in_bytes + out_bytes
    dec_s, app_s, f16_s = dec_ms / 1e3, app_ms / 1e3, f16_ms / 1e3
    achieved = (packed + io) / dec_s / 1e9
    fmt = f"{c['k_fmt']} K / {c['v_fmt']} V"
    result = {
        "metric": METRIC,
        "value": round(packed / dec_s / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"int8": "int8", "int4": "int4", "int2": "int2", "fp4": "fp4"}[c["k_fmt"]],
        "data": f"synthetic, drawn on the GPU from a seeded generator ({c['data']}){extra}",
        "config": {"workload": c["name"], "B": B, "Hq": Hq, "Hkv": H, "head_dim": 128, "context": T,
                   "prefill_tokens": P, "formats": fmt, "rotation": c["rotation"], "input": c["dtype"],
                   **({"window_blocks": list(args.window)} if args.window is not None else {}),
                   **({"needles": nn} if nn else {})},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "decode_split (splits merged by their last workgroup)" + (" + bound_kernel" if c["keep"] else ""),
                     "bytes_per_call": packed + io},
        "decode_us": round(dec_s * 1e6, 2),
        "decode_us_min_batch": round(dec_min * 1e3, 2),
        "decode_timing": "median over 8 batches of the mean of 16 back-to-back calls, after untimed ones",
        "decode_grid_workgroups": kvq.decode_splits(p, seq) * B * H * ((Hq // H + 3) // 4),
        "decode_splits": kvq.decode_splits(p, seq),
        "fp16_decode_us": round(f16_s * 1e6, 2),
        "fp16_decode_pct_hbm_peak": round(100 * dense_bytes / f16_s / 1e9 / HBM_PEAK_GBS, 2),
        "speedup_vs_fp16": round(f16_s / dec_s, 3),
        "append_us": round(app_s * 1e6, 2),
        "append_mvec_s": round(vecs / app_s / 1e6, 1),
        "append_gbs": round(app_bytes / app_s / 1e9, 1),
        "append_pct_hbm_peak": round(100 * app_bytes / app_s / 1e9 / HBM_PEAK_GBS, 2),
    }
    if c["rotation"] == "dense":
        # the write side is bound by the exact fp32 rotation: 2 * 128 * 128 flops per vector on
        # fp32 K=1 MFMA chains (dense fp32 matrix peak 157.3 TFLOP/s)
        tf = vecs * 2 * 128 * 128 / app_s / 1e12
        result["append_roofline"] = {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_F32_PEAK_TFLOPS,
                                     "unit": "TFLOP/s", "frac": round(tf / MFMA_F32_PEAK_TFLOPS, 4),
                                     "kernel": "append_dense_int2_kernel"}
    else:
        # the fast append is VALU work (the exact fp32 rotation, quotients and packing; for FP4
        # the scale search): its instruction count per launch against the VALU issue peak
        valu = append_valu_roofline(c["name"], app_s) if args.window is None else None
        if valu is not None:
            result["append_roofline"] = valu
    if args.adaptive is not None:
        result["adaptive"] = adaptive_ladder(args, c, p, caches, q, seq, ws, out, cert, bnd, flg, batch_time, n_each)
        # the same step without the ladder: the bound and the certified decode with its flags
        # (decode_us above), and dense fp16 attention over the originals
        result["adaptive"]["certified_decode_us"] = result["decode_us"]
        result["adaptive"]["fp16_decode_us"] = result["fp16_decode_us"]
        progress("adaptive ladder timed")
    if args.copy_calibration:
        src = torch.full((256 << 20,), 3, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
    print(json.dumps(result))


def adaptive_ladder(args, c, p, caches, q, seq, ws, out, cert, bnd, flg, batch_time, n_each):
    """Times of the adaptive-precision ladder on the certified cache, stage by stage."""
    import torch
    import bit_kv_cache_append_amd as kvq
    tau_cov, eps, tau_v, margin, max_inv = args.adaptive
    B, Hq, H, T = c["B"], c["Hq"], c["Hkv"], c["T"]
    nrot = len(caches)
    mass = torch.empty((B, Hq, T // 64), dtype=torch.float32, device=q.device)
    prom = torch.empty_like(flg)
    inv = torch.empty((B, Hq), dtype=torch.int32, device=q.device)
    fail = torch.empty((B, Hq), dtype=torch.uint8, device=q.device)

    def stages(i, which):
        cc = caches[i % nrot]
        if "bound" in which:
            kvq.error_bound(p, cc, q, seq, c["tau"], bound=bnd, flags=flg)
        if "mass" in which:
            kvq.block_mass(p, cc, q, seq, mass=mass)
        if "select" in which:
            kvq.select_blocks(p, mass, seq, tau_cov, flags_in=flg, flags_out=prom)
        if "promote" in which:
            kvq.promote_values(p, cc, mass, seq, tau_v, prom)
        if "rank" in which:
            kvq.ranking_check(p, cc, q, seq, mass, tau_cov, margin, max_inv, out=(inv, fail))
        if "decode" in which:
            kvq.decode_attn(p, cc, q, seq, flags=prom, certificate=True, ws=ws, out=out, cert=cert)
        if "fallback" in which:
            kvq.dense_fallback(p, cc, q, seq, eps, out, cert, fail=fail, ws=ws)

    allst = ("bound", "mass", "select", "promote", "rank", "decode", "fallback")
    for i in range(nrot):
        stages(i, allst)
    torch.cuda.synchronize()
    step_ms = batch_time(lambda i: stages(i, allst), n_each)
    bound_ms = batch_time(lambda i: stages(i, ("bound",)), n_each)
    mass_ms = batch_time(lambda i: stages(i, ("mass",)), n_each)
    sel_ms = batch_time(lambda i: stages(i, ("select",)), n_each)
    stages(0, ("bound", "mass", "select"))
    p0 = prom.clone()
    prom_ms = batch_time(lambda i: (prom.copy_(p0), stages(0, ("promote",))), n_each)
    copy_ms = batch_time(lambda i: prom.copy_(p0), n_each)
    rank_ms = batch_time(lambda i: stages(0, ("rank",)), n_each)
    stages(0, ("promote",))
    dec_ms = batch_time(lambda i: stages(0, ("decode",)), n_each)
    c0 = cert.clone()
    fb_ms = batch_time(lambda i: (cert.copy_(c0), stages(0, ("fallback",))), n_each)
    torch.cuda.synchronize()
    pr = prom.cpu().numpy()
    nbound = int(flg.sum().item())
    nfail = int(fail.sum().item())
    nfall = int(((c0 > eps) | (fail != 0)).sum().item())
    sizes = kvq.buffer_bytes(p)
    kbytes = sizes["k_codes"] + sizes["k_meta"] + B * Hq * 128 * 2 + B * Hq * (T // 64) * 4
    invn = inv.cpu().numpy()
    return {
        "tau_cov": tau_cov, "eps": eps, "tau_v": tau_v, "ranking_margin": margin, "ranking_max_inversions": max_inv,
        "data": f"{c['needles']} retrieval needles per (sequence, kv head), queries that seek them",
        "step_us": round(step_ms * 1e3, 2),
        "error_bound_us": round(bound_ms * 1e3, 2),
        "block_mass_us": round(mass_ms * 1e3, 2),
        "select_us": round(sel_ms * 1e3, 2),
        "promote_values_us": round(max(prom_ms - copy_ms, 0.0) * 1e3, 2),
        "ranking_check_us": round(rank_ms * 1e3, 2),
        "decode_promoted_us": round(dec_ms * 1e3, 2),
        "fallback_us_incl_cert_copy": round(fb_ms * 1e3, 2),
        "blocks": int(prom.numel()), "blocks_flagged_by_bound": nbound,
        "blocks_promoted": int(((pr & 1) != 0).sum()), "blocks_value_promoted": int(((pr & 3) == 2).sum()),
        "heads": B * Hq, "heads_failing_ranking_check": nfail, "heads_fallen_back": nfall,
        "inversions_max": int(invn.max()), "heads_with_inversions": int((invn > 0).sum()),
        "block_mass_roofline": {"bound": "hbm", "achieved": round(kbytes / (mass_ms / 1e3) / 1e9, 1),
                                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(kbytes / (mass_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                                "kernel": "score_kernel + mass_kernel", "bytes_per_call": kbytes},
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one MI355X; --gpus {args.gpus} is not supported (the library runs on one GPU).",
              file=sys.stderr)
        sys.exit(2)
    if args.workload != 2:
        bench_workload(args.workload, args)
        return
    import torch
    import bit_kv_cache_append_amd as kvq
    import synth

    kvq.lib()  # fail loudly if the HIP library is missing

    def progress(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")
    c = synth.config(2, rotation=args.rotation)
    B, Hq, H, T, P = c["B"], c["Hq"], c["Hkv"], c["T"], c["prefill"]
    t_gen = time.perf_counter()
    k_all = synth.kv_all(c, 0, 0, T, workers=args.workers)
    v_all = synth.kv_all(c, 1, 0, T, workers=args.workers)
    q_np = synth.queries(c)
    t_gen = time.perf_counter() - t_gen
    progress(f"inputs generated in {t_gen:.1f} s")
    k_dev = kvq.to_device_bits(k_all)
    v_dev = kvq.to_device_bits(v_all)
    del k_all, v_all
    q = kvq.to_device_bits(q_np)
    s_dev = torch.from_numpy(synth.signs(c).copy()).to(dev)
    p = kvq.params_from_config(c)
    seq = [T] * B
    # NROT caches with the context [0, T - P) appended once (untimed), NROT copies of the prefill input
    caches = [kvq.Cache(p, signs=s_dev) for _ in range(NROT)]
    k_ctx = k_dev[:, :, :T - P].contiguous()
    v_ctx = v_dev[:, :, :T - P].contiguous()
    for cc in caches:
        kvq.append(p, cc, k_ctx, v_ctx, [0] * B)
    del k_ctx, v_ctx
    k_pre = [k_dev[:, :, T - P:].contiguous() for _ in range(NROT)]
    v_pre = [v_dev[:, :, T - P:].contiguous() for _ in range(NROT)]
    for cc in caches:  # every cache holds the full context before any decode
        kvq.append(p, cc, k_pre[0], v_pre[0], [T - P] * B)
    ws = kvq.workspace(p)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
    # fp16 baseline: two copies of the dense K/V (2 x 512 MiB) in rotation
    kd = [k_dev, k_dev.clone()]
    vd = [v_dev, v_dev.clone()]
    dws = kvq.workspace(p)
    dout = torch.empty_like(out)
    flush_buf = torch.ones(1 << 27, dtype=torch.int64, device=dev)  # 1 GiB
    sink = torch.zeros((), dtype=torch.int64, device=dev)
    torch.cuda.synchronize()
    progress("caches filled")

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def batch_time(fn, n):
        """Mean ms per call of fn(i) for n back-to-back calls (events around the batch)."""
        e0, e1 = ev(), ev()
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def do_append(i):
        kvq.append(p, caches[i % NROT], k_pre[i % NROT], v_pre[i % NROT], [T - P] * B)

    def do_decode(i):
        kvq.decode_attn(p, caches[i % NROT], q, seq, ws=ws, out=out)

    def do_dense(i):
        kvq.decode_attn_dense(p, kd[i % 2], vd[i % 2], q, seq, ws=dws, out=dout)

    def step(i):
        do_append(i)
        do_decode(i + 2)

    # warm-up, then the timed steps (whole hot path)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_ms = batch_time(lambda i: step(args.warmup + i), args.steps)
    wall = time.perf_counter() - t0
    progress(f"{args.steps} steps timed")
    # each kernel sequence on its own over the rotating buffers
    n_each = max(args.steps, 4 * NROT)
    batch_time(do_decode, 16 * NROT)  # untimed: the clocks settle under this load first
    dec_ms, dec_min = median_of_batches(batch_time, do_decode, 16, 32)
    batch_time(do_append, 4 * NROT)
    app_ms, _ = median_of_batches(batch_time, do_append, 8, 16)
    batch_time(do_dense, 16)  # the same-shape baseline gets the same untimed start
    f16_ms, _ = median_of_batches(batch_time, do_dense, 8, 16)
    progress("per-kernel batches timed")
    # isolated calls: 1 GiB read flush, events around each call
    # isolated calls: 10 warm-ups, then the median of 50, each after a 1 GiB read flush
    iso = []
    for i in range(60):
        torch.sum(flush_buf, dim=0, out=sink)
        e0, e1 = ev(), ev()
        e0.record()
        do_decode(i)
        e1.record()
        if i >= 10:
            iso.append((e0, e1))
    torch.cuda.synchronize()
    iso_ms = float(np.median([a.elapsed_time(b) for a, b in iso]))
    # int4 vs fp16 outputs on the same query (quantization effect, informational)
    do_decode(0)
    do_dense(0)
    torch.cuda.synchronize()
    rel = (out - dout).abs().amax(dim=-1) / dout.abs().amax(dim=-1)
    int4_vs_fp16_maxrel = float(rel.max().item())

    kv_bytes = B * H * T * (64 + 8) * 2            # packed K and V: codes + fp16 group scales
    io_bytes = B * Hq * 128 * 2 + B * Hq * 128 * 4  # query in, fp32 output out
    f16_bytes = B * H * T * 128 * 2 * 2
    vecs = B * H * P * 2
    app_bytes = vecs * (256 + 72)
    dec_s, f16_s, app_s = dec_ms / 1e3, f16_ms / 1e3, app_ms / 1e3
    dec_gbs = kv_bytes / dec_s / 1e9
    achieved = (kv_bytes + io_bytes) / dec_s / 1e9
    n_splits = kvq.decode_splits(p, seq)
    result = {
        "metric": METRIC,
        "value": round(dec_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4",
        "data": "synthetic (seeded fp16 N(0,1) K/V with outlier channels; no model weights)",
        "config": {"workload": "llama3-8b-shaped GQA int4 decode + prefill append", "B": B, "Hq": Hq, "Hkv": H,
                   "head_dim": 128, "context": T, "prefill_tokens": P, "k_fmt": "int4 g32", "v_fmt": "int4 g32",
                   "rotation": {"sign_fwht": "sign+fwht", "srft": "sign+srft"}[args.rotation]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "decode_split<int4 g32, int4 g32> (one kvq_decode_attn call: one launch, splits merged by their last workgroup)",
                     "bytes_per_call": kv_bytes + io_bytes},
        "decode_us": round(dec_s * 1e6, 2),
        "decode_pct_hbm_peak": round(100 * dec_gbs / HBM_PEAK_GBS, 2),
        "decode_isolated_call_us": round(iso_ms * 1e3, 2),
        "decode_isolated_timing": "median of 50 single calls, each after a 1 GiB read flush (includes one launch)",
        "decode_us_min_batch": round(dec_min * 1e3, 2),
        "decode_timing": "median over 32 batches of the mean of 16 back-to-back calls over 4 rotating caches",
        "decode_grid_workgroups": n_splits * B * H * ((Hq // H + 3) // 4),
        "decode_splits": n_splits,
        "fp16_decode_us": round(f16_s * 1e6, 2),
        "fp16_decode_gbs": round(f16_bytes / f16_s / 1e9, 1),
        "fp16_decode_pct_hbm_peak": round(100 * f16_bytes / f16_s / 1e9 / HBM_PEAK_GBS, 2),
        "int4_speedup_vs_fp16": round(f16_s / dec_s, 3),
        "int4_fp16_equivalent_gbs": round(f16_bytes / dec_s / 1e9, 1),
        "int4_vs_fp16_out_max_rel": round(int4_vs_fp16_maxrel, 5),
        "append_us": round(app_s * 1e6, 2),
        "append_mvec_s": round(vecs / app_s / 1e6, 1),
        "append_gbs": round(app_bytes / app_s / 1e9, 1),
        "append_pct_hbm_peak": round(100 * app_bytes / app_s / 1e9 / HBM_PEAK_GBS, 2),
        "wall_ms_per_step": round(wall / args.steps * 1e3, 4),
        "input_gen_s": round(t_gen, 2),
    }
    result["roofline"]["traffic"] = kernel_traffic("bit_kv_cache_append_amd/csrc/kvq_decode.hip")
    valu = append_valu_roofline(c["name"] + ("-srft" if args.rotation == "srft" else ""), app_s)
    if valu is not None:
        result["append_roofline"] = valu
    if args.copy_calibration:
        src = torch.full((256 << 20,), 3, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(c, sample_b=4)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
