#!/usr/bin/env python3
"""Decode-attention and append throughput of the int4 KV cache on one MI355X.

Workload (Llama-3-8B-shaped GQA decode): B=16 sequences, 32 query heads over 8
kv heads, head_dim 128, context 8192; fp16 K/V N(0,1) with 10 seeded (head,
channel) pairs x8; sign + Walsh-Hadamard rotation; symmetric int4 with one fp16
scale per 32 channels for K and V.

One step = the whole hot path over one batch:
  1. kvq_append of a 4096-token prefill into every sequence (positions
     4096..8191; 16 x 8 x 4096 K and V vectors), then
  2. kvq_decode_attn of one query token per (sequence, query head) over all 8192
     positions.
Before each timed kernel the L2 and the 256 MB Infinity Cache are flushed by
reading a 1 GiB buffer (a reduction; reading leaves only clean lines behind, so
no write-back lands inside the timed kernel), so the packed cache (144 MiB) is
read from HBM.  Each
kernel is bracketed by HIP events on the stream it runs on.

value = decode effective KV GB/s = packed K/V bytes (codes + scales) / mean
decode time.  The same-shape fp16 decode (kvq_decode_attn_dense) is timed the
same way for the int4-vs-fp16 comparison; append throughput is reported in
Mvec/s.  The CPU oracle is timed on a bounded sample as a reported baseline.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
METRIC = "decode-attn effective KV GB/s & % HBM peak (int4 vs fp16); append Mvec/s"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workers", type=int, default=min(16, os.cpu_count() or 1))
    return ap.parse_args()


def cpu_baseline(c, sample_b):
    """Time the oracle on sample_b sequences of the same workload (reported baseline only)."""
    from threadpoolctl import threadpool_limits
    import synth
    from oracle import attention, codec
    T, P = c["T"], c["prefill"]
    H = c["Hkv"]
    with threadpool_limits(1):
        cs = synth.config(2, B=sample_b)
        k = synth.kv_all(cs, 0, 0, T)
        v = synth.kv_all(cs, 1, 0, T)
        s = synth.signs(cs)
        oc = codec.Cache(sample_b, H, T, cs["k_fmt"], cs["v_fmt"], cs["k_group"], cs["v_group"])
        codec.append(oc, k[:, :, :T - P], v[:, :, :T - P], np.zeros(sample_b, int), "f16", "sign_fwht", s,
                     scale_mode=cs["scale_mode"])
        t0 = time.perf_counter()
        codec.append(oc, k[:, :, T - P:], v[:, :, T - P:], np.full(sample_b, T - P), "f16", "sign_fwht", s,
                     scale_mode=cs["scale_mode"])
        t_app = time.perf_counter() - t0
        q = synth.queries(cs)
        t0 = time.perf_counter()
        attention.decode_attention(oc, q, "f16", np.full(sample_b, T), "sign_fwht", s)
        t_dec = time.perf_counter() - t0
    kv_bytes = sample_b * H * T * 144
    vecs = sample_b * H * P * 2
    return {
        "value": kv_bytes / t_dec / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": (f"{sample_b} of {c['B']} sequences: decode over {T} tokens (all {c['Hq']} q heads) took "
                   f"{t_dec:.2f} s; the {P}-token prefill append of those sequences ({vecs} vectors) took "
                   f"{t_app:.2f} s"),
        "append_mvec_s": vecs / t_app / 1e6,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one MI355X; --gpus {args.gpus} is not supported (this build runs on one GPU).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_kv_cache_append_amd as kvq
    import synth

    kvq.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    c = synth.config(2)
    B, Hq, H, T, P = c["B"], c["Hq"], c["Hkv"], c["T"], c["prefill"]
    t_gen = time.perf_counter()
    k_all = synth.kv_all(c, 0, 0, T, workers=args.workers)
    v_all = synth.kv_all(c, 1, 0, T, workers=args.workers)
    q_np = synth.queries(c)
    t_gen = time.perf_counter() - t_gen
    k_dev = kvq.to_device_bits(k_all)
    v_dev = kvq.to_device_bits(v_all)
    del k_all, v_all
    q = kvq.to_device_bits(q_np)
    k_pre = k_dev[:, :, T - P:].contiguous()
    v_pre = v_dev[:, :, T - P:].contiguous()
    s_dev = torch.from_numpy(synth.signs(c).copy()).to(dev)
    p = kvq.params_from_config(c)
    cache = kvq.Cache(p, signs=s_dev)
    ws = kvq.workspace(p)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
    seq = [T] * B
    # context [0, T - P) once, untimed
    kvq.append(p, cache, k_dev[:, :, :T - P].contiguous(), v_dev[:, :, :T - P].contiguous(), [0] * B)
    flush_buf = torch.ones(1 << 27, dtype=torch.int64, device=dev)  # 1 GiB
    sink = torch.zeros((), dtype=torch.int64, device=dev)

    def flush():
        torch.sum(flush_buf, dim=0, out=sink)

    torch.cuda.synchronize()

    def step(i, ev):
        flush()
        ev[0].record()
        kvq.append(p, cache, k_pre, v_pre, [T - P] * B)
        ev[1].record()
        flush()
        ev[2].record()
        kvq.decode_attn(p, cache, q, seq, ws=ws, out=out)
        ev[3].record()

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for i in range(args.warmup):
        step(i, mk())
    torch.cuda.synchronize()
    events = [mk() for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    app_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    dec_ms = np.array([e[2].elapsed_time(e[3]) for e in events])

    # same-shape fp16 decode (dense K/V already resident: the inputs themselves)
    dws = kvq.workspace(p)
    dout = torch.empty_like(out)
    fev = []
    for i in range(args.warmup + args.steps):
        flush()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        kvq.decode_attn_dense(p, k_dev, v_dev, q, seq, ws=dws, out=dout)
        e[1].record()
        if i >= args.warmup:
            fev.append(e)
    torch.cuda.synchronize()
    f16_ms = np.array([e[0].elapsed_time(e[1]) for e in fev])
    rel = (out - dout).abs().amax(dim=-1) / dout.abs().amax(dim=-1)
    int4_vs_fp16_maxrel = float(rel.max().item())

    kv_bytes = B * H * T * (64 + 8) * 2           # packed K and V: codes + fp16 group scales
    io_bytes = B * Hq * 128 * 2 + B * Hq * 128 * 4  # query in, fp32 output out
    f16_bytes = B * H * T * 128 * 2 * 2
    vecs = B * H * P * 2
    app_bytes = vecs * (256 + 72)
    dec_s = dec_ms.mean() / 1e3
    f16_s = f16_ms.mean() / 1e3
    app_s = app_ms.mean() / 1e3
    dec_gbs = kv_bytes / dec_s / 1e9
    result = {
        "metric": METRIC,
        "value": round(dec_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4",
        "data": "synthetic (seeded fp16 N(0,1) K/V with outlier channels; no model weights)",
        "config": {"workload": "llama3-8b-shaped GQA int4 decode + prefill append", "B": B, "Hq": Hq, "Hkv": H,
                   "head_dim": 128, "context": T, "prefill_tokens": P, "k_fmt": "int4 g32", "v_fmt": "int4 g32",
                   "rotation": "sign+fwht"},
        "roofline": {"bound": "hbm", "achieved": round((kv_bytes + io_bytes) / dec_s / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round((kv_bytes + io_bytes) / dec_s / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "decode_split<int4,g32,int4> (one launch per kvq_decode_attn)"},
        "decode_us": round(dec_s * 1e6, 2),
        "decode_pct_hbm_peak": round(100 * dec_gbs / HBM_PEAK_GBS, 2),
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
        "input_gen_s": round(t_gen, 2),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(c, sample_b=8)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
