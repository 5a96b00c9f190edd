"""Workloads for the layout-checking library (not a test module: test_gpu_debug_build.py
runs it).  Every entry point over every key/value format, rotation, the window, the
certified cache, the adaptive ladder and the per-channel factors, at small shapes with
ragged sequences and appends in pieces.  run_all() returns the outputs by name; run as a
script in a process of its own, with KVQ_LIB naming the library to load, it saves them to
an .npz file and prints one JSON line with the library's debug status:

    KVQ_LIB=bit_kv_cache_append_amd/libkvq_debug.so python tests/debug_layout_run.py OUT.npz
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for _p in (ROOT, HERE):
    if _p not in sys.path:
        sys.path.insert(0, _p)

import bit_kv_cache_append_amd as kvq  # noqa: E402
import synth  # noqa: E402
from gpu_harness import dev_bits, setup_rotation  # noqa: E402

# (name, workload, sequence lengths, append pieces)
CASES = [
    ("c1-int4-pieces", synth.config(1), [1024], [600, 424]),
    ("c2-int4-ragged", synth.config(2, B=3, T=2112), [2112, 2000, 65], [1088, 1024]),
    ("int4-g16-srft", synth.config(2, B=2, T=320, rotation="srft", k_group=16, v_group=16), [320, 257], [320]),
    ("int8k-int4v-g128", synth.config(1, B=2, Hq=8, Hkv=2, T=384, k_fmt="int8", v_fmt="int4", k_group=128,
                                      v_group=128), [384, 100], [200, 184]),
    ("int2-dense", synth.config(4, B=2, T=384), [384, 321], [384]),
    ("int2-fwht", synth.config(4, B=2, T=256, rotation="sign_fwht"), [256, 200], [256]),
    ("fp4-srft", synth.config(5, B=2, T=320, rotation="srft"), [320, 130], [320]),
    ("int4-window", synth.config(2, B=2, T=640, sink_blocks=1, recent_blocks=2), [640, 500], [300, 340]),
    ("fp4-window", synth.config(5, B=2, T=448, sink_blocks=1, recent_blocks=1), [448, 448], [448]),
    ("certified", synth.config(3, B=2, Hq=8, Hkv=2, T=4096, n_plant=3), [4096, 3947], [4096]),
    ("certified-window", synth.config(3, B=2, Hq=8, Hkv=2, T=1024, n_plant=3, sink_blocks=1, recent_blocks=2),
     [1024, 700], [512, 512]),
    ("int4-lambda", synth.config(2, B=2, T=512), [512, 435], [512]),
]


def _calib(c):
    ck = np.stack([synth.calibration(c, 0, h) for h in range(c["Hkv"])])
    cv = np.stack([synth.calibration(c, 1, h) for h in range(c["Hkv"])])
    return dev_bits(ck), dev_bits(cv)


def run_all():
    """Outputs by name: '<case>/<buffer>' (bit-exact ones) and '<case>/out...' (decodes)."""
    import torch
    res = {}
    for name, c, seq, pieces in CASES:
        print(f"[debug-build] {name}", flush=True)
        s, r16, s_dev, r_dev = setup_rotation(c)
        p = kvq.params_from_config(c)
        g = kvq.Cache(p, signs=s_dev, rot_f16=r_dev)
        if c["k_fmt"] == "int2":
            g.clip_k, g.clip_v = kvq.calibrate_clip(p, g, *_calib(c), ratio=c["clip_ratio"])
        if name.endswith("lambda"):
            g.lambda_k, g.lambda_v = kvq.calibrate_lambda(p, g, *_calib(c))
        t0 = 0
        for n in pieces:
            k = synth.kv_all(c, 0, t0, n)
            v = synth.kv_all(c, 1, t0, n)
            kvq.append(p, g, dev_bits(k), dev_bits(v), [t0] * c["B"])
            t0 += n
        q = dev_bits(synth.queries(c))
        for bn, t in g.bufs.items():
            if t is not None:
                res[f"{name}/{bn}"] = t
        res[f"{name}/out"] = kvq.decode_attn(p, g, q, seq)
        res[f"{name}/out_noalloc"] = kvq.decode_attn_noalloc(p, g, q, seq)
        if c["keep"]:
            _, fl = kvq.error_bound(p, g, q, seq, c["tau"])
            res[f"{name}/bound_flags"] = fl.clone()
            mass = kvq.block_mass(p, g, q, seq)
            sel = kvq.select_blocks(p, mass, seq, 0.9, flags_in=fl)
            kvq.promote_values(p, g, mass, seq, 1e-4, sel)
            inv, fail = kvq.ranking_check(p, g, q, seq, mass, 0.9, margin=0.0, max_inversions=0)
            out, cert = kvq.decode_attn(p, g, q, seq, flags=sel, certificate=True)
            kvq.dense_fallback(p, g, q, seq, 1e-3, out, cert, fail=fail)
            res.update({f"{name}/mass": mass, f"{name}/flags": sel, f"{name}/inversions": inv,
                        f"{name}/out_ladder": out, f"{name}/cert_ladder": cert})
        elif c["rotation"] != "dense":
            res[f"{name}/mass"] = kvq.block_mass(p, g, q, seq)
    # the fp16 same-shape decode over uncompressed rows
    c = synth.config(2, B=2, T=1088)
    print("[debug-build] fp16 decode", flush=True)
    p = kvq.params_from_config(c, rotation="none")
    k = dev_bits(synth.kv_all(c, 0, 0, c["T"]))
    v = dev_bits(synth.kv_all(c, 1, 0, c["T"]))
    res["fp16/out"] = kvq.decode_attn_dense(p, k, v, dev_bits(synth.queries(c)), [1088, 77])
    torch.cuda.synchronize()
    return {n: t.cpu().numpy() for n, t in res.items()}


if __name__ == "__main__":
    out = run_all()
    np.savez(sys.argv[1], **{n.replace("/", "|"): a for n, a in out.items()})
    code, i0, i1, count = kvq.debug_status(clear=True)
    print(json.dumps({"lib": os.path.basename(kvq.LIB_PATH), "code": code, "index0": i0, "index1": i1,
                      "failures": count, "outputs": len(out)}), flush=True)
