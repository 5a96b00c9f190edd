"""GPU test of kvq_decode_attn_noalloc (the decode on the library's fixed per-device
workspace) against kvq_decode_attn with a caller workspace, through the C ABI.

Two calls in a row on the fixed workspace, the second with a smaller input (fewer
sequences, shorter contexts, another cache shape), then a certified call with flags
and certificate.  Each output is compared with the workspace entry point's output on
the same inputs and with the oracle's fp64 attention over the same packed bytes, per
output row max |a - b| / max |b| <= 2e-3; the certificates within 2^-7 relative.
"""
import numpy as np
import pytest
import torch

import bit_kv_cache_append_amd as kvq
import synth
from oracle import attention
from gpu_harness import dev_bits, make_gpu_cache, oracle_view_of_gpu, setup_rotation

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _case(c, seq):
    s, r16, s_dev, r_dev = setup_rotation(c)
    p, gcache = make_gpu_cache(c, s_dev, r_dev)
    T = c["T"]
    k = synth.kv_all(c, 0, 0, T)
    v = synth.kv_all(c, 1, 0, T)
    kvq.append(p, gcache, dev_bits(k), dev_bits(v), [0] * c["B"])
    torch.cuda.synchronize()
    return s, r16, p, gcache


def _rows_close(got, ref, tag):
    err = attention.row_rel_err(got, ref)
    print(f"[noalloc] {tag}: max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= TOL, f"{tag}: {err.max():.3e}"


def test_noalloc_two_calls_second_smaller():
    big = synth.config(2, B=3, T=1088)
    small = synth.config(2, B=2, Hq=8, Hkv=2, T=320)
    for name, c, seq in (("larger", big, [1088, 1000, 65]), ("smaller", small, [320, 129])):
        print(f"[noalloc] call {name}: B={c['B']} Hq={c['Hq']} Hkv={c['Hkv']} seq={seq}", flush=True)
        s, r16, p, gcache = _case(c, seq)
        q = synth.queries(c)
        qd = dev_bits(q)
        out_na = kvq.decode_attn_noalloc(p, gcache, qd, seq)
        torch.cuda.synchronize()
        out_na = out_na.cpu().numpy()
        out_ws = kvq.decode_attn(p, gcache, qd, seq).cpu().numpy()
        _rows_close(out_na, out_ws, f"{name}: noalloc vs workspace")
        oc = oracle_view_of_gpu(c, gcache)
        ref, _ = attention.decode_attention(oc, q, c["dtype"], np.array(seq), c["rotation"], s, r16)
        _rows_close(out_na, ref, f"{name}: noalloc vs oracle")


def test_noalloc_certified_flags_and_certificate():
    c = synth.config(3, B=2, T=1024)
    seq = [1024, 700]
    print(f"[noalloc] certified call: seq={seq}", flush=True)
    s, r16, p, gcache = _case(c, seq)
    q = synth.queries(c)
    qd = dev_bits(q)
    _, flags = kvq.error_bound(p, gcache, qd, seq, c["tau"])
    out_na, cert_na = kvq.decode_attn_noalloc(p, gcache, qd, seq, flags=flags, certificate=True)
    out_ws, cert_ws = kvq.decode_attn(p, gcache, qd, seq, flags=flags, certificate=True)
    torch.cuda.synchronize()
    _rows_close(out_na.cpu().numpy(), out_ws.cpu().numpy(), "certified: noalloc vs workspace")
    cn, cw = cert_na.cpu().numpy(), cert_ws.cpu().numpy()
    assert np.all(np.abs(cn - cw) <= cw * 2.0 ** -7 + 1e-12), f"certificates differ: {cn} vs {cw}"
