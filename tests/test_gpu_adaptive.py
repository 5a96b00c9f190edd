"""GPU parity of adaptive precision ("Runtime-Certified Bounded-Error Quantized
Attention", Methodology section 3), through the C ABI:

* kvq_block_mass against the oracle's fp64 block masses over the library's own
  codes (decoded by the oracle's unpacker): |got - ref| <= 1e-4 |ref| + 1e-7;
* kvq_select_blocks bit-identical to the oracle's selection applied to the
  library's own fp32 masses (the choice is a function of those masses; the
  masses themselves are checked against the oracle above), with and without the
  bound's flags, in place;
* the whole ladder on the certified workload: bound flags, scoring pass, top-K*
  promotion, decode with the promoted flags and the certificate, and the dense
  fallback of the heads whose certificate exceeds eps - against the oracle's
  attention with the same flags (2e-3 per row) and dense attention for the rows
  that fell back.
"""
import numpy as np
import pytest
import torch

import bit_kv_cache_append_amd as kvq
import synth
from oracle import adaptive, attention, bound
from gpu_harness import dev_bits, make_gpu_cache, oracle_view_of_gpu, setup_rotation

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _filled(c):
    s, r16, s_dev, r_dev = setup_rotation(c)
    p, g = make_gpu_cache(c, s_dev, r_dev)
    if c["k_fmt"] == "int2" or c["v_fmt"] == "int2":
        ck = np.stack([synth.calibration(c, 0, h) for h in range(c["Hkv"])])
        cv = np.stack([synth.calibration(c, 1, h) for h in range(c["Hkv"])])
        g.clip_k, g.clip_v = kvq.calibrate_clip(p, g, dev_bits(ck), dev_bits(cv), ratio=c.get("clip_ratio", 0.9))
    k = synth.kv_all(c, 0, 0, c["T"])
    v = synth.kv_all(c, 1, 0, c["T"])
    kvq.append(p, g, dev_bits(k), dev_bits(v), [0] * c["B"])
    torch.cuda.synchronize()
    return s, r16, p, g


CASES = {
    "int8k-int4v-certified": (synth.config(3, B=2, T=2048), [2048, 1500]),
    "int4-gqa-ragged": (synth.config(2, B=3, T=1088), [1088, 1000, 0]),
    "int4-g128-none": (synth.config(1, B=2, Hq=8, Hkv=2, T=512, rotation="none", k_group=128, v_group=128),
                       [512, 65]),
    "int2-dense-bf16": (synth.config(4, B=2, T=1024, dtype="bf16"), [1024, 777]),
    "fp4-search": (synth.config(5, B=2, T=1024), [1024, 701]),
    "int4-srft": (synth.config(2, B=2, T=640, rotation="srft"), [640, 300]),
    "int4-g16": (synth.config(2, B=2, T=640, k_group=16, v_group=16), [640, 129]),
    # two groups of four query heads per kv head, and a partial group of two
    "int4-gqa8-two-groups": (synth.config(2, B=2, Hq=16, Hkv=2, T=640), [640, 513]),
    "int8k-int4v-gqa2": (synth.config(3, B=1, Hq=4, Hkv=2, T=512), [450]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_block_mass_and_selection_match_oracle(name):
    c, seq = CASES[name]
    print(f"[adaptive] case {name}", flush=True)
    s, r16, p, g = _filled(c)
    q = synth.queries(c)
    qd = dev_bits(q)
    mass = kvq.block_mass(p, g, qd, seq)
    torch.cuda.synchronize()
    got = mass.cpu().numpy()
    oc = oracle_view_of_gpu(c, g)
    ref = adaptive.block_mass(oc, q, c["dtype"], np.array(seq), c["rotation"], s, r16)
    err = np.abs(got - ref) - (1e-4 * np.abs(ref) + 1e-7)
    print(f"[adaptive] {name}: max |mass - ref| {np.abs(got - ref).max():.3e}", flush=True)
    assert (err <= 0).all(), f"{name}: block mass off by {np.abs(got - ref).max():.3e}"
    for b in range(c["B"]):
        nb = (seq[b] + 63) // 64
        assert not got[b, :, nb:].any()
    for tau in (0.0, 0.5, 0.9, 0.995, 1.0):
        fl = kvq.select_blocks(p, mass, seq, tau)
        torch.cuda.synchronize()
        want = adaptive.select_blocks(got, np.array(seq), tau, c["Hkv"])
        assert np.array_equal(fl.cpu().numpy(), want), f"{name}: selection differs at tau_cov {tau}"
    with pytest.raises(kvq.KvqError) as e:  # coverage is a fraction: the call rejects 2
        kvq.select_blocks(p, mass, seq, 2.0)
    assert e.value.status == -1
    # union with given flags, in place
    base = np.zeros((c["B"], c["Hkv"], c["T"] // 64), np.uint8)
    base[:, :, 1] = 1
    fl = torch.from_numpy(base.copy()).cuda()
    kvq.select_blocks(p, mass, seq, 0.9, flags_in=fl, flags_out=fl)
    torch.cuda.synchronize()
    assert np.array_equal(fl.cpu().numpy(), adaptive.select_blocks(got, np.array(seq), 0.9, c["Hkv"], base))


# With N(0,1) queries the attention over this cache is diffuse: covering 99.5 % of the
# estimated mass promotes most blocks and leaves every certificate at 0; covering half of it
# leaves certificates above eps, so heads must fall back.
@pytest.mark.parametrize("tau_cov,eps_q,must_fall_back", [(0.995, 0.5, False), (0.5, 0.5, True), (0.5, 0.0, True)])
def test_adaptive_ladder_on_the_certified_cache(tau_cov, eps_q, must_fall_back):
    c = synth.config(3, B=2, T=4096)
    seq = [4096, 3000]
    print(f"[adaptive] ladder tau_cov={tau_cov}", flush=True)
    s, r16, p, g = _filled(c)
    q = synth.queries(c)
    qd = dev_bits(q)
    _, bflags = kvq.error_bound(p, g, qd, seq, c["tau"])
    mass = kvq.block_mass(p, g, qd, seq)
    flags = kvq.select_blocks(p, mass, seq, tau_cov, flags_in=bflags)
    out, cert = kvq.decode_attn(p, g, qd, seq, flags=flags, certificate=True)
    torch.cuda.synchronize()
    out0, cert0 = out.cpu().numpy().copy(), cert.cpu().numpy().copy()
    fln = flags.cpu().numpy()
    want_flags = adaptive.select_blocks(mass.cpu().numpy(), np.array(seq), tau_cov, c["Hkv"], bflags.cpu().numpy())
    assert np.array_equal(fln, want_flags)
    n_bound, n_all = int(bflags.sum().item()), int(fln.sum())
    print(f"[adaptive] blocks flagged by the bound {n_bound}, promoted in all {n_all} of {fln.size}", flush=True)
    assert n_all >= n_bound
    oc = oracle_view_of_gpu(c, g)
    ref, pmass = attention.decode_attention(oc, q, c["dtype"], np.array(seq), c["rotation"], s, flags=fln)
    rows = [(b, hq) for b in range(c["B"]) for hq in range(c["Hq"])]
    err = attention.row_rel_err(out0, ref)
    assert max(err[b, hq] for b, hq in rows) <= TOL
    desc = bound.block_descriptors(oc, c["dtype"], c["rotation"], s)
    E_or = bound.certificate(desc, q, c["dtype"], np.array(seq), fln, pmass)
    assert np.all(cert0 >= E_or * (1 - 1e-5)) and np.all(cert0 <= E_or * (1 + 2.0 ** -7) + 1e-9)
    # rung 3: heads whose certificate exceeds eps are recomputed densely
    eps = float(np.quantile(cert0, eps_q))
    kvq.dense_fallback(p, g, qd, seq, eps, out, cert)
    torch.cuda.synchronize()
    out1, cert1 = out.cpu().numpy(), cert.cpu().numpy()
    dense = attention.dense_attention(oc.k_orig, oc.v_orig, q, c["dtype"], np.array(seq))
    want_out, want_cert, redo = adaptive.dense_fallback(out0, cert0, eps, dense)
    print(f"[adaptive] eps {eps:.3e}: {int(redo.sum())} of {redo.size} heads fell back", flush=True)
    assert redo.any() or not must_fall_back
    assert np.array_equal(cert1, want_cert.astype(np.float32))
    assert np.array_equal(out1[~redo], out0[~redo])
    if redo.any():
        assert attention.row_rel_err(out1[redo], dense[redo]).max() <= TOL
    # after the fallback every row's exact-arithmetic result is within its certificate of dense
    # attention (the rows that fell back are dense attention, certificate 0)
    exact = np.where(redo[..., None], dense, ref)
    assert np.all(np.linalg.norm(exact - dense, axis=-1) <= want_cert + 1e-12)
