"""GPU parity of the per-channel rescale ("When Quantization Is Free", Methodology
sections 2 and 3: one scale per coordinate, then the per-group scales), through
the C ABI:

* kvq_calibrate_lambda bit-identical to the oracle's calibrated factors;
* kvq_append with factors: codes and metadata bit-identical to the oracle's
  (INT2: the clip thresholds calibrated on the rescaled vectors, also identical);
* kvq_decode_attn and kvq_block_mass with factors against the oracle (2e-3 per
  row; masses 1e-4 relative), on data with outlier channels;
* factors with the fp16 copy and the certified descriptors: codes, originals and
  descriptors against the oracle (descriptors in [exact, exact (1 + 2^-8)], the
  residuals taken in the unscaled basis), bound flags equal, certified decode and
  its certificate against the oracle, and the certificate bounding the error to
  dense attention.
"""
import numpy as np
import pytest
import torch

import bit_kv_cache_append_amd as kvq
import synth
from oracle import adaptive, attention, bound, codec
from gpu_harness import assert_bytes_equal, dev_bits, make_oracle_cache, setup_rotation

pytestmark = pytest.mark.gpu
TOL = 2e-3

CASES = {
    "int4-fwht-f16": synth.config(2, B=2, T=512),
    "int4-g128-none-outliers": synth.config(1, B=2, Hq=8, Hkv=2, T=384, rotation="none", k_group=128, v_group=128),
    "int2-dense-bf16-clip": synth.config(4, B=2, T=384, dtype="bf16"),
    "fp4-srft": synth.config(5, B=2, T=320, rotation="srft"),
    # the pairing the page describes: per-channel factors with groups of 16
    "int4-g16-srft": synth.config(2, B=2, T=320, rotation="srft", k_group=16, v_group=16),
}


def _calib(c):
    ck = np.stack([synth.calibration(c, 0, h) for h in range(c["Hkv"])])
    cv = np.stack([synth.calibration(c, 1, h) for h in range(c["Hkv"])])
    return ck, cv


@pytest.mark.parametrize("name", list(CASES))
def test_rescaled_cache_matches_oracle(name):
    c = CASES[name]
    print(f"[rescale] case {name}", flush=True)
    s, r16, s_dev, r_dev = setup_rotation(c)
    p = kvq.params_from_config(c)
    g = kvq.Cache(p, signs=s_dev, rot_f16=r_dev)
    ck, cv = _calib(c)
    lk, lv = kvq.calibrate_lambda(p, g, dev_bits(ck), dev_bits(cv))
    torch.cuda.synchronize()
    want_k = codec.calibrate_lambda(ck, c["dtype"], c["rotation"], s, r16)
    want_v = codec.calibrate_lambda(cv, c["dtype"], c["rotation"], s, r16)
    assert np.array_equal(lk.cpu().numpy(), want_k) and np.array_equal(lv.cpu().numpy(), want_v)
    g.lambda_k, g.lambda_v = lk, lv
    oc = make_oracle_cache(c)
    oc.lam_k, oc.lam_v = want_k, want_v
    clip = (None, None)
    if c["k_fmt"] == "int2":
        tk, tv = kvq.calibrate_clip(p, g, dev_bits(ck), dev_bits(cv), ratio=c["clip_ratio"])
        torch.cuda.synchronize()
        ok = codec.calibrate_clip(ck, c["dtype"], c["rotation"], s, r16, c["clip_ratio"], lam=want_k)
        ov = codec.calibrate_clip(cv, c["dtype"], c["rotation"], s, r16, c["clip_ratio"], lam=want_v)
        assert np.array_equal(tk.cpu().numpy(), ok) and np.array_equal(tv.cpu().numpy(), ov)
        g.clip_k, g.clip_v = tk, tv
        clip = (ok, ov)
    T = c["T"]
    k = synth.kv_all(c, 0, 0, T)
    v = synth.kv_all(c, 1, 0, T)
    kvq.append(p, g, dev_bits(k), dev_bits(v), [0] * c["B"])
    torch.cuda.synchronize()
    codec.append(oc, k, v, np.zeros(c["B"], int), c["dtype"], c["rotation"], s, r16, clip[0], clip[1],
                 c["scale_mode"])
    assert_bytes_equal(oc, g, name)
    seq = [T, T - 77]
    q = synth.queries(c)
    out = kvq.decode_attn(p, g, dev_bits(q), seq)
    mass = kvq.block_mass(p, g, dev_bits(q), seq)
    torch.cuda.synchronize()
    ref, _ = attention.decode_attention(oc, q, c["dtype"], np.array(seq), c["rotation"], s, r16)
    err = attention.row_rel_err(out.cpu().numpy(), ref).max()
    print(f"[rescale] {name}: max row rel err {err:.3e}", flush=True)
    assert err <= TOL
    mref = adaptive.block_mass(oc, q, c["dtype"], np.array(seq), c["rotation"], s, r16)
    got = mass.cpu().numpy()
    assert np.all(np.abs(got - mref) <= 1e-4 * np.abs(mref) + 1e-7)
    # the factors matter: the same codes read without them give a different attention
    plain = make_oracle_cache(c)
    for n in ("k_codes", "k_meta", "v_codes", "v_meta"):
        getattr(plain, n)[...] = getattr(oc, n)
    other, _ = attention.decode_attention(plain, q, c["dtype"], np.array(seq), c["rotation"], s, r16)
    assert attention.row_rel_err(other, ref).max() > 10 * TOL


@pytest.mark.parametrize("rotation", ["sign_fwht", "srft"])
def test_rescaled_certified_cache(rotation):
    """Factors together with the certified descriptors ("When Quantization Is Free",
    Methodology sections 2-3, with "Runtime-Certified Bounded-Error Quantized Attention",
    Methodology sections 1-2): the descriptors hold the residuals taken back to the unscaled
    basis, so the bound flags and the certificate keep their meaning."""
    c = synth.config(3, B=2, Hq=8, Hkv=2, T=1024, n_plant=3, rotation=rotation)  # 3 planted of 16 blocks
    print(f"[rescale] certified {rotation}", flush=True)
    s, r16, s_dev, r_dev = setup_rotation(c)
    p = kvq.params_from_config(c)
    g = kvq.Cache(p, signs=s_dev, rot_f16=r_dev)
    ck, cv = _calib(c)
    lk, lv = kvq.calibrate_lambda(p, g, dev_bits(ck), dev_bits(cv))
    torch.cuda.synchronize()
    g.lambda_k, g.lambda_v = lk, lv
    oc = make_oracle_cache(c)
    oc.lam_k, oc.lam_v = lk.cpu().numpy(), lv.cpu().numpy()
    T = c["T"]
    k = synth.kv_all(c, 0, 0, T)
    v = synth.kv_all(c, 1, 0, T)
    kvq.append(p, g, dev_bits(k), dev_bits(v), [0] * c["B"])
    torch.cuda.synchronize()
    codec.append(oc, k, v, np.zeros(c["B"], int), c["dtype"], c["rotation"], s, r16, None, None, c["scale_mode"])
    assert_bytes_equal(oc, g, f"certified-rescaled-{rotation}")
    seq = np.array([T, T - 77])
    want = bound.block_descriptors(oc, c["dtype"], c["rotation"], s, r16)
    got = g.bufs["blk_desc"].cpu().numpy().reshape(want.shape)
    assert np.all(got >= want), "descriptors must bound the exact errors"
    assert np.all(got <= want * (1 + 2.0 ** -8) + 1e-6 * np.abs(want).max()), "descriptors too loose"
    q = synth.queries(c)
    qd = dev_bits(q)
    _, fl = kvq.error_bound(p, g, qd, list(seq), c["tau"])
    out, cert = kvq.decode_attn(p, g, qd, list(seq), flags=fl, certificate=True)
    torch.cuda.synchronize()
    fln = fl.cpu().numpy()
    want_bnd, want_fl = bound.error_bound(want, q, c["dtype"], seq, c["tau"])
    # (the library's descriptors are rounded outward by up to 2^-8: blocks whose exact bound
    # lies that close to tau may go either way)
    sure = np.abs(want_bnd - c["tau"]) > 0.01 * c["tau"]
    assert np.array_equal(fln[sure], want_fl[sure]), "flags differ from the oracle's"
    ref, mass = attention.decode_attention(oc, q, c["dtype"], seq, c["rotation"], s, r16, flags=fln)
    err = attention.row_rel_err(out.cpu().numpy(), ref).max()
    print(f"[rescale] certified {rotation}: {int(fln.sum())} blocks flagged, max row rel err {err:.3e}", flush=True)
    assert err <= TOL
    E = cert.cpu().numpy()
    E_or = bound.certificate(want, q, c["dtype"], seq, fln, mass)
    assert np.all(E >= E_or * (1 - 1e-5)) and np.all(E <= E_or * (1 + 2.0 ** -7) + 1e-9)
    dense = attention.dense_attention(oc.k_orig, oc.v_orig, q, c["dtype"], seq)
    assert np.all(np.linalg.norm(ref - dense, axis=-1) <= E), "certificate must bound the error"
