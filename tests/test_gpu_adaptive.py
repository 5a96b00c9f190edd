"""GPU parity of adaptive precision ("Runtime-Certified Bounded-Error Quantized
Attention", Methodology section 3), through the C ABI:

* kvq_block_mass against the oracle's fp64 block masses over the library's own
  codes (decoded by the oracle's unpacker): |got - ref| <= 1e-4 |ref| + 1e-7;
* kvq_select_blocks bit-identical to the oracle's selection applied to the
  library's own fp32 masses (the choice is a function of those masses; the
  masses themselves are checked against the oracle above), with and without the
  bound's flags, in place; and equal to the selection from the oracle's own fp64
  masses for every kv head whose query heads have no near tie at their cut;
* the whole ladder on the certified workload: bound flags, scoring pass, top-K*
  promotion, decode with the promoted flags and the certificate, and the dense
  fallback of the heads whose certificate exceeds eps - against the oracle's
  attention with the same flags (2e-3 per row) and dense attention for the rows
  that fell back;
* on the certified workload with retrieval needles (peaked attention, top-K* of a
  few blocks): kvq_promote_values bit-identical to the oracle's rung 2 applied to
  the library's fp32 masses and descriptors, and in agreement with the oracle's
  fp64 masses and descriptors wherever the product is not within 2 % of tau_v;
  decode with value-only flags against the oracle's attention and certificate;
  kvq_ranking_check's inversion count inside the oracle's [lo, hi] (fp64 block
  scores from the originals, pairs within 1e-3 of the margin counted as either)
  and its fail flags where that range decides them; and the ladder with every
  rung, fallback triggered by the check as well as the certificate.
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


def _unambiguous_heads(mass64, seq, tau, n_kv):
    """[B, Hkv] True where every query head's top-K* cut is clear of ties and of tau_cov."""
    B, Hq, _ = mass64.shape
    G = Hq // n_kv
    ok = np.ones((B, n_kv), bool)
    for b in range(B):
        nb = (int(seq[b]) + 63) // 64
        if nb == 0:
            continue
        for hq in range(Hq):
            m = mass64[b, hq, :nb]
            order = sorted(range(nb), key=lambda i: (-m[i], i))
            run = np.cumsum(m[order])
            k = len(adaptive.top_blocks(m.astype(np.float32), nb, tau))
            near_tau = np.any(np.abs(run - tau) < 2e-4)
            tie = k < nb and abs(m[order[k - 1]] - m[order[k]]) <= 2e-4 * max(m[order[k - 1]], 1e-30)
            if near_tau or tie:
                ok[b, hq // G] = False
    return ok


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
        fln = fl.cpu().numpy()
        want = adaptive.select_blocks(got, np.array(seq), tau, c["Hkv"])
        assert np.array_equal(fln, want), f"{name}: selection differs at tau_cov {tau}"
        # independent of the library's masses: the oracle's own fp64 masses choose the same
        # blocks for every kv head none of whose query heads has a near tie at its cut
        # (a running sum within 2e-4 of tau_cov, or equal masses within 2e-4 across the cut)
        sure = _unambiguous_heads(ref, np.array(seq), tau, c["Hkv"])
        want64 = adaptive.select_blocks(ref.astype(np.float32), np.array(seq), tau, c["Hkv"])
        assert np.array_equal(fln[sure], want64[sure]), f"{name}: selection from fp64 masses differs at {tau}"
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


# ---------------------------------------------------------------- retrieval needles: rungs 2 and 3
NEEDLES = synth.config(3, B=2, T=4096, needles=4)
WIN = 1e-3  # fp32 block scores: log-sum-exp of 64 dot products of 128 terms, |logits| <= ~25


def _needle_state(seq):
    c = NEEDLES
    s, r16, p, g = _filled(c)
    q = synth.queries(c)
    qd = dev_bits(q)
    mass = kvq.block_mass(p, g, qd, seq)
    torch.cuda.synchronize()
    return c, s, p, g, q, qd, mass


def _ev(c, g):
    return g.bufs["blk_desc"].view(c["B"], c["Hkv"], c["T"] // 64, 3)[..., 1].cpu().numpy()


@pytest.mark.parametrize("tau_cov,tau_v", [(0.5, 1e-4), (0.9, 1e-6), (0.995, 0.0)])
def test_promote_values_matches_oracle(tau_cov, tau_v):
    seq = [4096, 3000]
    print(f"[adaptive] promote values tau_cov={tau_cov} tau_v={tau_v}", flush=True)
    c, s, p, g, q, qd, mass = _needle_state(seq)
    fl = kvq.select_blocks(p, mass, seq, tau_cov)
    torch.cuda.synchronize()
    f0 = fl.cpu().numpy().copy()
    kvq.promote_values(p, g, mass, seq, tau_v, fl)
    torch.cuda.synchronize()
    got = fl.cpu().numpy()
    m32 = mass.cpu().numpy()
    want = adaptive.promote_values(m32, _ev(c, g), np.array(seq), tau_v, c["Hkv"], f0)
    assert np.array_equal(got, want)
    nval = int(((got & 3) == 2).sum())
    print(f"[adaptive] {int((got & 1).sum())} blocks promoted, {nval} value-promoted of {got.size}", flush=True)
    # the oracle's own fp64 masses and descriptors choose the same blocks away from the threshold
    oc = oracle_view_of_gpu(c, g)
    ref_mass = adaptive.block_mass(oc, q, c["dtype"], np.array(seq), c["rotation"], s)
    desc = bound.block_descriptors(oc, c["dtype"], c["rotation"], s)
    G = c["Hq"] // c["Hkv"]
    prod = (ref_mass.reshape(c["B"], c["Hkv"], G, -1) * desc[..., 1][:, :, None, :]).max(axis=2)
    nb = np.array([(t + 63) // 64 for t in seq])
    live = (np.arange(prod.shape[-1])[None, None, :] < nb[:, None, None]) & ((f0 & 1) == 0)
    sure = live & (np.abs(prod - tau_v) > 0.02 * tau_v + 1e-12)
    assert np.array_equal(((got & 2) != 0)[sure], (prod > tau_v)[sure])
    if tau_v > 0 and tau_cov < 0.9:
        assert nval > 0, "the case must promote some values"


def test_value_promoted_decode_matches_oracle():
    seq = [4096, 3000]
    print("[adaptive] decode with value-only flags", flush=True)
    c, s, p, g, q, qd, mass = _needle_state(seq)
    fl = kvq.select_blocks(p, mass, seq, 0.5)
    kvq.promote_values(p, g, mass, seq, 1e-4, fl)
    out, cert = kvq.decode_attn(p, g, qd, seq, flags=fl, certificate=True)
    torch.cuda.synchronize()
    fln = fl.cpu().numpy()
    assert ((fln & 3) == 2).any() and ((fln & 1) != 0).any()
    oc = oracle_view_of_gpu(c, g)
    ref, pmass = attention.decode_attention(oc, q, c["dtype"], np.array(seq), c["rotation"], s, flags=fln)
    err = attention.row_rel_err(out.cpu().numpy(), ref)
    print(f"[adaptive] value-only flags: max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= TOL
    desc = bound.block_descriptors(oc, c["dtype"], c["rotation"], s)
    E_or = bound.certificate(desc, q, c["dtype"], np.array(seq), fln, pmass)
    E = cert.cpu().numpy()
    assert np.all(E >= E_or * (1 - 1e-5)) and np.all(E <= E_or * (1 + 2.0 ** -7) + 1e-9)
    # value promotion must lower the certificate against the same keys without it
    _, cert0 = kvq.decode_attn(p, g, qd, seq, flags=torch.from_numpy(fln & 1).cuda(), certificate=True)
    torch.cuda.synchronize()
    assert np.all(E <= cert0.cpu().numpy() * (1 + 1e-6))


# (with both sequences whole, the near-tie needles of sequence 1's first kv head are in range)
@pytest.mark.parametrize("tau_cov,margin,max_inv,seq", [(0.995, 0.0, 0, [4096, 4096]), (0.995, 0.05, 0, [4096, 3000]),
                                                        (1.0, 0.0, 3, [4096, 3000])])
def test_ranking_check_matches_oracle(tau_cov, margin, max_inv, seq):
    print(f"[adaptive] ranking check tau_cov={tau_cov} margin={margin} max_inv={max_inv}", flush=True)
    c, s, p, g, q, qd, mass = _needle_state(seq)
    inv, fail = kvq.ranking_check(p, g, qd, seq, mass, tau_cov, margin, max_inv)
    torch.cuda.synchronize()
    got, gfail = inv.cpu().numpy(), fail.cpu().numpy()
    oc = oracle_view_of_gpu(c, g)
    score = adaptive.block_scores_fp16(oc.k_orig, q, c["dtype"], np.array(seq))
    lo, hi = adaptive.ranking_inversions(mass.cpu().numpy(), score, np.array(seq), tau_cov, margin, window=WIN)
    print(f"[adaptive] inversions: max {got.max()}, heads with some {int((got > 0).sum())} of {got.size}, "
          f"undecided pairs in {int((lo != hi).sum())} heads", flush=True)
    assert np.all((lo <= got) & (got <= hi)), (got, lo, hi)
    assert np.array_equal(gfail != 0, got > max_inv)
    decided = (lo > max_inv) == (hi > max_inv)
    assert np.array_equal((gfail != 0)[decided], (lo > max_inv)[decided])
    if tau_cov == 0.995 and margin == 0.0:
        assert (got > 0).any(), "the near ties of the needle workload invert some heads"
        assert np.array_equal(gfail != 0, got > 0)


def test_ranking_check_empty_and_short_sequences():
    seq = [0, 70]
    c, s, p, g, q, qd, mass = _needle_state(seq)
    inv, fail = kvq.ranking_check(p, g, qd, seq, mass, 1.0, 0.0, 0)
    torch.cuda.synchronize()
    oc = oracle_view_of_gpu(c, g)
    score = adaptive.block_scores_fp16(oc.k_orig, q, c["dtype"], np.array(seq))
    lo, hi = adaptive.ranking_inversions(mass.cpu().numpy(), score, np.array(seq), 1.0, 0.0, window=WIN)
    got = inv.cpu().numpy()
    assert not got[0].any() and not fail.cpu().numpy()[0].any()
    assert np.all((lo <= got) & (got <= hi))


@pytest.mark.parametrize("tau_cov,tau_v,eps", [(0.995, 1e-6, 1e-3), (0.9, 1e-5, 0.0)])
def test_adaptive_ladder_with_needles(tau_cov, tau_v, eps):
    seq = [4096, 4096]
    print(f"[adaptive] needle ladder tau_cov={tau_cov} tau_v={tau_v} eps={eps}", flush=True)
    c, s, p, g, q, qd, mass = _needle_state(seq)
    _, bflags = kvq.error_bound(p, g, qd, seq, c["tau"])
    flags = kvq.select_blocks(p, mass, seq, tau_cov, flags_in=bflags)
    kvq.promote_values(p, g, mass, seq, tau_v, flags)
    inv, fail = kvq.ranking_check(p, g, qd, seq, mass, tau_cov, 0.0, 0)
    out, cert = kvq.decode_attn(p, g, qd, seq, flags=flags, certificate=True)
    torch.cuda.synchronize()
    out0, cert0, fl0 = out.cpu().numpy().copy(), cert.cpu().numpy().copy(), fail.cpu().numpy().copy()
    m32 = mass.cpu().numpy()
    want = adaptive.promote_values(m32, _ev(c, g), np.array(seq), tau_v,
                                   c["Hkv"], adaptive.select_blocks(m32, np.array(seq), tau_cov, c["Hkv"],
                                                                    bflags.cpu().numpy()))
    fln = flags.cpu().numpy()
    assert np.array_equal(fln, want)
    # peaked attention: every head's top-K* is a handful of blocks
    kstar = max(len(adaptive.top_blocks(m32[b, hq], 64, tau_cov)) for b in range(2) for hq in range(c["Hq"]))
    print(f"[adaptive] largest K* {kstar}; promoted {int((fln & 1).sum())}, value-only "
          f"{int(((fln & 3) == 2).sum())}, bound {int(bflags.sum().item())} of {fln.size}; "
          f"{int(fl0.sum())} heads fail the ranking check", flush=True)
    assert kstar <= 6
    oc = oracle_view_of_gpu(c, g)
    ref, pmass = attention.decode_attention(oc, q, c["dtype"], np.array(seq), c["rotation"], s, flags=fln)
    assert attention.row_rel_err(out0, ref).max() <= TOL
    kvq.dense_fallback(p, g, qd, seq, eps, out, cert, fail=fail)
    torch.cuda.synchronize()
    out1, cert1 = out.cpu().numpy(), cert.cpu().numpy()
    dense = attention.dense_attention(oc.k_orig, oc.v_orig, q, c["dtype"], np.array(seq))
    want_out, want_cert, redo = adaptive.dense_fallback(out0, cert0, eps, dense, fl0)
    assert np.array_equal(cert1, want_cert.astype(np.float32))
    assert np.array_equal(out1[~redo], out0[~redo])
    if redo.any():
        assert attention.row_rel_err(out1[redo], dense[redo]).max() <= TOL
    exact = np.where(redo[..., None], dense, ref)
    assert np.all(np.linalg.norm(exact - dense, axis=-1) <= want_cert + 1e-12)


def test_fallback_on_failed_heads_only():
    # certificate NULL: only the check's fail flags trigger the recompute
    seq = [4096, 2500]
    c, s, p, g, q, qd, mass = _needle_state(seq)
    out = kvq.decode_attn(p, g, qd, seq)
    torch.cuda.synchronize()
    out0 = out.cpu().numpy().copy()
    fail = torch.zeros((c["B"], c["Hq"]), dtype=torch.uint8, device="cuda")
    fail[0, 3] = 1
    fail[1, 17] = 1
    kvq.dense_fallback(p, g, qd, seq, 0.0, out, None, fail=fail)
    torch.cuda.synchronize()
    out1 = out.cpu().numpy()
    oc = oracle_view_of_gpu(c, g)
    dense = attention.dense_attention(oc.k_orig, oc.v_orig, q, c["dtype"], np.array(seq))
    redo = fail.cpu().numpy() != 0
    assert np.array_equal(out1[~redo], out0[~redo])
    assert attention.row_rel_err(out1[redo], dense[redo]).max() <= TOL


def test_fallback_many_units():
    """More (sequence, kv head, head group) units than the fallback's shared-memory list
    holds (216 x 64 = 13824 > 13312): every workgroup walks all the unit and split pairs and
    skips the units without a row to recompute; the failed rows equal dense fp64 attention over
    the originals and every other row is left as it was."""
    B, H, T = 216, 64, 64
    p = kvq.make_params(B, H, H, T, k_fmt="int8", v_fmt="int4", k_group=128, v_group=128, keep_fp16_copy=True)
    g = kvq.Cache(p, signs=torch.from_numpy(synth.signs(synth.config(3)).copy()).cuda())
    gen = torch.Generator(device="cuda")
    gen.manual_seed(99)
    k = torch.randn((B, H, T, 128), generator=gen, device="cuda").half().view(torch.int16)
    v = torch.randn((B, H, T, 128), generator=gen, device="cuda").half().view(torch.int16)
    q = torch.randn((B, H, 128), generator=gen, device="cuda").half().view(torch.int16)
    seq = [T] * (B - 1) + [37]
    kvq.append(p, g, k, v, [0] * B)
    out = kvq.decode_attn(p, g, q, seq)
    torch.cuda.synchronize()
    out0 = out.cpu().numpy().copy()
    fail = torch.zeros((B, H), dtype=torch.uint8, device="cuda")
    rows = [(0, 3), (100, 17), (215, 63)]
    for b, h in rows:
        fail[b, h] = 1
    kvq.dense_fallback(p, g, q, seq, 0.0, out, None, fail=fail)
    torch.cuda.synchronize()
    out1 = out.cpu().numpy()
    redo = fail.cpu().numpy() != 0
    assert np.array_equal(out1[~redo], out0[~redo])
    kb = g.bufs["k_orig"].cpu().numpy().view(np.uint16).reshape(B, H, T, 128)
    vb = g.bufs["v_orig"].cpu().numpy().view(np.uint16).reshape(B, H, T, 128)
    qb = q.cpu().numpy().view(np.uint16)
    for b, h in rows:
        ref = attention.dense_attention(kb[b:b + 1, h:h + 1], vb[b:b + 1, h:h + 1], qb[b:b + 1, h:h + 1], "f16",
                                        np.array([seq[b]]))
        err = attention.row_rel_err(out1[b:b + 1, h:h + 1], ref).max()
        print(f"[adaptive] many-units fallback row ({b}, {h}): rel err {err:.2e}", flush=True)
        assert err <= TOL
