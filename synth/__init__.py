"""Seeded synthetic inputs for the five workloads (shared by tests, bench and smoke).

This module only draws random numbers and rounds them to the input dtypes.  It
holds none of the compression or attention arithmetic: rotations, scales,
codes, attention and bounds live in the HIP library (product) and in the CPU
oracle (tests), which never share code.  The one rotation-related draw here is
the dense orthogonal matrix itself (a Haar sample, made from the QR
factorisation of a seeded Gaussian matrix with the signs of R's diagonal moved
into Q), which the method takes as a fixed input, like the sign vector.

Seeding.  Every stream is keyed by numpy SeedSequence(1234, spawn_key=(cfg,
stream, ...)), with streams K=0, V=1, q=2, signs=3, outliers=4, R=5, U=6,
calib=7, plant=8, needle=9.  K/V streams are further keyed by (b, kv head, chunk of 4096
tokens), so any slice of any sequence can be regenerated on its own.

Workloads (d = 128 throughout; stand-ins for model KV activations, since the
pages' models and datasets are not used):
  1 tiny int4        B=1  Hq=1  Hkv=1 T=1024   fp16 N(0,1), 2 seeded channels x10
  2 llama3-8b gqa    B=16 Hq=32 Hkv=8 T=8192   fp16 N(0,1), 10 (head, channel) x8;
                                               4096-token prefill append
  3 certified        B=32 Hq=32 Hkv=8 T=32768  K 0.02 N(0,1), V 0.0015 N(0,1) fp16,
                                               10 planted blocks per (b, head);
                                               with needles=n: n retrieval needles
                                               per (b, head) and queries that seek
                                               them (peaked attention)
  4 int2 dense       B=64 Hq=32 Hkv=8 T=32768  fp16 U diag(i^-1/2) z, U Haar per head
  5 fp4 search       B=8  Hq=32 Hkv=8 T=131072 bf16 Student-t (nu = 4)
"""

import numpy as np

D = 128
CHUNK = 4096
ROOT_SEED = 1234
ST_K, ST_V, ST_Q, ST_SIGNS, ST_OUTL, ST_R, ST_U, ST_CALIB, ST_PLANT, ST_NEEDLE = range(10)

CONFIGS = {
    1: dict(cfg=1, name="tiny-int4", B=1, Hq=1, Hkv=1, T=1024, dtype="f16",
            k_fmt="int4", v_fmt="int4", k_group=32, v_group=32, scale_mode="absmax",
            rotation="sign_fwht", keep=False, data="gauss", outlier_mode="channels",
            n_outliers=2, outlier_factor=10.0, prefill=1024),
    2: dict(cfg=2, name="llama3-8b-gqa-int4", B=16, Hq=32, Hkv=8, T=8192, dtype="f16",
            k_fmt="int4", v_fmt="int4", k_group=32, v_group=32, scale_mode="absmax",
            rotation="sign_fwht", keep=False, data="gauss", outlier_mode="head_channels",
            n_outliers=10, outlier_factor=8.0, prefill=4096),
    3: dict(cfg=3, name="certified-int8k-int4v", B=32, Hq=32, Hkv=8, T=32768, dtype="f16",
            k_fmt="int8", v_fmt="int4", k_group=128, v_group=128, scale_mode="absmax",
            rotation="sign_fwht", keep=True, data="certified", k_sigma=0.02, v_sigma=0.0015,
            n_plant=10, plant_factor=10.0, tau=1e-2, prefill=4096,
            needles=0, needle_q=16.0, needle_top=20.0, needle_tie_every=8),
    4: dict(cfg=4, name="int2-dense-rotation", B=64, Hq=32, Hkv=8, T=32768, dtype="f16",
            k_fmt="int2", v_fmt="int2", k_group=32, v_group=32, scale_mode="absmax",
            rotation="dense", keep=False, data="anisotropic", clip_ratio=0.9,
            calib_tokens=4096, prefill=4096),
    5: dict(cfg=5, name="fp4-e4m3-scale-search", B=8, Hq=32, Hkv=8, T=131072, dtype="bf16",
            k_fmt="fp4", v_fmt="fp4", k_group=16, v_group=16, scale_mode="search9",
            rotation="sign_fwht", keep=False, data="student_t", nu=4.0, prefill=4096),
}


def config(cfg_id, **over):
    """A copy of workload cfg_id with fields overridden (e.g. smaller B or T)."""
    c = dict(CONFIGS[cfg_id])
    c.update(over)
    return c


def _rng(*key):
    return np.random.default_rng(np.random.SeedSequence(ROOT_SEED, spawn_key=tuple(int(k) for k in key)))


def to_f16_bits(x):
    """fp32/fp64 values -> fp16 bit patterns (IEEE round-to-nearest-even)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_bf16_bits(x):
    """fp32 values -> bf16 bit patterns (round-to-nearest-even on the top 16 bits)."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = b + 0x7FFF + ((b >> 16) & 1)
    return (b >> 16).astype(np.uint16)


def to_bits(x, dtype):
    return to_f16_bits(x) if dtype == "f16" else to_bf16_bits(x)


def signs(c):
    """The fixed random sign vector (+1/-1, int8 [128])."""
    r = _rng(c["cfg"], ST_SIGNS)
    return np.where(r.integers(0, 2, size=D) == 1, 1, -1).astype(np.int8)


def dense_rotation_f16(c):
    """A Haar-random orthogonal 128x128 matrix, rounded to fp16 (bit patterns)."""
    g = _rng(c["cfg"], ST_R).standard_normal((D, D))
    qm, rm = np.linalg.qr(g)
    qm = qm * np.sign(np.diag(rm))[None, :]
    return to_f16_bits(qm)


def _outlier_channels(c, tensor):
    """Channels scaled up, per kv head: list of arrays (one per head)."""
    r = _rng(c["cfg"], ST_OUTL, tensor)
    if c.get("outlier_mode") == "channels":
        ch = r.choice(D, size=c["n_outliers"], replace=False)
        return [ch for _ in range(c["Hkv"])]
    if c.get("outlier_mode") == "head_channels":
        pairs = r.choice(c["Hkv"] * D, size=c["n_outliers"], replace=False)
        return [np.sort(pairs[pairs // D == h] % D) for h in range(c["Hkv"])]
    return [np.zeros(0, np.int64) for _ in range(c["Hkv"])]


def _haar(r):
    g = r.standard_normal((D, D))
    qm, rm = np.linalg.qr(g)
    return qm * np.sign(np.diag(rm))[None, :]


def anisotropic_basis(c, tensor, h):
    """The orthogonal basis U (fp64 [128, 128]) of the anisotropic law of (tensor, kv head):
    vectors are U diag(i^-1/2) z with z ~ N(0, 1)."""
    return _haar(_rng(c["cfg"], ST_U, tensor, h))


def planted(c, b, h):
    """For the certified workload: [(block, token offset)] of planted outlier tokens."""
    nblk = c["T"] // 64
    r = _rng(c["cfg"], ST_PLANT, b, h)
    blocks = np.sort(r.choice(nblk, size=min(c["n_plant"], nblk), replace=False))
    offs = r.integers(0, 64, size=len(blocks))
    return list(zip(blocks.tolist(), offs.tolist()))


def needle_plan(c, b, h):
    """Retrieval needles of (sequence b, kv head h) in the certified workload with
    needles=n: (u, positions, logits).  u is a seeded unit direction; needle i sits at
    a seeded position in its own 64-token block and its key is logits[i] sqrt(128) /
    needle_q * u, so that a query needle_q u + (I - u u^T) z of the head's group gives it
    the logit logits[i] (softmax scale 1/sqrt(128)).  logits[i] = top - i with top
    drawn in needle_top +- 0.5; in one stream of every needle_tie_every the second needle
    sits 0.005 below the first (a near tie that quantization noise may invert)."""
    r = _rng(c["cfg"], ST_NEEDLE, b, h)
    u = r.standard_normal(D)
    u /= np.linalg.norm(u)
    n = int(c["needles"])
    blocks = r.choice(c["T"] // 64, size=n, replace=False)
    pos = blocks * 64 + r.integers(0, 64, size=n)
    logits = c["needle_top"] + r.uniform(-0.5, 0.5) - np.arange(n, dtype=np.float64)
    if n > 1 and (b * c["Hkv"] + h) % c["needle_tie_every"] == 0:
        logits[1] = logits[0] - 0.005
    return u, pos, logits


def _chunk_values(c, tensor, b, h, chunk):
    """fp32/fp64 values [CHUNK, 128] of one 4096-token chunk of a K or V stream."""
    st = ST_K if tensor == 0 else ST_V
    r = _rng(c["cfg"], st, b, h, chunk)
    kind = c["data"]
    if kind == "gauss":
        x = r.standard_normal((CHUNK, D), dtype=np.float32)
        ch = _outlier_channels(c, tensor)[h]
        x[:, ch] *= np.float32(c["outlier_factor"])
        return x
    if kind == "certified":
        sig = c["k_sigma"] if tensor == 0 else c["v_sigma"]
        return r.standard_normal((CHUNK, D), dtype=np.float32) * np.float32(sig)
    if kind == "anisotropic":
        u = anisotropic_basis(c, tensor, h)
        z = r.standard_normal((CHUNK, D))
        lam = 1.0 / np.sqrt(np.arange(1, D + 1, dtype=np.float64))
        return (z * lam[None, :]) @ u.T
    if kind == "student_t":
        return r.standard_t(c["nu"], size=(CHUNK, D)).astype(np.float32)
    raise ValueError(kind)


def kv_slice(c, tensor, b, h, t0, n):
    """Input bit patterns (uint16 [n, 128], fp16 or bf16) of tokens [t0, t0+n).

    tensor: 0 = K, 1 = V.  Independent of how the sequence is sliced.
    """
    out = np.empty((n, D), dtype=np.float64)
    t = t0
    while t < t0 + n:
        ck = t // CHUNK
        lo = t - ck * CHUNK
        hi = min(CHUNK, t0 + n - ck * CHUNK)
        out[t - t0:t - t0 + hi - lo] = _chunk_values(c, tensor, b, h, ck)[lo:hi]
        t += hi - lo
    if c["data"] == "certified":
        for blk, off in planted(c, b, h):
            pos = blk * 64 + off
            if t0 <= pos < t0 + n:
                out[pos - t0] *= c["plant_factor"]
        if tensor == 0 and c.get("needles"):
            u, npos, nlog = needle_plan(c, b, h)
            for p_, l_ in zip(npos, nlog):
                if t0 <= p_ < t0 + n:
                    out[p_ - t0] = l_ * np.sqrt(D) / c["needle_q"] * u
    return to_bits(out, c["dtype"])


def one_blas_thread():
    """Pool-worker initialiser: one BLAS thread per worker process (many workers each
    running a full-width BLAS thread pool oversubscribe the host many times over)."""
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def kv_all(c, tensor, t0, n, workers=1, start_method="fork"):
    """[B, Hkv, n, 128] uint16 for tokens [t0, t0+n) of every stream.

    workers > 1 draws the streams in a process pool; use start_method="spawn" in a
    process that has already initialised the GPU (the workers only run NumPy).
    """
    B, H = c["B"], c["Hkv"]
    out = np.empty((B, H, n, D), dtype=np.uint16)
    jobs = [(b, h) for b in range(B) for h in range(H)]
    if workers > 1 and len(jobs) > 1:
        import multiprocessing as mp
        ctx = mp.get_context(start_method)
        with ctx.Pool(min(workers, len(jobs)), initializer=one_blas_thread) as pool:
            res = pool.starmap(kv_slice, [(c, tensor, b, h, t0, n) for b, h in jobs])
        for (b, h), r in zip(jobs, res):
            out[b, h] = r
    else:
        for b, h in jobs:
            out[b, h] = kv_slice(c, tensor, b, h, t0, n)
    return out


def queries(c, step=0):
    """Query bit patterns [B, Hq, 128]: N(0,1) in the input dtype; with needles, the
    query of a head of kv head h is needle_q u + (I - u u^T) z, z the N(0,1) draw and u
    the needle direction of (b, h)."""
    r = _rng(c["cfg"], ST_Q, step)
    z = r.standard_normal((c["B"], c["Hq"], D), dtype=np.float32)
    if not c.get("needles"):
        return to_bits(z, c["dtype"])
    q = z.astype(np.float64)
    G = c["Hq"] // c["Hkv"]
    for b in range(c["B"]):
        for h in range(c["Hkv"]):
            u = needle_plan(c, b, h)[0]
            for hq in range(h * G, (h + 1) * G):
                q[b, hq] = c["needle_q"] * u + q[b, hq] - (q[b, hq] @ u) * u
    return to_bits(q, c["dtype"])


def calibration(c, tensor, h):
    """Calibration tokens [calib_tokens, 128] (bits) for clip thresholds, same law as the data."""
    n = c.get("calib_tokens", 4096)
    st_r = _rng(c["cfg"], ST_CALIB, tensor, h)
    if c["data"] == "anisotropic":
        u = anisotropic_basis(c, tensor, h)
        z = st_r.standard_normal((n, D))
        lam = 1.0 / np.sqrt(np.arange(1, D + 1, dtype=np.float64))
        return to_bits((z * lam[None, :]) @ u.T, c["dtype"])
    return to_bits(st_r.standard_normal((n, D)), c["dtype"])
