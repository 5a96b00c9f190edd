"""Oracle side of the full-size GPU parity tests, run in worker processes.

Each worker regenerates one (sequence, kv head) stream from the seeded input
generator, appends it to a one-stream oracle cache and returns SHA-256 digests of
the packed arrays; the test compares them with digests of the library's bytes of
the same stream.  Nothing here sees a library output.
"""
import hashlib

import numpy as np

import synth
from oracle import codec

ARRAYS = ("k_codes", "k_meta", "v_codes", "v_meta")


def digests_of(arrays):
    return tuple(hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest() for a in arrays)


def stream_digests(c, b, h, r16=None, clip=None):
    """Digests of the oracle's packed bytes of stream (b, h) holding tokens [0, T)."""
    T = c["T"]
    k = synth.kv_slice(c, 0, b, h, 0, T)
    v = synth.kv_slice(c, 1, b, h, 0, T)
    one = dict(c, B=1, Hkv=1, Hq=1)
    oc = codec.Cache(1, 1, T, one["k_fmt"], one["v_fmt"], one["k_group"], one["v_group"], keep_fp16_copy=one["keep"])
    ck = cv = None
    if clip is not None:
        ck, cv = clip[0][h:h + 1], clip[1][h:h + 1]
    codec.append(oc, k[None, None], v[None, None], np.array([0]), c["dtype"], c["rotation"], synth.signs(c), r16,
                 clip_k=ck, clip_v=cv, scale_mode=c["scale_mode"])
    return (b, h), digests_of([getattr(oc, n)[0, 0] for n in ARRAYS])
