"""Python binding of libkvq (ctypes): argument marshalling only.

Every computation runs in the HIP kernels of libkvq.so; this module turns torch
tensors into device pointers and the current HIP stream, calls the C entry
points of the same names (kvq_append, kvq_error_bound, kvq_decode_attn,
kvq_decode_attn_dense, kvq_decode_attn_noalloc, kvq_calibrate_clip, kvq_block_mass, kvq_select_blocks,
kvq_promote_values, kvq_ranking_check, kvq_dense_fallback, kvq_calibrate_lambda, kvq_buffer_bytes, kvq_decode_workspace_bytes, kvq_decode_splits,
kvq_debug_status) and raises KvqError on a non-zero status.  There is no fallback: if
the library is not built, importing the functions raises.  KVQ_LIB in the environment
names another build of the library to load (the layout-checking libkvq_debug.so).
"""

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("KVQ_LIB") or os.path.join(_HERE, "libkvq.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libkvq_debug.so")

F16, BF16 = 0, 1
INT4, INT8, INT2, FP4 = 0, 1, 2, 3
ROT_NONE, ROT_SIGN_FWHT, ROT_DENSE, ROT_SRFT = 0, 1, 2, 3
SCALE_ABSMAX, SCALE_SEARCH9, SCALE_SEARCH_OFFSETS = 0, 1, 2
BUF_NAMES = ("k_codes", "k_meta", "v_codes", "v_meta", "blk_desc", "k_orig", "v_orig", "k_win", "v_win")

_FMT = {"int4": INT4, "int8": INT8, "int2": INT2, "fp4": FP4}
_ROT = {"none": ROT_NONE, "sign_fwht": ROT_SIGN_FWHT, "dense": ROT_DENSE, "srft": ROT_SRFT}
_DT = {"f16": F16, "bf16": BF16}
_SM = {"absmax": SCALE_ABSMAX, "search9": SCALE_SEARCH9, "offsets": SCALE_SEARCH_OFFSETS}


class KvqError(RuntimeError):
    def __init__(self, status, name, detail):
        super().__init__(f"{name} ({status}): {detail}")
        self.status = status


class Params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("max_ctx", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
        ("k_fmt", ctypes.c_int32), ("v_fmt", ctypes.c_int32), ("k_group", ctypes.c_int32),
        ("v_group", ctypes.c_int32), ("scale_mode", ctypes.c_int32), ("rotation", ctypes.c_int32),
        ("keep_fp16_copy", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("sink_blocks", ctypes.c_int32), ("recent_blocks", ctypes.c_int32),
    ]


class CacheStruct(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("k_codes", "k_meta", "v_codes", "v_meta", "blk_desc",
                                               "k_orig", "v_orig", "signs", "rot_f16", "clip_k", "clip_v",
                                               "k_win", "v_win", "lambda_k", "lambda_v")]


_lib = None


def lib():
    """The loaded libkvq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run python -m bit_kv_cache_append_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, P = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER
        L.kvq_abi_version.restype = i32
        L.kvq_status_str.restype = ctypes.c_char_p
        L.kvq_status_str.argtypes = [i32]
        L.kvq_last_error.restype = ctypes.c_char_p
        if hasattr(L, "kvq_debug_status"):  # (libraries of ABI version 5 and later)
            L.kvq_debug_status.restype = i32
            L.kvq_debug_status.argtypes = [P(ctypes.c_uint32), i32]
        L.kvq_buffer_bytes.restype = i32
        L.kvq_buffer_bytes.argtypes = [P(Params), P(ctypes.c_size_t)]
        L.kvq_decode_workspace_bytes.restype = ctypes.c_size_t
        L.kvq_decode_workspace_bytes.argtypes = [P(Params)]
        L.kvq_decode_splits.restype = i32
        L.kvq_decode_splits.argtypes = [P(Params), P(i32)]
        L.kvq_append.restype = i32
        L.kvq_append.argtypes = [P(Params), P(CacheStruct), vp, vp, P(i32), i32, vp]
        L.kvq_error_bound.restype = i32
        L.kvq_error_bound.argtypes = [P(Params), P(CacheStruct), vp, P(i32), ctypes.c_float, vp, vp, vp]
        L.kvq_decode_attn.restype = i32
        L.kvq_decode_attn.argtypes = [P(Params), P(CacheStruct), vp, P(i32), vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.kvq_decode_attn_noalloc.restype = i32
        L.kvq_decode_attn_noalloc.argtypes = [P(Params), P(CacheStruct), vp, P(i32), vp, vp, vp, vp]
        L.kvq_decode_attn_dense.restype = i32
        L.kvq_decode_attn_dense.argtypes = [P(Params), vp, vp, vp, P(i32), vp, vp, ctypes.c_size_t, vp]
        L.kvq_block_mass.restype = i32
        L.kvq_block_mass.argtypes = [P(Params), P(CacheStruct), vp, P(i32), vp, vp]
        L.kvq_select_blocks.restype = i32
        L.kvq_select_blocks.argtypes = [P(Params), vp, P(i32), ctypes.c_float, vp, vp, vp]
        L.kvq_promote_values.restype = i32
        L.kvq_promote_values.argtypes = [P(Params), P(CacheStruct), vp, P(i32), ctypes.c_float, vp, vp]
        L.kvq_ranking_check.restype = i32
        L.kvq_ranking_check.argtypes = [P(Params), P(CacheStruct), vp, P(i32), vp, ctypes.c_float, ctypes.c_float,
                                        i32, vp, vp, vp]
        L.kvq_dense_fallback.restype = i32
        L.kvq_dense_fallback.argtypes = [P(Params), P(CacheStruct), vp, P(i32), ctypes.c_float, vp, vp, vp, vp,
                                         ctypes.c_size_t, vp]
        L.kvq_calibrate_lambda.restype = i32
        L.kvq_calibrate_lambda.argtypes = [P(Params), P(CacheStruct), vp, vp, i32, vp, vp, vp]
        L.kvq_calibrate_clip.restype = i32
        L.kvq_calibrate_clip.argtypes = [P(Params), P(CacheStruct), vp, vp, i32, ctypes.c_float, vp, vp, vp]
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        L = lib()
        raise KvqError(status, L.kvq_status_str(status).decode(), L.kvq_last_error().decode())


def make_params(B, Hq, Hkv, max_ctx, k_fmt="int4", v_fmt="int4", k_group=32, v_group=32, dtype="f16",
                scale_mode="absmax", rotation="sign_fwht", keep_fp16_copy=False, softmax_scale=0.0,
                sink_blocks=0, recent_blocks=0):
    """Build the C params struct (format names as strings or the integer constants)."""
    def enum(v, table):
        return table[v] if isinstance(v, str) else int(v)
    return Params(B, Hq, Hkv, 128, max_ctx, enum(dtype, _DT), enum(k_fmt, _FMT), enum(v_fmt, _FMT), k_group,
                  v_group, enum(scale_mode, _SM), enum(rotation, _ROT), int(bool(keep_fp16_copy)),
                  float(softmax_scale), int(sink_blocks), int(recent_blocks))


def params_from_config(c, **over):
    """Params for a workload dict of the synth module (shape and format fields only)."""
    d = dict(B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], max_ctx=c["T"], k_fmt=c["k_fmt"], v_fmt=c["v_fmt"],
             k_group=c["k_group"], v_group=c["v_group"], dtype=c["dtype"], scale_mode=c["scale_mode"],
             rotation=c["rotation"], keep_fp16_copy=c["keep"], sink_blocks=c.get("sink_blocks", 0),
             recent_blocks=c.get("recent_blocks", 0))
    d.update(over)
    return make_params(**d)


def buffer_bytes(p):
    out = (ctypes.c_size_t * len(BUF_NAMES))()
    _check(lib().kvq_buffer_bytes(ctypes.byref(p), out))
    return {n: int(out[i]) for i, n in enumerate(BUF_NAMES)}


def decode_workspace_bytes(p):
    return int(lib().kvq_decode_workspace_bytes(ctypes.byref(p)))


def debug_status(clear=True):
    """kvq_debug_status (debug library only): (code of the first failed layout check or 0,
    its two indices, failures counted); raises KvqError(KVQ_ERR_UNSUPPORTED) on the release
    library."""
    out = (ctypes.c_uint32 * 4)()
    _check(lib().kvq_debug_status(out, int(bool(clear))))
    return tuple(int(x) for x in out)


def decode_splits(p, seq_len):
    """kvq_decode_splits: context splits of a decode call with these sequence lengths."""
    return int(lib().kvq_decode_splits(ctypes.byref(p), _i32(seq_len)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _i32(a):
    arr = (ctypes.c_int32 * len(a))(*[int(x) for x in a])
    return arr


class Cache:
    """The device buffers of one cache, allocated with torch (zero-filled)."""

    def __init__(self, p, device="cuda", signs=None, rot_f16=None, clip_k=None, clip_v=None, lambda_k=None,
                 lambda_v=None):
        import torch
        self.p = p
        sizes = buffer_bytes(p)
        self.bufs = {}
        for name, nbytes in sizes.items():
            if name == "blk_desc":
                self.bufs[name] = torch.zeros(max(nbytes // 4, 1), dtype=torch.float32, device=device) if nbytes else None
            elif nbytes:
                self.bufs[name] = torch.zeros(nbytes, dtype=torch.uint8, device=device)
            else:
                self.bufs[name] = None
        self.signs = signs
        self.rot_f16 = rot_f16
        self.clip_k = clip_k
        self.clip_v = clip_v
        self.lambda_k = lambda_k
        self.lambda_v = lambda_v

    def struct(self):
        b = self.bufs
        ptr = lambda t: None if t is None else t.data_ptr()
        return CacheStruct(*[ptr(b[n]) for n in BUF_NAMES[:7]], ptr(self.signs), ptr(self.rot_f16),
                           ptr(self.clip_k), ptr(self.clip_v), ptr(b["k_win"]), ptr(b["v_win"]),
                           ptr(self.lambda_k), ptr(self.lambda_v))


def append(p, cache, k_new, v_new, start_pos, stream=None):
    """kvq_append: k_new/v_new device [B, Hkv, n_new, 128] (fp16/bf16 or their bits)."""
    n_new = int(k_new.shape[2])
    cs = cache.struct()
    _check(lib().kvq_append(ctypes.byref(p), ctypes.byref(cs), _ptr(k_new), _ptr(v_new), _i32(start_pos), n_new,
                            stream if stream is not None else _stream()))


def error_bound(p, cache, q, seq_len, tau, bound=None, flags=None, stream=None):
    """kvq_error_bound: returns (bound fp32 [B, Hkv, nt], flags uint8 [B, Hkv, nt])."""
    import torch
    nt = p.max_ctx // 64
    if bound is None:
        bound = torch.empty((p.batch, p.n_kv_heads, nt), dtype=torch.float32, device=q.device)
    if flags is None:
        flags = torch.empty((p.batch, p.n_kv_heads, nt), dtype=torch.uint8, device=q.device)
    cs = cache.struct()
    _check(lib().kvq_error_bound(ctypes.byref(p), ctypes.byref(cs), _ptr(q), _i32(seq_len), float(tau),
                                 _ptr(bound), _ptr(flags), stream if stream is not None else _stream()))
    return bound, flags


def workspace(p, device="cuda"):
    """A decode workspace: split arrival counters (zero between calls) and split records."""
    import torch
    n = decode_workspace_bytes(p)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def decode_attn(p, cache, q, seq_len, flags=None, certificate=False, ws=None, out=None, cert=None, stream=None):
    """kvq_decode_attn: returns out fp32 [B, Hq, 128] (and the certificate [B, Hq] if asked)."""
    import torch
    if out is None:
        out = torch.empty((p.batch, p.n_q_heads, 128), dtype=torch.float32, device=q.device)
    if certificate and cert is None:
        cert = torch.empty((p.batch, p.n_q_heads), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(p, q.device)
    cs = cache.struct()
    _check(lib().kvq_decode_attn(ctypes.byref(p), ctypes.byref(cs), _ptr(q), _i32(seq_len), _ptr(flags), _ptr(out),
                                 _ptr(cert) if certificate else None, _ptr(ws), ws.numel() * ws.element_size(),
                                 stream if stream is not None else _stream()))
    return (out, cert) if certificate else out


def decode_attn_noalloc(p, cache, q, seq_len, flags=None, certificate=False, out=None, cert=None, stream=None):
    """kvq_decode_attn_noalloc: kvq_decode_attn on the library's fixed per-device workspace."""
    import torch
    if out is None:
        out = torch.empty((p.batch, p.n_q_heads, 128), dtype=torch.float32, device=q.device)
    if certificate and cert is None:
        cert = torch.empty((p.batch, p.n_q_heads), dtype=torch.float32, device=q.device)
    cs = cache.struct()
    _check(lib().kvq_decode_attn_noalloc(ctypes.byref(p), ctypes.byref(cs), _ptr(q), _i32(seq_len), _ptr(flags),
                                         _ptr(out), _ptr(cert) if certificate else None,
                                         stream if stream is not None else _stream()))
    return (out, cert) if certificate else out


def decode_attn_dense(p, k, v, q, seq_len, ws=None, out=None, stream=None):
    """kvq_decode_attn_dense over uncompressed [B, Hkv, Tmax, 128] K/V."""
    import torch
    if out is None:
        out = torch.empty((p.batch, p.n_q_heads, 128), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(p, q.device)
    _check(lib().kvq_decode_attn_dense(ctypes.byref(p), _ptr(k), _ptr(v), _ptr(q), _i32(seq_len), _ptr(out), _ptr(ws),
                                       ws.numel() * ws.element_size(), stream if stream is not None else _stream()))
    return out


def block_mass(p, cache, q, seq_len, mass=None, stream=None):
    """kvq_block_mass: estimated attention mass per block, fp32 [B, Hq, max_ctx // 64]."""
    import torch
    if mass is None:
        mass = torch.empty((p.batch, p.n_q_heads, p.max_ctx // 64), dtype=torch.float32, device=q.device)
    cs = cache.struct()
    _check(lib().kvq_block_mass(ctypes.byref(p), ctypes.byref(cs), _ptr(q), _i32(seq_len), _ptr(mass),
                                stream if stream is not None else _stream()))
    return mass


def select_blocks(p, mass, seq_len, tau_cov, flags_in=None, flags_out=None, stream=None):
    """kvq_select_blocks: promotion flags uint8 [B, Hkv, max_ctx // 64] (flags_out may be flags_in)."""
    import torch
    if flags_out is None:
        flags_out = torch.empty((p.batch, p.n_kv_heads, p.max_ctx // 64), dtype=torch.uint8, device=mass.device)
    _check(lib().kvq_select_blocks(ctypes.byref(p), _ptr(mass), _i32(seq_len), float(tau_cov), _ptr(flags_in),
                                   _ptr(flags_out), stream if stream is not None else _stream()))
    return flags_out


def promote_values(p, cache, mass, seq_len, tau_v, flags, stream=None):
    """kvq_promote_values: bit 1 on the blocks whose mass * ev exceeds tau_v (flags in place)."""
    cs = cache.struct()
    _check(lib().kvq_promote_values(ctypes.byref(p), ctypes.byref(cs), _ptr(mass), _i32(seq_len), float(tau_v),
                                    _ptr(flags), stream if stream is not None else _stream()))
    return flags


def ranking_check(p, cache, q, seq_len, mass, tau_cov, margin=0.0, max_inversions=0, out=None, stream=None):
    """kvq_ranking_check: (inversions int32 [B, Hq], fail uint8 [B, Hq]) (out: that pair to fill)."""
    import torch
    if out is None:
        inv = torch.empty((p.batch, p.n_q_heads), dtype=torch.int32, device=mass.device)
        fl = torch.empty((p.batch, p.n_q_heads), dtype=torch.uint8, device=mass.device)
    else:
        inv, fl = out
    cs = cache.struct()
    _check(lib().kvq_ranking_check(ctypes.byref(p), ctypes.byref(cs), _ptr(q), _i32(seq_len), _ptr(mass),
                                   float(tau_cov), float(margin), int(max_inversions), _ptr(inv), _ptr(fl),
                                   stream if stream is not None else _stream()))
    return inv, fl


def dense_fallback(p, cache, q, seq_len, eps, out, cert, fail=None, ws=None, stream=None):
    """kvq_dense_fallback: rows with cert > eps, or fail set, recomputed densely from the
    originals (in place; cert may be None when fail is given)."""
    if ws is None:
        ws = workspace(p, q.device)
    cs = cache.struct()
    _check(lib().kvq_dense_fallback(ctypes.byref(p), ctypes.byref(cs), _ptr(q), _i32(seq_len), float(eps),
                                    _ptr(fail), _ptr(out), _ptr(cert), _ptr(ws), ws.numel() * ws.element_size(),
                                    stream if stream is not None else _stream()))
    return out, cert


def calibrate_clip(p, cache, calib_k, calib_v, ratio=0.9, stream=None):
    """kvq_calibrate_clip: calib_k/v device [Hkv, n, 128]; returns (clip_k, clip_v) fp32 [Hkv, 128]."""
    import torch
    ck = torch.empty((p.n_kv_heads, 128), dtype=torch.float32, device=calib_k.device)
    cv = torch.empty((p.n_kv_heads, 128), dtype=torch.float32, device=calib_k.device)
    cs = cache.struct()
    _check(lib().kvq_calibrate_clip(ctypes.byref(p), ctypes.byref(cs), _ptr(calib_k), _ptr(calib_v),
                                    int(calib_k.shape[1]), float(ratio), _ptr(ck), _ptr(cv),
                                    stream if stream is not None else _stream()))
    return ck, cv


def calibrate_lambda(p, cache, calib_k, calib_v, stream=None):
    """kvq_calibrate_lambda: per-channel rescale factors fp32 [Hkv, 128] of K and V."""
    import torch
    lk = torch.empty((p.n_kv_heads, 128), dtype=torch.float32, device=calib_k.device)
    lv = torch.empty((p.n_kv_heads, 128), dtype=torch.float32, device=calib_k.device)
    cs = cache.struct()
    _check(lib().kvq_calibrate_lambda(ctypes.byref(p), ctypes.byref(cs), _ptr(calib_k), _ptr(calib_v),
                                      int(calib_k.shape[1]), _ptr(lk), _ptr(lv),
                                      stream if stream is not None else _stream()))
    return lk, lv


def to_device_bits(a, device="cuda"):
    """numpy uint16 bit patterns -> a torch int16 device tensor with the same bits."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)
