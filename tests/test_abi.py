"""CPU checks of the C-ABI library: it loads, exports every declared entry point,
reports sizes, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re

import pytest

import bit_kv_cache_append_amd as kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = kvq.lib()
    names = _declared()
    assert "kvq_append" in names and "kvq_decode_attn" in names and "kvq_error_bound" in names
    for n in names:
        assert hasattr(L, n), f"{n} not exported"
    assert L.kvq_abi_version() == 5


def test_debug_library_exports_the_same_symbols():
    """libkvq_debug.so (the layout-checking build) loads and exports every declared entry
    point; the release library has no checks and says so without touching a device."""
    assert os.path.exists(kvq.DEBUG_LIB_PATH), "build with python -m bit_kv_cache_append_amd.build --all"
    D = ctypes.CDLL(kvq.DEBUG_LIB_PATH)
    for n in _declared():
        assert hasattr(D, n), f"{n} not exported by the debug library"
    assert D.kvq_abi_version() == 5
    with pytest.raises(kvq.KvqError) as e:
        kvq.debug_status()
    assert e.value.status == -2  # KVQ_ERR_UNSUPPORTED


def test_buffer_sizes():
    p = kvq.make_params(16, 32, 8, 8192, "int4", "int4", 32, 32)
    sz = kvq.buffer_bytes(p)
    streams = 16 * 8
    assert sz["k_codes"] == streams * 8192 * 64
    assert sz["k_meta"] == streams * 8192 * 8
    assert sz["v_codes"] == streams * 8192 * 64
    assert sz["v_meta"] == streams * 8192 * 8
    assert sz["blk_desc"] == 0 and sz["k_orig"] == 0
    p3 = kvq.make_params(32, 32, 8, 32768, "int8", "int4", 128, 128, keep_fp16_copy=True)
    s3 = kvq.buffer_bytes(p3)
    assert s3["k_codes"] == 256 * 32768 * 128 and s3["k_meta"] == 256 * 32768 * 2
    assert s3["v_meta"] == 256 * 32768 * 2 and s3["blk_desc"] == 256 * 512 * 12
    p4 = kvq.make_params(64, 32, 8, 32768, "int2", "int2", rotation="dense")
    s4 = kvq.buffer_bytes(p4)
    assert s4["k_codes"] == 512 * 32768 * 32 and s4["k_meta"] == 512 * 32768 * 16
    p5 = kvq.make_params(8, 32, 8, 131072, "fp4", "fp4", dtype="bf16", scale_mode="search9")
    s5 = kvq.buffer_bytes(p5)
    assert s5["k_codes"] == 64 * 131072 * 64 and s5["v_meta"] == 64 * 131072 * 8
    assert s5["k_win"] == 0 and s5["v_win"] == 0
    assert kvq.decode_workspace_bytes(p) > 0
    # full-precision window: (sink + recent) blocks of 64 rows of 128 16-bit values per stream
    pw = kvq.make_params(64, 32, 8, 32768, "int2", "int2", rotation="dense", sink_blocks=1, recent_blocks=2)
    sw = kvq.buffer_bytes(pw)
    assert sw["k_win"] == sw["v_win"] == 512 * 3 * 64 * 256
    assert sw["k_codes"] == s4["k_codes"]


@pytest.mark.parametrize("sink,recent", [(-1, 0), (0, -2), (3, 2)])
def test_invalid_window_rejected(sink, recent):
    p = kvq.make_params(2, 8, 2, 256, sink_blocks=sink, recent_blocks=recent)  # 4 blocks of 64
    with pytest.raises(kvq.KvqError) as e:
        kvq.buffer_bytes(p)
    assert e.value.status == -1


def test_window_needs_buffers_without_gpu():
    L = kvq.lib()
    p = kvq.make_params(2, 8, 2, 256, sink_blocks=1, recent_blocks=1)
    fake = 1 << 20  # never dereferenced: validation fails first
    cs = kvq.CacheStruct(k_codes=fake, k_meta=fake, v_codes=fake, v_meta=fake, signs=fake)
    starts = (ctypes.c_int32 * 2)(0, 0)
    st = L.kvq_append(ctypes.byref(p), ctypes.byref(cs), fake, fake, starts, 4, None)
    assert st == -1 and b"k_win" in L.kvq_last_error()


@pytest.mark.parametrize("field,value", [("head_dim", 64), ("max_ctx", 100), ("batch", 0), ("n_q_heads", 7),
                                         ("k_group", 64), ("v_group", 8), ("v_fmt", 1), ("rotation", 9)])
def test_invalid_params_rejected(field, value):
    p = kvq.make_params(2, 8, 2, 256)
    setattr(p, field, value)
    with pytest.raises(kvq.KvqError) as e:
        kvq.buffer_bytes(p)
    assert e.value.status in (-1, -2)


def test_group_16_is_int4_only():
    # groups of 16 ("When Quantization Is Free", Methodology section 3): 8 fp16 scales per token
    p = kvq.make_params(2, 8, 2, 256, k_group=16, v_group=16)
    q = kvq.make_params(2, 8, 2, 256, k_group=32, v_group=32)
    sizes16, sizes32 = kvq.buffer_bytes(p), kvq.buffer_bytes(q)
    assert sizes16["k_meta"] == 2 * 2 * 256 * 16 and sizes32["k_meta"] == 2 * 2 * 256 * 8
    assert sizes16["v_meta"] == 2 * 2 * 4 * 8 * 64 * 2
    r = kvq.make_params(2, 8, 2, 256, k_fmt="int8", k_group=16)
    with pytest.raises(kvq.KvqError) as e:
        kvq.buffer_bytes(r)
    assert e.value.status == -1


def test_null_pointers_rejected_without_gpu():
    L = kvq.lib()
    p = kvq.make_params(2, 8, 2, 256)
    cs = kvq.CacheStruct()
    starts = (ctypes.c_int32 * 2)(0, 0)
    st = L.kvq_append(ctypes.byref(p), ctypes.byref(cs), None, None, starts, 4, None)
    assert st == -1 and b"NULL" in L.kvq_last_error()
    seq = (ctypes.c_int32 * 2)(10, 10)
    st = L.kvq_decode_attn(ctypes.byref(p), ctypes.byref(cs), None, seq, None, None, None, None, 0, None)
    assert st == -1
    assert L.kvq_status_str(-3) == b"KVQ_ERR_WORKSPACE"


def test_adaptive_entry_points_validate_without_gpu():
    L = kvq.lib()
    p = kvq.make_params(2, 8, 2, 256)
    seq = (ctypes.c_int32 * 2)(10, 10)
    fake = 1 << 20  # never dereferenced: validation fails first
    cs = kvq.CacheStruct(k_codes=fake, k_meta=fake, v_codes=fake, v_meta=fake, signs=fake)
    assert L.kvq_block_mass(ctypes.byref(p), ctypes.byref(cs), None, seq, None, None) == -1
    assert L.kvq_select_blocks(ctypes.byref(p), fake, seq, ctypes.c_float(1.5), None, fake, None) == -1
    assert b"tau_cov" in L.kvq_last_error()
    big = kvq.make_params(1, 8, 2, 64 * 8192)
    one = (ctypes.c_int32 * 1)(10)
    assert L.kvq_select_blocks(ctypes.byref(big), fake, one, ctypes.c_float(0.9), None, fake, None) == -2
    # the dense fallback, value promotion and ranking check read the originals or the
    # descriptors: they need keep_fp16_copy
    st = L.kvq_dense_fallback(ctypes.byref(p), ctypes.byref(cs), fake, seq, ctypes.c_float(0.1), None, fake, fake,
                              fake, 1 << 30, None)
    assert st == -1 and b"keep_fp16_copy" in L.kvq_last_error()
    st = L.kvq_promote_values(ctypes.byref(p), ctypes.byref(cs), fake, seq, ctypes.c_float(0.1), fake, None)
    assert st == -1 and b"keep_fp16_copy" in L.kvq_last_error()
    st = L.kvq_ranking_check(ctypes.byref(p), ctypes.byref(cs), fake, seq, fake, ctypes.c_float(0.9),
                             ctypes.c_float(0.0), 0, fake, fake, None)
    assert st == -1 and b"keep_fp16_copy" in L.kvq_last_error()
    kp = kvq.make_params(2, 8, 2, 256, k_fmt="int8", k_group=128, keep_fp16_copy=True)
    kc = kvq.CacheStruct(k_codes=fake, k_meta=fake, v_codes=fake, v_meta=fake, signs=fake, blk_desc=fake,
                         k_orig=fake, v_orig=fake)
    # the fallback needs at least one trigger: a certificate or the check's fail flags
    st = L.kvq_dense_fallback(ctypes.byref(kp), ctypes.byref(kc), fake, seq, ctypes.c_float(0.1), None, fake, None,
                              fake, 1 << 30, None)
    assert st == -1 and b"both NULL" in L.kvq_last_error()
    # and a workspace of kvq_decode_workspace_bytes
    st = L.kvq_dense_fallback(ctypes.byref(kp), ctypes.byref(kc), fake, seq, ctypes.c_float(0.1), fake, fake, fake,
                              fake, 256, None)
    assert st == -3 and b"workspace" in L.kvq_last_error()
    for tau_cov, margin, max_inv, what in ((1.5, 0.0, 0, b"tau_cov"), (0.9, -1.0, 0, b"margin"),
                                           (0.9, float("inf"), 0, b"margin"), (0.9, 0.0, -1, b"max_inversions")):
        st = L.kvq_ranking_check(ctypes.byref(kp), ctypes.byref(kc), fake, seq, fake, ctypes.c_float(tau_cov),
                                 ctypes.c_float(margin), max_inv, fake, fake, None)
        assert st == -1 and what in L.kvq_last_error()
    st = L.kvq_promote_values(ctypes.byref(kp), ctypes.byref(kc), fake, seq, ctypes.c_float(-1.0), fake, None)
    assert st == -1 and b"tau_v" in L.kvq_last_error()


def test_noalloc_decode_rejects_oversize_without_gpu():
    # kvq_decode_attn_noalloc keeps its counters and records in a fixed 8 MiB array per
    # device; calls that need more are refused on the host before anything is enqueued
    L = kvq.lib()
    fake = 1 << 20  # never dereferenced: validation fails first
    cs = kvq.CacheStruct(k_codes=fake, k_meta=fake, v_codes=fake, v_meta=fake, signs=fake)
    # 256 x 64 query rows, one split each: 256 * 64 * 1056 bytes of records > 8 MiB - 64 KiB
    p = kvq.make_params(256, 64, 64, 64)
    seq = (ctypes.c_int32 * 256)(*([64] * 256))
    st = L.kvq_decode_attn_noalloc(ctypes.byref(p), ctypes.byref(cs), fake, seq, None, fake, None, None)
    assert st == -3 and b"split records" in L.kvq_last_error()
    # 256 sequences x 128 kv heads: 128 KiB of arrival counters > 64 KiB
    p = kvq.make_params(256, 256, 128, 64)
    st = L.kvq_decode_attn_noalloc(ctypes.byref(p), ctypes.byref(cs), fake, seq, None, fake, None, None)
    assert st == -3 and b"split counters" in L.kvq_last_error()
    # other argument errors are reported as for kvq_decode_attn
    p = kvq.make_params(2, 8, 2, 256)
    two = (ctypes.c_int32 * 2)(10, 10)
    assert L.kvq_decode_attn_noalloc(ctypes.byref(p), ctypes.byref(cs), None, two, None, fake, None, None) == -1


def test_certified_cache_with_dense_rotation_rejected_without_gpu():
    # the block descriptors are rotated-basis residual norms: they bound original-basis errors
    # only for an orthogonal rotation, and the fp16-rounded dense matrix is not orthogonal
    L = kvq.lib()
    p = kvq.make_params(2, 8, 2, 256, "int2", "int2", rotation="dense", keep_fp16_copy=True)
    fake = 1 << 20  # never dereferenced: validation fails first
    cs = kvq.CacheStruct(k_codes=fake, k_meta=fake, v_codes=fake, v_meta=fake, blk_desc=fake, k_orig=fake,
                         v_orig=fake, rot_f16=fake)
    starts = (ctypes.c_int32 * 2)(0, 0)
    st = L.kvq_append(ctypes.byref(p), ctypes.byref(cs), fake, fake, starts, 4, None)
    assert st == -2 and b"dense" in L.kvq_last_error()
