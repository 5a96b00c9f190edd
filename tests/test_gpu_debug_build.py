"""The layout-checking build on the GPU.

libkvq_debug.so is the library compiled with KVQ_DEBUG: its kernels check every stream,
position, chunk, block, split-record and counter index they address against the call's
sizes and record failures instead of stopping.  A child process loads it (KVQ_LIB) and
runs every entry point over every format, rotation, the window, the certified cache, the
adaptive ladder and the per-channel factors (tests/debug_layout_run.py); no check may
fail, and its outputs must be those of the release library run here on the same inputs:
packed bytes, flags, masses and inversion counts identical, attention outputs and
certificates equal up to the fp32 order of the run-time chunk sharing.
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bit_kv_cache_append_amd as kvq
import debug_layout_run
from oracle import attention

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.timeout(600)
def test_debug_build_checks_pass_and_outputs_match(tmp_path):
    assert os.path.exists(kvq.DEBUG_LIB_PATH), "build with python -m bit_kv_cache_append_amd.build --all"
    npz = str(tmp_path / "debug_outputs.npz")
    env = dict(os.environ, KVQ_LIB=kvq.DEBUG_LIB_PATH)
    print("[debug-build] child process with the debug library", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "debug_layout_run.py"), npz], env=env,
                       capture_output=True, text=True, timeout=540)
    print(r.stdout[-3000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0, "the debug-library run failed"
    st = json.loads(r.stdout.strip().splitlines()[-1])
    assert st["lib"] == "libkvq_debug.so"
    assert st["code"] == 0 and st["failures"] == 0, f"layout checks failed: {st}"
    dbg = {k.replace("|", "/"): v for k, v in np.load(npz).items()}
    print("[debug-build] the same workloads on the release library", flush=True)
    rel = debug_layout_run.run_all()
    assert set(dbg) == set(rel) and st["outputs"] == len(rel)
    for n, a in rel.items():
        b = dbg[n]
        assert a.shape == b.shape, n
        if "/out" in n:
            d = float(attention.row_rel_err(b.reshape(-1, 1, 128), a.reshape(-1, 1, 128)).max())
            assert d <= 1e-3, f"{n}: debug and release outputs differ by {d:.2e}"
        elif "/cert" in n:
            assert np.allclose(b, a, rtol=1e-4, atol=1e-9), n
        else:
            assert np.array_equal(a, b), f"{n} differs between the debug and release libraries"
