"""Build libkvq.so (HIP, gfx950) in place.

    python -m bit_kv_cache_append_amd.build            # libkvq.so
    python -m bit_kv_cache_append_amd.build --debug    # libkvq_debug.so (layout checks)
    python -m bit_kv_cache_append_amd.build --all      # both

The debug library is the same sources compiled with KVQ_DEBUG: its kernels check
every index they address against the call's sizes and record failures for
kvq_debug_status (the release library compiles the checks out).

Every translation unit is compiled with hipcc for gfx950 only.  The write-side
unit is compiled with -ffp-contract=off so that its fp32 arithmetic keeps the
rounding order it is written in; fp32 division is correctly rounded everywhere.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libkvq.so")
OUT_DEBUG = os.path.join(HERE, "libkvq_debug.so")
BUILD = os.path.join(HERE, "_build")

ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]
SOURCES = {
    "kvq_append.hip": ["-ffp-contract=off"],
    "kvq_decode.hip": [],
    "kvq_bound.hip": [],
    "kvq_adaptive.hip": [],
    "kvq_api.cpp": [],
}


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src, extra, bdir=BUILD):
    obj = os.path.join(bdir, src + ".o")
    cmd = [hipcc()] + COMMON + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=True, debug=False):
    """Compile every translation unit and link the library; debug=True: libkvq_debug.so."""
    bdir = os.path.join(BUILD, "debug") if debug else BUILD
    out = OUT_DEBUG if debug else OUT
    flags = ["-DKVQ_DEBUG"] if debug else []
    os.makedirs(bdir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda kv: _compile(kv[0], kv[1] + flags, bdir), SOURCES.items()))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    try:
        if "--debug" not in sys.argv:
            build()
        if "--debug" in sys.argv or "--all" in sys.argv:
            build(debug=True)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
