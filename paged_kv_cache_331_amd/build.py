"""Build the gfx950 HIP library ``libpa_gfx950.so`` in-tree with hipcc, and
the benchmark's read-probe library ``libpa_probe_gfx950.so`` beside it.

Usage: ``python -m paged_kv_cache_331_amd.build`` (or ``__graft_entry__.build()``).
Every call recompiles. Objects go to ``_build/`` next to this file; the
library is linked to a temporary name and renamed into place.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libpa_gfx950.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ("pa_api.hip", "pa_decode.hip", "pa_cache.hip", "pa_prefill.hip",
           "pa_pool.cpp")
ARCH = "gfx950"
# Read-bandwidth probes used by bench.py only: a library of their own.
PROBE_SOURCE = os.path.join(CSRC, "probe", "pa_probe.hip")
PROBE_LIB_PATH = os.path.join(PKG, "libpa_probe_gfx950.so")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-function",
    # No packed-fp32 VALU instructions anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Matrix-core accumulators in VGPRs: with AGPR accumulators every
    # attention step copied them out for the (rarely taken) softmax rescale;
    # prefill measured 6% faster without those copies.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    path = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError(f"hipcc not found (looked for {path})")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in res.stdout.splitlines()
                    if "packed-fp32-ops" not in line)   # host pass does not know the feature
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link the shared library."""
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([cc, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    probe_obj = os.path.join(BUILD_DIR, "pa_probe.o")
    cmds.append([cc, *COMMON_FLAGS, "-c", PROBE_SOURCE, "-o", probe_obj])
    with ThreadPoolExecutor(min(len(cmds), 8)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    for path, inputs in ((LIB_PATH, objs), (PROBE_LIB_PATH, [probe_obj])):
        tmp = path + f".tmp{os.getpid()}"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *inputs], verbose)
        os.replace(tmp, path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
