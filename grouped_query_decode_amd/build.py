"""Build libgqa.so (gfx950 only) in-tree with hipcc.

    python -m grouped_query_decode_amd.build      # or build() from Python

Every source in csrc/ is compiled to an object in _build/ (in parallel) and the
objects are linked into grouped_query_decode_amd/libgqa.so.  Two measurement
libraries are built beside it: libgqa_probe.so (the benchmark's HBM read
probe, csrc/probe/) and libgqa_timeline.so (the same sources compiled with
GQA_DECODE_TIMELINE: the matrix-core decode kernel also records per-workgroup
phase timestamps; used by ``bench.py --timeline`` only).  Packed float32
instructions are disabled for all device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libgqa.so")
PROBE_DIR = os.path.join(CSRC, "probe")
PROBE_LIB_PATH = os.path.join(PKG_DIR, "libgqa_probe.so")
TIMELINE_LIB_PATH = os.path.join(PKG_DIR, "libgqa_timeline.so")

ARCH = "gfx950"
COMMON_FLAGS = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgqa.so)")


def sources(folder: str = CSRC) -> list[str]:
    return sorted(os.path.join(folder, f) for f in os.listdir(folder)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(src: str, cc: str, variant: str = "") -> str:
    obj = os.path.join(BUILD_DIR, variant + os.path.relpath(src, CSRC).replace(os.sep, "__") + ".o")
    cmd = [cc, "-x", "hip", "-c", src, "-o", obj] + COMMON_FLAGS
    if variant == "timeline__":
        cmd.append("-DGQA_DECODE_TIMELINE=1")
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs: list[str], cc: str, path: str) -> None:
    tmp = path + ".tmp"
    cmd = [cc, "-shared", "-o", tmp] + objs + [f"--offload-arch={ARCH}", "-fPIC"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    probe_srcs = sources(PROBE_DIR)
    jobs = [(s, "") for s in srcs + probe_srcs] + [(s, "timeline__") for s in srcs]
    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], cc, j[1]), jobs))
    n, m = len(srcs), len(probe_srcs)
    _link(objs[:n], cc, LIB_PATH)
    _link(objs[n:n + m], cc, PROBE_LIB_PATH)
    _link(objs[n + m:], cc, TIMELINE_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {n} sources, {PROBE_LIB_PATH} from {m}, "
              f"{TIMELINE_LIB_PATH} from {n}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
