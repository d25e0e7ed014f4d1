"""Build libgqa.so (gfx950 only) in-tree with hipcc.

    python -m grouped_query_decode_amd.build      # or build() from Python

Every source in csrc/ is compiled to an object in _build/ (in parallel) and the
objects are linked into grouped_query_decode_amd/libgqa.so; the benchmark's
measurement probes (csrc/probe/) go into a separate libgqa_probe.so.  Packed
float32 instructions are disabled for all device code.
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


def _compile(src: str, cc: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.relpath(src, CSRC).replace(os.sep, "__") + ".o")
    cmd = [cc, "-x", "hip", "-c", src, "-o", obj] + COMMON_FLAGS
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
    with ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(probe_srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, cc), srcs + probe_srcs))
    _link(objs[:len(srcs)], cc, LIB_PATH)
    _link(objs[len(srcs):], cc, PROBE_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources and {PROBE_LIB_PATH} from "
              f"{len(probe_srcs)}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
