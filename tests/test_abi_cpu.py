"""Host-side checks of libgqa.so's C ABI.  No GPU: every call here returns before
the library makes any HIP call (argument checks, empty problems, planning)."""

import ctypes
import os
import re

import pytest

import grouped_query_decode_amd as gqa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
F32, BF16 = 0, 1
P = ctypes.c_void_p(4096)        # aligned, non-null, never dereferenced on these paths
P_MIS = ctypes.c_void_p(4100)    # misaligned


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gqa.library_path()):
        pytest.fail("libgqa.so is not built: run __graft_entry__.build() first")
    return gqa.load_library()


def test_header_declares_the_api():
    names = declared_functions()
    for n in ("gqa_decode", "gqa_decode_split", "gqa_decode_append", "gqa_prefill_causal",
              "gqa_prefill_chunk", "gqkva_decode", "gqkva_decode_workspace_bytes",
              "gqkva_prefill_causal", "kv_meanpool_heads", "kv_meanpool_heads_batch",
              "gqa_decode_workspace_bytes", "gqa_decode_num_splits", "gqa_status_string",
              "gqa_last_error", "gqa_version", "gqa_decode_noalloc"):
        assert n in names, n


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(gqa.library_path())
    for name in declared_functions():
        assert hasattr(raw, name), f"{name} declared in include/gqa.h but not exported"


def test_probe_library_exports_its_header():
    """The benchmark's measurement probes live in their own libgqa_probe.so."""
    path = os.path.join(os.path.dirname(gqa.library_path()), "libgqa_probe.so")
    if not os.path.exists(path):
        pytest.fail("libgqa_probe.so is not built: run __graft_entry__.build() first")
    raw = ctypes.CDLL(path)
    names = declared_functions(os.path.join(ROOT, "include", "gqa_probe.h"))
    assert names == ["gqa_probe_hbm_read", "gqa_probe_lds_rate", "gqa_probe_time_decode_calls",
                     "gqa_probe_valu_rate"]
    for name in names:
        assert hasattr(raw, name)
    f = raw.gqa_probe_hbm_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p]
    f.restype = ctypes.c_int
    # invalid arguments are refused on the host (nothing enqueued, no GPU needed)
    assert f(P, 1 << 20, P, 1024, 3, None) == 1           # unroll
    assert f(P, 1000, P, 1024, 8, None) == 1              # not a multiple of 16
    assert f(P_MIS, 1 << 20, P, 1024, 8, None) == 1       # misaligned
    assert f(ctypes.c_void_p(0), 1 << 20, P, 1024, 8, None) == 1
    assert f(P, 1 << 20, P, 0, 8, None) == 1              # blocks
    r = raw.gqa_probe_valu_rate
    r.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    r.restype = ctypes.c_int
    assert r(P, 3, 1024, None) == 1                       # kind
    assert r(ctypes.c_void_p(0), 0, 1024, None) == 1
    assert r(P, 0, 0, None) == 1
    lr = raw.gqa_probe_lds_rate
    lr.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lr.restype = ctypes.c_int
    assert lr(P, 2, 512, None) == 1                       # kind
    assert lr(ctypes.c_void_p(0), 0, 512, None) == 1
    assert lr(P, 1, 0, None) == 1
    t = raw.gqa_probe_time_decode_calls
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    t.argtypes = ([vp] * 5 + [i32, vp] + [i32] * 5 + [ctypes.c_float] + [i32] * 2 +
                  [vp, ctypes.c_size_t, i32, i32, vp, ctypes.c_size_t, vp, vp, vp])
    t.restype = i32
    arr = (vp * 1)(P.value)
    ms = ctypes.c_float(0.0)
    fn = ctypes.cast(ctypes.CDLL(gqa.library_path()).gqa_decode_split, vp)
    args = lambda f, n_in, calls, H, G, lead=None: (f, arr, arr, arr, arr, n_in, P, 1, H, G, 128,  # noqa: E731
                                                    16, 0.1, 1, 0, None, 0, 1, calls, lead, 1 << 20,
                                                    None, None, ctypes.byref(ms))
    assert t(*args(vp(0), 1, 10, 8, 2)) == 1              # no entry point
    assert t(*args(fn, 0, 10, 8, 2)) == 1                 # no inputs
    assert t(*args(fn, 1, 0, 8, 2)) == 1                  # no calls
    assert t(*args(fn, 1, 10, 8, 2, lead=P)) == 1         # a lead read without a sink
    # a call the library refuses on the host (H not a multiple of G) stops the
    # loop with status 2 before any GPU work
    assert t(*args(fn, 1, 10, 8, 3)) == 2


def test_status_strings(lib):
    assert lib.gqa_status_string(0) == b"GQA_OK"
    assert lib.gqa_status_string(1) == b"GQA_ERR_INVALID_ARG"
    assert lib.gqa_status_string(3) == b"GQA_ERR_WORKSPACE"
    assert lib.gqa_status_string(99) == b"GQA_ERR_UNKNOWN"
    assert lib.gqa_version() >= 100


def _decode(lib, q=P, k=P, v=P, sl=P, out=P, B=2, H=8, G=2, d=64, n=128, scale=0.125, dt=BF16,
            splits=0, ws=None, ws_bytes=0):
    return lib.gqa_decode_split(q, k, v, sl, out, B, H, G, d, n, scale, dt, splits,
                                ws if ws is not None else ctypes.c_void_p(0), ws_bytes, None)


def test_decode_rejects_bad_arguments(lib):
    assert _decode(lib, H=6, G=4) == INVALID
    assert "multiple" in lib.gqa_last_error().decode()
    assert _decode(lib, G=0) == INVALID
    assert _decode(lib, B=-1) == INVALID
    assert _decode(lib, n=-5) == INVALID
    assert _decode(lib, dt=7) == INVALID
    assert _decode(lib, scale=float("nan")) == INVALID
    assert _decode(lib, scale=float("inf")) == INVALID
    assert _decode(lib, q=ctypes.c_void_p(0)) == INVALID
    assert _decode(lib, sl=ctypes.c_void_p(0)) == INVALID
    assert _decode(lib, k=P_MIS) == INVALID
    assert "aligned" in lib.gqa_last_error().decode()
    assert _decode(lib, splits=-1) == INVALID
    assert _decode(lib, d=96) == UNSUPPORTED
    assert _decode(lib, d=256) == UNSUPPORTED


def test_decode_empty_batch_is_a_noop(lib):
    # B = 0: valid, nothing to do, no pointer is looked at
    z = ctypes.c_void_p(0)
    assert _decode(lib, q=z, k=z, v=z, sl=z, out=z, B=0) == OK
    assert lib.gqa_last_error() == b""


def test_decode_workspace_checked_before_launch(lib):
    # 4 sequences x 8 K/V heads: 32 work groups, planned as 4 splits
    need = lib.gqa_decode_workspace_bytes(4, 32, 8, 128, 1024, 0)
    assert need > 0
    assert _decode(lib, B=4, H=32, G=8, d=128, n=1024) == WORKSPACE
    assert _decode(lib, B=4, H=32, G=8, d=128, n=1024, ws=P, ws_bytes=need - 1) == WORKSPACE
    assert _decode(lib, B=4, H=32, G=8, d=128, n=1024, ws=P_MIS, ws_bytes=need) == WORKSPACE
    # forced splits need one whatever the planner would choose
    assert _decode(lib, B=16, H=32, G=8, d=128, n=1024, splits=2) == WORKSPACE


def test_split_planner_is_host_only_and_consistent(lib):
    shapes = [(1, 8, 2, 64, 128), (16, 32, 32, 128, 1024), (16, 32, 8, 128, 1024),
              (16, 32, 1, 128, 1024), (32, 64, 8, 64, 2048), (64, 32, 8, 128, 32768)]
    for B, H, G, d, n in shapes:
        S = lib.gqa_decode_num_splits(B, H, G, d, n)
        assert 1 <= S <= max(1, n)
        ws = lib.gqa_decode_workspace_bytes(B, H, G, d, n, 0)
        if S == 1:
            assert ws == 0
        else:
            o_bytes = B * H * S * d * 4
            assert ws == 65536 + (o_bytes + 255) // 256 * 256 + B * H * S * 2 * 4
        assert ws == lib.gqa_decode_workspace_bytes(B, H, G, d, n, S)
    # long ragged caches are cut into bounded slices
    assert lib.gqa_decode_num_splits(64, 32, 8, 128, 32768) >= 11
    # unsplit from 128 work groups per split, else about 192 in all; splits of
    # 256 .. 3072 positions (32 queries per K/V head count as two work groups)
    planned = {(16, 32, 32, 128, 1024): 1, (16, 32, 8, 128, 1024): 1, (16, 32, 4, 128, 1024): 3,
               (16, 32, 1, 128, 1024): 4, (32, 64, 8, 64, 2048): 1, (1, 8, 2, 64, 128): 1,
               (64, 32, 8, 128, 32768): 11, (8, 32, 8, 128, 1024): 3, (4, 32, 8, 128, 4096): 6}
    for shape, S in planned.items():
        assert lib.gqa_decode_num_splits(*shape) == S, shape
    # forced split counts
    assert lib.gqa_decode_workspace_bytes(1, 8, 2, 64, 128, 1) == 0
    assert lib.gqa_decode_workspace_bytes(1, 8, 2, 64, 128, 7) > 0
    # invalid shapes
    assert lib.gqa_decode_num_splits(1, 6, 4, 64, 128) == 0
    assert lib.gqa_decode_workspace_bytes(1, 6, 4, 64, 128, 0) == ctypes.c_size_t(-1).value


def test_prefill_rejects_bad_arguments(lib):
    def call(q=P, k=P, v=P, out=P, B=2, T=64, H=8, G=2, d=128, scale=0.1, dt=BF16):
        return lib.gqa_prefill_causal(q, k, v, out, B, T, H, G, d, scale, dt, None)
    assert call(H=8, G=3) == INVALID
    assert call(T=-1) == INVALID
    assert call(v=ctypes.c_void_p(0)) == INVALID
    assert call(out=P_MIS) == INVALID
    assert call(scale=float("-inf")) == INVALID
    assert call(d=80) == UNSUPPORTED
    # 2^32 query rows: within the element guard (2^38 elements) but past the
    # kernels' 32-bit row count
    assert call(B=65536, T=65536, H=1, G=1, d=64) == INVALID
    z = ctypes.c_void_p(0)
    assert call(q=z, k=z, v=z, out=z, T=0) == OK
    assert call(q=z, k=z, v=z, out=z, B=0) == OK


def test_meanpool_rejects_bad_arguments(lib):
    def call(w=P, o=P, H=64, G=8, n=4096 * 64, dt=BF16):
        return lib.kv_meanpool_heads(w, o, H, G, n, dt, None)
    assert call(G=3) == INVALID
    assert call(G=0) == INVALID
    assert call(n=-1) == INVALID
    assert call(w=ctypes.c_void_p(0)) == INVALID
    assert call(o=P_MIS) == INVALID
    assert call(dt=5) == INVALID
    assert call(w=ctypes.c_void_p(0), o=ctypes.c_void_p(0), n=0) == OK


def test_meanpool_batch_rejects_bad_arguments(lib):
    def arr(*ptrs):
        return (ctypes.c_void_p * len(ptrs))(*ptrs)

    def call(ws=None, os_=None, count=2, H=64, G=8, n=4096 * 64, dt=BF16):
        ws = arr(P, P) if ws is None else ws
        os_ = arr(P, P) if os_ is None else os_
        return lib.kv_meanpool_heads_batch(ws, os_, count, H, G, n, dt, None)
    assert call(count=-1) == INVALID
    assert call(count=17) == INVALID            # beyond GQA_MEANPOOL_MAX_BATCH
    assert call(G=3) == INVALID
    assert call(ws=arr(P, ctypes.c_void_p(0))) == INVALID
    assert call(os_=arr(P, P_MIS)) == INVALID
    assert call(ws=None, count=2, dt=5) == INVALID
    assert lib.kv_meanpool_heads_batch(None, None, 2, 64, 8, 4096, BF16, None) == INVALID
    # count 0 and empty heads are valid no-ops (nothing is read)
    assert lib.kv_meanpool_heads_batch(None, None, 0, 64, 8, 4096, BF16, None) == OK
    assert call(ws=arr(ctypes.c_void_p(0), ctypes.c_void_p(0)), n=0) == OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(gqa, "_lib", None)
    monkeypatch.setattr(gqa, "_PKG_DIR", str(tmp_path))
    with pytest.raises(RuntimeError, match="no fallback"):
        gqa.load_library()


def test_binding_rejects_host_tensors(lib):
    import torch
    q = torch.zeros(1, 8, 64)
    k = torch.zeros(1, 2, 16, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        gqa.decode(q, k, k, torch.zeros(1, dtype=torch.int32))
    # a caller's workspace is checked like the tensors (never passed on as a host pointer)
    with pytest.raises(ValueError, match="workspace must be a GPU tensor"):
        gqa._workspace_args(torch.zeros(1 << 16, dtype=torch.uint8), torch.device("cuda:0"), 4096)
    assert gqa._workspace_args(None, torch.device("cuda:0"), 0) == (None, 0)


def _append(lib, q=P, kn=P, vn=P, k=P, v=P, sl=P, out=P, B=2, H=8, G=2, d=64, n=128, scale=0.125,
            dt=BF16, splits=0, ws=None, ws_bytes=0):
    return lib.gqa_decode_append(q, kn, vn, k, v, sl, out, B, H, G, d, n, scale, dt, splits,
                                 ws if ws is not None else ctypes.c_void_p(0), ws_bytes, None)


def test_decode_append_rejects_bad_arguments(lib):
    z = ctypes.c_void_p(0)
    assert _append(lib, kn=z) == INVALID
    assert _append(lib, vn=z) == INVALID
    assert _append(lib, kn=P_MIS) == INVALID
    assert "aligned" in lib.gqa_last_error().decode()
    assert _append(lib, H=6, G=4) == INVALID
    assert _append(lib, d=96) == UNSUPPORTED
    assert _append(lib, B=4, H=32, G=8, d=128, n=1024) == WORKSPACE
    # B = 0: nothing to do, no pointer looked at
    assert _append(lib, q=z, kn=z, vn=z, k=z, v=z, sl=z, out=z, B=0) == OK


def _chunk(lib, q=P, k=P, v=P, ctx=P, out=P, B=2, T=16, H=8, G=2, d=64, n=128, scale=0.125, dt=BF16):
    return lib.gqa_prefill_chunk(q, k, v, ctx, out, B, T, H, G, d, n, scale, dt, None)


def test_prefill_chunk_rejects_bad_arguments(lib):
    z = ctypes.c_void_p(0)
    assert _chunk(lib, ctx=z) == INVALID
    assert _chunk(lib, n=0) == INVALID
    assert _chunk(lib, H=6, G=4) == INVALID
    assert _chunk(lib, k=P_MIS) == INVALID
    assert _chunk(lib, dt=9) == INVALID
    assert _chunk(lib, scale=float("nan")) == INVALID
    assert _chunk(lib, d=80) == UNSUPPORTED
    assert _chunk(lib, q=z, k=z, v=z, ctx=z, out=z, B=0) == OK
    assert _chunk(lib, q=z, k=z, v=z, ctx=z, out=z, T=0) == OK


def test_gqkva_arguments_and_workspace(lib):
    z = ctypes.c_void_p(0)
    def dec(**kw):
        a = dict(q=P, k=P, v=P, sl=P, out=P, B=2, gq=3, gkv=2, d=64, n=128, scale=0.1, dt=BF16, S=0)
        a.update(kw)
        return lib.gqkva_decode(a["q"], a["k"], a["v"], a["sl"], a["out"], a["B"], a["gq"], a["gkv"], a["d"],
                                a["n"], a["scale"], a["dt"], a["S"], z, 0, None)
    assert dec(gkv=0) == INVALID
    assert dec(gq=0) == INVALID
    assert dec(d=96) == UNSUPPORTED
    assert dec(q=z, k=z, v=z, sl=z, out=z, B=0) == OK
    # a ratio that is not a whole number is fine for GQKVA: only the workspace is missing here
    assert dec(B=4, gq=3, gkv=8, d=128, n=1024) == WORKSPACE
    need = lib.gqkva_decode_workspace_bytes(4, 3, 8, 128, 1024, 0)
    S = lib.gqa_decode_num_splits(4, 8, 8, 128, 1024)           # same plan as G = 8 K/V heads
    assert S > 1
    assert need == 65536 + (4 * 24 * S * 128 * 4 + 255) // 256 * 256 + 4 * 24 * S * 2 * 4
    assert lib.gqkva_decode_workspace_bytes(16, 3, 8, 128, 1024, 0) == 0   # 128 work groups: unsplit
    assert lib.gqkva_decode_workspace_bytes(16, 3, 0, 128, 1024, 0) == ctypes.c_size_t(-1).value
    assert lib.gqkva_prefill_causal(z, z, z, z, 0, 16, 2, 3, 64, 0.1, BF16, None) == OK
    assert lib.gqkva_prefill_causal(P, P, P, P, 1, 16, 2, 0, 64, 0.1, BF16, None) == INVALID


C_CONSUMER = r"""
#include <stdio.h>
#include <string.h>
#include "gqa.h"

/* Host-only calls of the C ABI from plain C: planning, sizes and argument
   errors all return before any GPU work. */
int main(void) {
  char buf[16] __attribute__((aligned(16)));
  void* p = buf;
  int32_t lens[2] __attribute__((aligned(16))) = {1, 1};
  if (gqa_version() < 100) return 1;
  if (strcmp(gqa_status_string(GQA_OK), "GQA_OK") != 0) return 2;
  int s = gqa_decode_num_splits(16, 32, 8, 128, 1024);
  size_t ws = gqa_decode_workspace_bytes(16, 32, 8, 128, 1024, 0);
  if (s < 1 || (s > 1 && ws == 0)) return 3;
  /* H not a multiple of G: rejected on the host */
  gqa_status st = gqa_decode(p, p, p, lens, p, 2, 6, 4, 64, 16, 0.125f, GQA_DTYPE_BF16, NULL, 0, NULL);
  if (st != GQA_ERR_INVALID_ARG || strlen(gqa_last_error()) == 0) return 4;
  /* an empty batch is a successful no-op */
  if (gqa_prefill_causal(p, p, p, p, 0, 16, 8, 2, 64, 0.125f, GQA_DTYPE_BF16, NULL) != GQA_OK) return 5;
  printf("splits=%d workspace=%zu version=%d\n", s, ws, gqa_version());
  return 0;
}
"""


def test_plain_c_consumer(tmp_path, lib):
    """The header is C (not only C++): a C99 program includes it, links
    libgqa.so and makes host-side calls."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "consumer.c"
    src.write_text(C_CONSUMER)
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(gqa.library_path())
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                    "-o", str(exe), "-L", libdir, "-lgqa", f"-Wl,-rpath,{libdir}"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "splits=" in r.stdout


ABI_MAIN = r"""
#include "internal.h"
#include <cstdio>
int main(int argc, char**) {
  // an empty decode problem (B = 0) launches nothing once the check passes
  auto d = gqa::problem_for<gqa::DecodeProblem>();
  const hipError_t ed = gqa::launch_decode_mfma(d, nullptr);
  hipError_t ep = hipSuccess;
  if (argc > 1) {      // only with a mis-sized structure: refused before use
    auto p = gqa::problem_for<gqa::PrefillProblem>();
    ep = gqa::launch_prefill_mfma(p, nullptr);
  }
  std::printf("decode=%d prefill=%d\n", int(ed), int(ep));
  return (ed == gqa::kAbiMismatch && ep == gqa::kAbiMismatch) ? 0 : 1;
}
"""


@pytest.mark.parametrize("stale", [False, True])
def test_kernel_launchers_refuse_a_stale_argument_structure(tmp_path, lib, stale):
    """A program built against a copy of the internal header whose decode and
    prefill argument structures gained a field (as a stale or newer copy would)
    hands the library's launchers structures of the wrong size: they must
    refuse before any HIP call (this runs without a GPU).  With the header as
    shipped the same program's empty decode problem passes the check and
    launches nothing."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("no C++ compiler or ROCm headers")
    text = open(os.path.join(ROOT, "grouped_query_decode_amd", "csrc", "internal.h")).read()
    if stale:
        for anchor in ("  int dtype;                // kBF16 or kF16\n  HeadMap hm;\n  // G work",
                       "  const int32_t* ctx_lens;  // [B] or null\n"):
            assert text.count(anchor) == 1, anchor
            text = text.replace(anchor, "  const void* extra_field;\n" + anchor)
    (tmp_path / "internal.h").write_text(text)
    (tmp_path / "main.cpp").write_text(ABI_MAIN)
    exe = tmp_path / "abi_main"
    libdir = os.path.dirname(gqa.library_path())
    subprocess.run([gxx, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I", str(tmp_path), str(tmp_path / "main.cpp"), "-o", str(exe), "-L", libdir,
                    "-lgqa", f"-Wl,-rpath,{libdir}"], check=True)
    r = subprocess.run([str(exe)] + (["both"] if stale else []), capture_output=True, text=True,
                       timeout=60)
    if stale:
        assert r.returncode == 0, (r.stdout, r.stderr)
    else:
        assert r.returncode == 1 and r.stdout.strip() == "decode=0 prefill=0", (r.stdout, r.stderr)


def test_decode_noalloc_host_checks(lib):
    """gqa_decode_noalloc rejects invalid arguments and shapes whose split
    partials exceed its static scratch on the host, before any HIP call."""
    def call(B=2, H=8, G=2, d=64, n=128, splits=0, q=P, sl=P, dt=BF16):
        return lib.gqa_decode_noalloc(q, P, P, sl, P, B, H, G, d, n, 0.125, dt, splits, None)
    assert call(H=6, G=4) == INVALID
    assert call(q=ctypes.c_void_p(0)) == INVALID
    assert call(sl=ctypes.c_void_p(0)) == INVALID
    assert call(q=P_MIS) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(dt=9) == INVALID
    assert call(splits=-1) == INVALID
    assert call(B=0) == OK
    # 64 sequences x 1024 heads x d=128 in 16 splits: ~537 MB of partials
    assert call(B=64, H=1024, G=1, d=128, n=4096, splits=16) == WORKSPACE
    assert "static scratch" in lib.gqa_last_error().decode()
    need = lib.gqa_decode_workspace_bytes(64, 32, 8, 128, 32768, 0)
    assert 0 < need <= 32 << 20          # the ragged 32k workload fits
