"""Grouped-query attention on AMD MI355X: thin Python binding of libgqa.so.

The computation runs entirely in the HIP kernels of ``libgqa.so`` (built
in-tree by ``grouped_query_decode_amd.build``).  This module only checks and
marshals arguments: PyTorch tensors provide device memory, and the current
PyTorch stream is passed to the library.  There is no fallback: if the
library is missing, every call raises.

    decode(q, k_cache, v_cache, seqlens)        # one decode step, [B,H,d]
    decode_append(q, k_new, v_new, k_cache, v_cache, seqlens)  # append, then decode
    decode_noalloc(q, k_cache, v_cache, seqlens)  # decode with the library's static scratch
    prefill_causal(q, k, v)                     # causal prefill, [B,T,H,d]
    prefill_chunk(q, k_cache, v_cache, ctx_lens) # a prompt chunk after ctx cached positions
    gqkva_decode(q, k_cache, v_cache, seqlens)  # all query-group x K/V-group pairs
    gqkva_prefill_causal(q, k, v)
    meanpool_heads(w, G)                        # MHA -> GQA K/V conversion
    meanpool_heads_batch([wk, wv], G)           # several projections per launch
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "GQAError", "library_path", "load_library", "decode", "decode_append", "decode_noalloc",
    "decode_num_splits",
    "decode_workspace_bytes", "prefill_causal", "prefill_chunk", "gqkva_decode",
    "gqkva_prefill_causal", "meanpool_heads", "meanpool_heads_batch", "DTYPE_CODES",
]

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libgqa.so"
_lib = None
_workspaces: dict = {}

DTYPE_CODES = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}


class GQAError(RuntimeError):
    """A libgqa call returned a non-zero status."""

    def __init__(self, call: str, status: int, status_name: str, detail: str):
        super().__init__(f"{call}: {status_name}: {detail}")
        self.status = status
        self.status_name = status_name


def library_path() -> str:
    return os.path.join(_PKG_DIR, _LIB_NAME)


def load_library():
    """Load libgqa.so (once) and declare the C signatures from include/gqa.h."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m grouped_query_decode_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_int64
    lib.gqa_decode_num_splits.argtypes = [i32] * 5
    lib.gqa_decode_num_splits.restype = i32
    lib.gqa_decode_workspace_bytes.argtypes = [i32] * 6
    lib.gqa_decode_workspace_bytes.restype = sz
    lib.gqa_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    lib.gqa_decode.restype = i32
    lib.gqa_decode_split.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, i32,
                                     vp, sz, vp]
    lib.gqa_decode_split.restype = i32
    lib.gqa_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32,
                                      i32, vp, sz, vp]
    lib.gqa_decode_append.restype = i32
    lib.gqa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, i32, vp]
    lib.gqa_decode_noalloc.restype = i32
    lib.gqa_prefill_causal.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.gqa_prefill_causal.restype = i32
    lib.gqa_prefill_chunk.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.gqa_prefill_chunk.restype = i32
    lib.gqkva_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, i32, vp, sz, vp]
    lib.gqkva_decode.restype = i32
    lib.gqkva_decode_workspace_bytes.argtypes = [i32] * 6
    lib.gqkva_decode_workspace_bytes.restype = sz
    lib.gqkva_prefill_causal.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.gqkva_prefill_causal.restype = i32
    lib.kv_meanpool_heads.argtypes = [vp, vp, i32, i32, i64, i32, vp]
    lib.kv_meanpool_heads.restype = i32
    lib.kv_meanpool_heads_batch.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), i32, i32, i32, i64, i32, vp]
    lib.kv_meanpool_heads_batch.restype = i32
    lib.gqa_status_string.argtypes = [i32]
    lib.gqa_status_string.restype = ctypes.c_char_p
    lib.gqa_last_error.argtypes = []
    lib.gqa_last_error.restype = ctypes.c_char_p
    lib.gqa_version.argtypes = []
    lib.gqa_version.restype = i32
    _lib = lib
    return lib


def _check(call: str, status: int) -> None:
    if status != 0:
        lib = load_library()
        raise GQAError(call, status, lib.gqa_status_string(status).decode(),
                       lib.gqa_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return DTYPE_CODES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype} (float32, bfloat16 or float16)") from None


def _require_device(name: str, t: torch.Tensor, device) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_handle(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _workspace_args(workspace, dev, need: int):
    """The workspace pointer and size to pass: the caller's (checked to be on the
    call's GPU), else the cached one when the call needs any."""
    if workspace is None:
        if need <= 0:
            return None, 0
        workspace = _cached_workspace(dev, need)
    else:
        _require_device("workspace", workspace, dev)
    return workspace, workspace.numel() * workspace.element_size()


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def decode_num_splits(B: int, H: int, G: int, d: int, n_max: int) -> int:
    return int(load_library().gqa_decode_num_splits(B, H, G, d, n_max))


def decode_workspace_bytes(B: int, H: int, G: int, d: int, n_max: int, num_splits: int = 0) -> int:
    n = load_library().gqa_decode_workspace_bytes(B, H, G, d, n_max, num_splits)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid decode shape")
    return int(n)


def _cached_workspace(dev, need: int) -> torch.Tensor:
    """A zero-filled workspace per (device, current stream), grown on demand (the
    library keeps its counter header zero between calls, so it is cleared only
    when allocated).  Calls that overlap on one workspace would race, so calls
    on different streams get different workspaces."""
    key = (str(dev), _stream_handle(dev))
    t = _workspaces.get(key)
    if t is None or t.numel() < need:
        t = torch.zeros(max(need, 1 << 20), dtype=torch.uint8, device=dev)
        _workspaces[key] = t
    return t


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seqlens: torch.Tensor,
           scale: float | None = None, out: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None, num_splits: int = 0) -> torch.Tensor:
    """One GQA decode step: out[b,h] attends the first seqlens[b] cached positions.

    q [B,H,d]; k_cache, v_cache [B,G,Nmax,d]; seqlens [B] int32 (on the GPU).
    ``scale`` defaults to 1/sqrt(d) (as a float32 value).  ``num_splits`` = 0
    lets the library plan the split-N decomposition.  Without ``workspace`` a
    zero-filled buffer cached per (device, current stream) is used, so calls on
    one stream share it and calls on different streams do not.  A ``workspace``
    passed in must be a contiguous tensor on q's GPU, zero-filled before its
    first use (the library leaves it reusable); calls that may overlap must not
    share one.
    """
    lib = load_library()
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B,H,d] and k_cache [B,G,Nmax,d]")
    B, H, d = q.shape
    Bk, G, n_max, dk = k_cache.shape
    if (Bk, dk) != (B, d) or v_cache.shape != k_cache.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k_cache.shape)}, "
                         f"v {tuple(v_cache.shape)}")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share one dtype")
    if seqlens.dtype != torch.int32 or seqlens.shape != (B,):
        raise ValueError("seqlens must be an int32 tensor of shape [B]")
    dev = q.device
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("seqlens", seqlens)):
        _require_device(name, t, dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _require_device("out", out, dev)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q in shape and dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = decode_workspace_bytes(B, H, G, d, n_max, num_splits) if B > 0 else 0
    workspace, ws_bytes = _workspace_args(workspace, dev, need)
    st = lib.gqa_decode_split(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(out),
                              B, H, G, d, n_max, float(scale), _dtype_code(q), int(num_splits),
                              _ptr(workspace), ws_bytes, ctypes.c_void_p(_stream_handle(dev)))
    _check("gqa_decode", st)
    return out


def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   seqlens: torch.Tensor, out: torch.Tensor, scale: float | None = None,
                   num_splits: int = 0) -> torch.Tensor:
    """:func:`decode` through ``gqa_decode_noalloc``: the split partials live in
    the library's static per-GPU scratch, so the call allocates nothing (``out``
    must be given).  Calls that may overlap on one GPU race on that scratch."""
    lib = load_library()
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B,H,d] and k_cache [B,G,Nmax,d]")
    B, H, d = q.shape
    Bk, G, n_max, dk = k_cache.shape
    if (Bk, dk) != (B, d) or v_cache.shape != k_cache.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k_cache.shape)}, "
                         f"v {tuple(v_cache.shape)}")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share one dtype")
    if seqlens.dtype != torch.int32 or seqlens.shape != (B,):
        raise ValueError("seqlens must be an int32 tensor of shape [B]")
    dev = q.device
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("seqlens", seqlens),
                    ("out", out)):
        _require_device(name, t, dev)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib.gqa_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(out),
                                B, H, G, d, n_max, float(scale), _dtype_code(q), int(num_splits),
                                ctypes.c_void_p(_stream_handle(dev)))
    _check("gqa_decode_noalloc", st)
    return out


def decode_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                  v_cache: torch.Tensor, seqlens: torch.Tensor, scale: float | None = None,
                  out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                  num_splits: int = 0) -> torch.Tensor:
    """Append this step's k, v (k_new, v_new [B,G,d]) at slot seqlens[b]-1 of the
    caches (in place), then one decode step; see :func:`decode` for the rest."""
    lib = load_library()
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B,H,d] and k_cache [B,G,Nmax,d]")
    B, H, d = q.shape
    Bk, G, n_max, dk = k_cache.shape
    if (Bk, dk) != (B, d) or v_cache.shape != k_cache.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k_cache.shape)}, "
                         f"v {tuple(v_cache.shape)}")
    if k_new.shape != (B, G, d) or v_new.shape != (B, G, d):
        raise ValueError("k_new and v_new must be [B,G,d]")
    for t in (k_cache, v_cache, k_new, v_new):
        if t.dtype != q.dtype:
            raise TypeError("all tensors must share q's dtype")
    if seqlens.dtype != torch.int32 or seqlens.shape != (B,):
        raise ValueError("seqlens must be an int32 tensor of shape [B]")
    dev = q.device
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache),
                    ("v_cache", v_cache), ("seqlens", seqlens)):
        _require_device(name, t, dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _require_device("out", out, dev)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q in shape and dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = decode_workspace_bytes(B, H, G, d, n_max, num_splits) if B > 0 else 0
    workspace, ws_bytes = _workspace_args(workspace, dev, need)
    st = lib.gqa_decode_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                               _ptr(seqlens), _ptr(out), B, H, G, d, n_max, float(scale),
                               _dtype_code(q), int(num_splits), _ptr(workspace), ws_bytes,
                               ctypes.c_void_p(_stream_handle(dev)))
    _check("gqa_decode_append", st)
    return out


def prefill_causal(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """Causal GQA prefill: q [B,T,H,d], k/v [B,T,G,d] -> out [B,T,H,d]."""
    lib = load_library()
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B,T,H,d] and k, v [B,T,G,d]")
    B, T, H, d = q.shape
    Bk, Tk, G, dk = k.shape
    if (Bk, Tk, dk) != (B, T, d) or v.shape != k.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require_device(name, t, dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _require_device("out", out, dev)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q in shape and dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib.gqa_prefill_causal(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, T, H, G, d, float(scale),
                                _dtype_code(q), ctypes.c_void_p(_stream_handle(dev)))
    _check("gqa_prefill_causal", st)
    return out


def prefill_chunk(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, ctx_lens: torch.Tensor,
                  scale: float | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """A prompt chunk after ctx_lens[b] cached positions: q [B,T,H,d],
    k_cache/v_cache [B,G,Nmax,d] (the chunk's K/V already at ctx..ctx+T-1),
    ctx_lens [B] int32 -> out [B,T,H,d]; row t sees positions 0..ctx+t."""
    lib = load_library()
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q must be [B,T,H,d] and k_cache [B,G,Nmax,d]")
    B, T, H, d = q.shape
    Bk, G, n_max, dk = k_cache.shape
    if (Bk, dk) != (B, d) or v_cache.shape != k_cache.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k_cache.shape)}")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share one dtype")
    if ctx_lens.dtype != torch.int32 or ctx_lens.shape != (B,):
        raise ValueError("ctx_lens must be an int32 tensor of shape [B]")
    dev = q.device
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("ctx_lens", ctx_lens)):
        _require_device(name, t, dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _require_device("out", out, dev)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q in shape and dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib.gqa_prefill_chunk(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(ctx_lens), _ptr(out),
                               B, T, H, G, d, n_max, float(scale), _dtype_code(q),
                               ctypes.c_void_p(_stream_handle(dev)))
    _check("gqa_prefill_chunk", st)
    return out


def gqkva_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seqlens: torch.Tensor,
                 scale: float | None = None, out: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None, num_splits: int = 0) -> torch.Tensor:
    """GQKVA decode: q [B,g_q,d], caches [B,g_kv,Nmax,d] -> out [B, g_q*g_kv, d]; output
    head h pairs query group h // g_kv with K/V group h % g_kv."""
    lib = load_library()
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B,g_q,d] and k_cache [B,g_kv,Nmax,d]")
    B, g_q, d = q.shape
    Bk, g_kv, n_max, dk = k_cache.shape
    if (Bk, dk) != (B, d) or v_cache.shape != k_cache.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k_cache.shape)}")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share one dtype")
    if seqlens.dtype != torch.int32 or seqlens.shape != (B,):
        raise ValueError("seqlens must be an int32 tensor of shape [B]")
    dev = q.device
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("seqlens", seqlens)):
        _require_device(name, t, dev)
    shape = (B, g_q * g_kv, d)
    if out is None:
        out = torch.empty(shape, dtype=q.dtype, device=dev)
    else:
        _require_device("out", out, dev)
        if out.shape != shape or out.dtype != q.dtype:
            raise ValueError("out must be [B, g_q*g_kv, d] in q's dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = 0
    if B > 0:
        need = lib.gqkva_decode_workspace_bytes(B, g_q, g_kv, d, n_max, num_splits)
        if need == ctypes.c_size_t(-1).value:
            raise ValueError("invalid GQKVA decode shape")
    workspace, ws_bytes = _workspace_args(workspace, dev, need)
    st = lib.gqkva_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(out), B, g_q,
                          g_kv, d, n_max, float(scale), _dtype_code(q), int(num_splits),
                          _ptr(workspace), ws_bytes, ctypes.c_void_p(_stream_handle(dev)))
    _check("gqkva_decode", st)
    return out


def gqkva_prefill_causal(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
                         out: torch.Tensor | None = None) -> torch.Tensor:
    """Causal GQKVA prefill: q [B,T,g_q,d], k/v [B,T,g_kv,d] -> out [B,T,g_q*g_kv,d]."""
    lib = load_library()
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B,T,g_q,d] and k, v [B,T,g_kv,d]")
    B, T, g_q, d = q.shape
    Bk, Tk, g_kv, dk = k.shape
    if (Bk, Tk, dk) != (B, T, d) or v.shape != k.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require_device(name, t, dev)
    shape = (B, T, g_q * g_kv, d)
    if out is None:
        out = torch.empty(shape, dtype=q.dtype, device=dev)
    else:
        _require_device("out", out, dev)
        if out.shape != shape or out.dtype != q.dtype:
            raise ValueError("out must be [B, T, g_q*g_kv, d] in q's dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib.gqkva_prefill_causal(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, T, g_q, g_kv, d,
                                  float(scale), _dtype_code(q), ctypes.c_void_p(_stream_handle(dev)))
    _check("gqkva_prefill_causal", st)
    return out


def meanpool_heads(w: torch.Tensor, G: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """MHA -> GQA conversion: w [H, ...] -> [G, ...], the mean over each group's heads."""
    lib = load_library()
    if w.dim() < 1:
        raise ValueError("w must have a leading head dimension")
    H = w.shape[0]
    per_head = w[0].numel() if H > 0 else 0
    _require_device("w", w, w.device)
    if out is None:
        out = torch.empty((G,) + tuple(w.shape[1:]), dtype=w.dtype, device=w.device)
    else:
        _require_device("out", out, w.device)
        if out.shape != (G,) + tuple(w.shape[1:]) or out.dtype != w.dtype:
            raise ValueError("out must be [G, ...] in w's dtype")
    st = lib.kv_meanpool_heads(_ptr(w), _ptr(out), H, G, per_head, _dtype_code(w),
                               ctypes.c_void_p(_stream_handle(w.device)))
    _check("kv_meanpool_heads", st)
    return out


MEANPOOL_MAX_BATCH = 16


def meanpool_heads_batch(ws: list, G: int, outs: list | None = None) -> list:
    """kv_meanpool_heads_batch: several projections of one shape and dtype
    (e.g. a layer's K and V weights), each [H, ...] -> [G, ...], in one launch
    per MEANPOOL_MAX_BATCH projections."""
    lib = load_library()
    if not ws:
        return []
    w0 = ws[0]
    if w0.dim() < 1:
        raise ValueError("w must have a leading head dimension")
    for w in ws:
        if w.shape != w0.shape or w.dtype != w0.dtype:
            raise ValueError("every projection must have the first one's shape and dtype")
        _require_device("w", w, w0.device)
    H = w0.shape[0]
    per_head = w0[0].numel() if H > 0 else 0
    if outs is None:
        outs = [torch.empty((G,) + tuple(w0.shape[1:]), dtype=w0.dtype, device=w0.device) for _ in ws]
    elif len(outs) != len(ws):
        raise ValueError("one output per projection")
    for o in outs:
        _require_device("out", o, w0.device)
        if o.shape != (G,) + tuple(w0.shape[1:]) or o.dtype != w0.dtype:
            raise ValueError("out must be [G, ...] in w's dtype")
    for i in range(0, len(ws), MEANPOOL_MAX_BATCH):
        chunk_in, chunk_out = ws[i:i + MEANPOOL_MAX_BATCH], outs[i:i + MEANPOOL_MAX_BATCH]
        n = len(chunk_in)
        arr_in = (ctypes.c_void_p * n)(*[w.data_ptr() for w in chunk_in])
        arr_out = (ctypes.c_void_p * n)(*[o.data_ptr() for o in chunk_out])
        st = lib.kv_meanpool_heads_batch(arr_in, arr_out, n, H, G, per_head, _dtype_code(w0),
                                         ctypes.c_void_p(_stream_handle(w0.device)))
        _check("kv_meanpool_heads_batch", st)
    return outs
