"""ctypes binding of libvsa.so (argument marshalling only).

Every step of the computation runs in the HIP kernels behind include/vsa.h;
this module checks tensor dtypes, devices and shapes, hands raw device
pointers and the current HIP stream to the C ABI, and turns a non-OK status
into VSAError.  There is no fallback path: without the built library every
call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvsa.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "vsa.h")
BLOCK = 64
HEAD_DIM = 128

_lib = None
_lock = threading.Lock()

_c_void_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_size_t = ctypes.c_size_t
_f32 = ctypes.c_float

# (name, restype, argtypes)
_SIGNATURES = {
    "vsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "vsa_fwd_workspace_size": (_size_t, [_i32, _i32, _i32, _i32]),
    "vsa_fwd": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                               _i32, _i32, _i32, _i32, _i32, _f32, _c_void_p, _size_t, _c_void_p]),
    "vsa_fwd_ex": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                  _i32, _i32, _i32, _i32, _i32, _f32, ctypes.c_uint32, _c_void_p,
                                  _size_t, _c_void_p]),
    "vsa_fwd_prepacked_ex": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                            _i32, _i32, _i32, _i32, _i32, _f32, ctypes.c_uint32,
                                            _c_void_p, _size_t, _c_void_p]),
    "vsa_fwd_noalloc_max_bytes": (_size_t, []),
    "vsa_fwd_noalloc": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                       _c_void_p, _i32, _i32, _i32, _i32, _i32, _f32, _c_void_p]),
    "vsa_pack_values": (ctypes.c_int, [_c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _c_void_p,
                                       _size_t, _c_void_p]),
    "vsa_fwd_prepacked": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                         _i32, _i32, _i32, _i32, _i32, _f32, _c_void_p, _size_t,
                                         _c_void_p]),
    "vsa_preprocess": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                      _i32, _i32, _i32, _i32, _c_void_p]),
    "vsa_fwd_proxy_workspace_size": (_size_t, [_i32, _i32, _i32, _i32, _i32]),
    "vsa_fwd_proxy": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                     _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _i32,
                                     _i32, _f32, _c_void_p, _size_t, _c_void_p]),
    "vsa_fwd_lse": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                   _c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _i32, _f32,
                                   _c_void_p, _size_t, _c_void_p]),
    "vsa_merge": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                 _i32, _i32, _i32, _i32, _c_void_p]),
    "vsa_fwd_proxy_bitmask": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                             _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32,
                                             _i32, _i32, _i32, _f32, _c_void_p, _size_t,
                                             _c_void_p]),
    "vsa_fwd_proxy_bsr": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32,
                                         _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i32,
                                         _i32, _i32, _i32, _i32, _f32, _c_void_p, _size_t,
                                         _c_void_p]),
    "vsa_kc_stats": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32,
                                    _i32, _i32, _i32, _c_void_p]),
    "vsa_route_workspace_size": (_size_t, [_i32, _i32, _i32]),
    "vsa_route_topk": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32,
                                      _i32, _i32, _c_void_p, _size_t, _c_void_p]),
    "vsa_cube_count": (_size_t, [_i32, _i32, _i32]),
    "vsa_cube_vbs": (ctypes.c_int, [_i32, _i32, _i32, _c_void_p, _size_t]),
    "vsa_tile": (ctypes.c_int, [_c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _i32, _i32,
                                _c_void_p]),
    "vsa_untile": (ctypes.c_int, [_c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _i32, _i32,
                                  _c_void_p]),
}

VSA_OK = 0
FLAG_SHARED_SWEEP = 1      # VSA_FLAG_SHARED_SWEEP


class VSAError(RuntimeError):
    """A libvsa call returned a non-OK status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)}")


def load_library() -> ctypes.CDLL:
    """Load the in-tree libvsa.so (raises ImportError if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load_library().vsa_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != VSA_OK:
        raise VSAError(fn, status)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, device: torch.device, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be in GPU memory (got {t.device})")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _default_scale(sm_scale):
    return 1.0 / math.sqrt(HEAD_DIM) if sm_scale is None else float(sm_scale)


# Workspace cache: one buffer per (device, stream), reused by later calls of
# the same size on that stream.  Calls on one stream run in order, so they may
# share it; calls on different streams get different buffers (the library
# requires that calls sharing a workspace do not overlap in time).  A buffer is
# allocated while its stream is current, so the caching allocator orders its
# reuse after the work queued on that stream.
_ws_cache: dict = {}


def _workspace(device: torch.device, nbytes: int) -> torch.Tensor:
    key = (device, torch.cuda.current_stream(device).cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() != nbytes + 256:
        ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        _ws_cache.pop(key, None)
        while len(_ws_cache) >= 8:   # buffers of streams no longer in use
            _ws_cache.pop(next(iter(_ws_cache)))
        _ws_cache[key] = ws
    off = (-ws.data_ptr()) % 256
    return ws[off:off + nbytes]


def fwd_workspace_size(batch: int, seq_len: int, heads: int, head_dim: int = HEAD_DIM) -> int:
    return int(load_library().vsa_fwd_workspace_size(batch, seq_len, heads, head_dim))


def proxy_workspace_size(batch: int, seq_len: int, prefix_len: int, heads: int,
                         head_dim: int = HEAD_DIM) -> int:
    return int(load_library().vsa_fwd_proxy_workspace_size(batch, seq_len, prefix_len, heads,
                                                           head_dim))


def vsa_fwd(q, k, v, topk_idx, vbs, sm_scale=None, out=None, workspace=None, shared_sweep=False):
    """Fine block-sparse attention forward (C ABI vsa_fwd) on q's device and current stream.

    q, k, v: bf16 [B, S, H, 128]; topk_idx: int32 [B, H, S/64, topk]; vbs: int32 [S/64].
    shared_sweep: the timing-dependent tile order (vsa_fwd_ex, VSA_FLAG_SHARED_SWEEP).
    Returns out (bf16 [B, S, H, 128]).
    """
    lib = load_library()
    dev = q.device
    B, S, H, D = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, dev, (B, S, H, D))
    _need(vbs, "vbs", torch.int32, dev, (S // BLOCK,))
    _need(topk_idx, "topk_idx", torch.int32, dev)
    if topk_idx.dim() != 4 or tuple(topk_idx.shape[:3]) != (B, H, S // BLOCK):
        raise ValueError(f"topk_idx has shape {tuple(topk_idx.shape)}, expected (B, H, S/64, topk)")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, dev, (B, S, H, D))
    nbytes = fwd_workspace_size(B, S, H, D)
    if workspace is None:
        workspace = _workspace(dev, max(nbytes, 1))
    if shared_sweep:
        st = lib.vsa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(topk_idx), _ptr(vbs), _ptr(out), B, S, H,
                            D, topk_idx.shape[3], _default_scale(sm_scale), FLAG_SHARED_SWEEP,
                            _ptr(workspace), workspace.numel(), _stream(dev))
        _check("vsa_fwd_ex", st)
        return out
    st = lib.vsa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(topk_idx), _ptr(vbs), _ptr(out), B, S, H, D,
                     topk_idx.shape[3], _default_scale(sm_scale), _ptr(workspace),
                     workspace.numel(), _stream(dev))
    _check("vsa_fwd", st)
    return out


def vsa_fwd_noalloc(q, k, v, topk_idx, vbs, out, sm_scale=None):
    """vsa_fwd through the C ABI's allocation-free entry point (vsa_fwd_noalloc).

    `out` (bf16 [B, S, H, 128]) must be given: the call allocates nothing.
    """
    lib = load_library()
    dev = q.device
    B, S, H, D = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _need(t, name, torch.bfloat16, dev, (B, S, H, D))
    _need(vbs, "vbs", torch.int32, dev, (S // BLOCK,))
    _need(topk_idx, "topk_idx", torch.int32, dev)
    if topk_idx.dim() != 4 or tuple(topk_idx.shape[:3]) != (B, H, S // BLOCK):
        raise ValueError(f"topk_idx has shape {tuple(topk_idx.shape)}, expected (B, H, S/64, topk)")
    st = lib.vsa_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(topk_idx), _ptr(vbs), _ptr(out), B, S,
                             H, D, topk_idx.shape[3], _default_scale(sm_scale), _stream(dev))
    _check("vsa_fwd_noalloc", st)
    return out


def vsa_pack_values(v, vbs, workspace):
    """First stage of vsa_fwd: packed V tiles into workspace (uint8 device tensor)."""
    lib = load_library()
    dev = v.device
    B, S, H, D = v.shape
    _need(v, "v", torch.bfloat16, dev)
    _need(vbs, "vbs", torch.int32, dev, (S // BLOCK,))
    st = lib.vsa_pack_values(_ptr(v), _ptr(vbs), B, S, H, D, _ptr(workspace), workspace.numel(),
                             _stream(dev))
    _check("vsa_pack_values", st)


def vsa_fwd_prepacked(q, k, topk_idx, vbs, workspace, sm_scale=None, out=None, shared_sweep=False):
    """Second stage of vsa_fwd: attention over a workspace filled by vsa_pack_values
    (vsa_fwd_prepacked_ex with VSA_FLAG_SHARED_SWEEP when shared_sweep)."""
    lib = load_library()
    dev = q.device
    B, S, H, D = q.shape
    _need(q, "q", torch.bfloat16, dev)
    _need(k, "k", torch.bfloat16, dev, (B, S, H, D))
    _need(vbs, "vbs", torch.int32, dev, (S // BLOCK,))
    _need(topk_idx, "topk_idx", torch.int32, dev)
    if out is None:
        out = torch.empty_like(q)
    if shared_sweep:
        st = lib.vsa_fwd_prepacked_ex(_ptr(q), _ptr(k), _ptr(topk_idx), _ptr(vbs), _ptr(out), B, S,
                                      H, D, topk_idx.shape[3], _default_scale(sm_scale),
                                      FLAG_SHARED_SWEEP, _ptr(workspace), workspace.numel(),
                                      _stream(dev))
        _check("vsa_fwd_prepacked_ex", st)
        return out
    st = lib.vsa_fwd_prepacked(_ptr(q), _ptr(k), _ptr(topk_idx), _ptr(vbs), _ptr(out), B, S, H,
                               D, topk_idx.shape[3], _default_scale(sm_scale), _ptr(workspace),
                               workspace.numel(), _stream(dev))
    _check("vsa_fwd_prepacked", st)
    return out


def vsa_preprocess(k, v, vbs, kmean=None, vsum=None):
    """Block summaries (C ABI vsa_preprocess): returns (kmean, vsum), bf16 [B, S/64, H, 128]."""
    lib = load_library()
    dev = k.device
    B, S, H, D = k.shape
    _need(k, "k", torch.bfloat16, dev)
    _need(v, "v", torch.bfloat16, dev, (B, S, H, D))
    _need(vbs, "vbs", torch.int32, dev, (S // BLOCK,))
    shape = (B, S // BLOCK, H, D)
    if kmean is None:
        kmean = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    if vsum is None:
        vsum = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    _need(kmean, "kmean", torch.bfloat16, dev, shape)
    _need(vsum, "vsum", torch.bfloat16, dev, shape)
    st = lib.vsa_preprocess(_ptr(k), _ptr(v), _ptr(vbs), _ptr(kmean), _ptr(vsum), B, S, H, D,
                            _stream(dev))
    _check("vsa_preprocess", st)
    return kmean, vsum


def vsa_kc_stats(kmean, vbs, first_block: int, block_count: int, mean=None, var=None):
    """Mean and population variance of the block key means (C ABI vsa_kc_stats).

    kmean: bf16 [B, nblk, H, 128]; statistics over blocks [first_block,
    first_block + block_count) with vbs > 0.  Returns (mean, var), float32 [B, H, 128].
    """
    lib = load_library()
    dev = kmean.device
    B, nb, H, D = kmean.shape
    _need(kmean, "kmean", torch.bfloat16, dev)
    _need(vbs, "vbs", torch.int32, dev, (nb,))
    if mean is None:
        mean = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    if var is None:
        var = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    _need(mean, "kc_mean", torch.float32, dev, (B, H, D))
    _need(var, "kc_var_diag", torch.float32, dev, (B, H, D))
    _check("vsa_kc_stats", lib.vsa_kc_stats(_ptr(kmean), _ptr(vbs), _ptr(mean), _ptr(var), B, nb, H,
                                            D, int(first_block), int(block_count), _stream(dev)))
    return mean, var


def vsa_fwd_proxy(q, k, v, sel_idx, vbs, kmean, vsum, prefix_len, sm_scale=None, out=None,
                  workspace=None):
    """Packed [prefix | video] proxy-compensated forward (C ABI vsa_fwd_proxy)."""
    lib = load_library()
    dev = q.device
    B, S, H, D = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, dev, (B, S, H, D))
    nblk = S // BLOCK
    _need(vbs, "vbs", torch.int32, dev, (nblk,))
    _need(kmean, "kmean", torch.bfloat16, dev, (B, nblk, H, D))
    _need(vsum, "vsum", torch.bfloat16, dev, (B, nblk, H, D))
    _need(sel_idx, "sel_idx", torch.int32, dev)
    nv = (S - prefix_len) // BLOCK
    if sel_idx.dim() != 4 or tuple(sel_idx.shape[:3]) != (B, H, nv):
        raise ValueError(f"sel_idx has shape {tuple(sel_idx.shape)}, expected (B, H, Nv, max_sel)")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, dev, (B, S, H, D))
    nbytes = proxy_workspace_size(B, S, prefix_len, H, D)
    if workspace is None:
        workspace = _workspace(dev, max(nbytes, 1))
    st = lib.vsa_fwd_proxy(_ptr(q), _ptr(k), _ptr(v), _ptr(sel_idx), _ptr(vbs), _ptr(kmean),
                           _ptr(vsum), _ptr(out), B, S, prefix_len, H, D, sel_idx.shape[3],
                           _default_scale(sm_scale), _ptr(workspace), workspace.numel(),
                           _stream(dev))
    _check("vsa_fwd_proxy", st)
    return out


def cube_vbs(T: int, Hh: int, W: int):
    """Valid tokens per cube of a T x Hh x W grid (C ABI vsa_cube_vbs), numpy int32."""
    import numpy as np
    lib = load_library()
    n = int(lib.vsa_cube_count(T, Hh, W))
    if n == 0:
        raise ValueError(f"grid {T}x{Hh}x{W} has no valid cube layout")
    out = np.empty(n, dtype=np.int32)
    _check("vsa_cube_vbs", lib.vsa_cube_vbs(T, Hh, W, out.ctypes.data, n))
    return out


def vsa_tile(x, grid, out=None):
    """Natural [B, T*Hh*W, H, D] rows -> cube-major [B, 64*cubes, H, D] (C ABI vsa_tile)."""
    lib = load_library()
    T, Hh, W = grid
    B, N, H, D = x.shape
    if N != T * Hh * W:
        raise ValueError(f"x has {N} rows, grid {T}x{Hh}x{W} has {T * Hh * W}")
    cubes = int(lib.vsa_cube_count(T, Hh, W))
    if out is None:
        out = torch.empty((B, BLOCK * cubes, H, D), dtype=x.dtype, device=x.device)
    _need(x, "x", x.dtype, x.device)
    _need(out, "out", x.dtype, x.device, (B, BLOCK * cubes, H, D))
    if x.element_size() != 2:
        raise ValueError("vsa_tile moves 16-bit elements")
    _check("vsa_tile", lib.vsa_tile(_ptr(x), _ptr(out), B, T, Hh, W, H, D, _stream(x.device)))
    return out


def vsa_untile(xt, grid, out=None):
    """Cube-major [B, 64*cubes, H, D] rows -> natural [B, T*Hh*W, H, D] (C ABI vsa_untile)."""
    lib = load_library()
    T, Hh, W = grid
    B, S, H, D = xt.shape
    cubes = int(lib.vsa_cube_count(T, Hh, W))
    if S != BLOCK * cubes:
        raise ValueError(f"x_tiled has {S} rows, grid {T}x{Hh}x{W} needs {BLOCK * cubes}")
    if out is None:
        out = torch.empty((B, T * Hh * W, H, D), dtype=xt.dtype, device=xt.device)
    _need(xt, "x_tiled", xt.dtype, xt.device)
    _need(out, "out", xt.dtype, xt.device, (B, T * Hh * W, H, D))
    if xt.element_size() != 2:
        raise ValueError("vsa_untile moves 16-bit elements")
    _check("vsa_untile", lib.vsa_untile(_ptr(xt), _ptr(out), B, T, Hh, W, H, D, _stream(xt.device)))
    return out


def vsa_fwd_lse(q, k, v, topk_idx, vbs, sm_scale=None, out=None, lse=None, workspace=None):
    """Forward plus row log-sum-exp (C ABI vsa_fwd_lse): returns (out, lse [B, H, S] float32)."""
    lib = load_library()
    dev = q.device
    B, S, H, D = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, dev, (B, S, H, D))
    _need(vbs, "vbs", torch.int32, dev, (S // BLOCK,))
    _need(topk_idx, "topk_idx", torch.int32, dev)
    if topk_idx.dim() != 4 or tuple(topk_idx.shape[:3]) != (B, H, S // BLOCK):
        raise ValueError(f"topk_idx has shape {tuple(topk_idx.shape)}, expected (B, H, S/64, topk)")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    _need(out, "out", torch.bfloat16, dev, (B, S, H, D))
    _need(lse, "lse", torch.float32, dev, (B, H, S))
    nbytes = fwd_workspace_size(B, S, H, D)
    if workspace is None:
        workspace = _workspace(dev, max(nbytes, 1))
    st = lib.vsa_fwd_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(topk_idx), _ptr(vbs), _ptr(out), _ptr(lse),
                         B, S, H, D, topk_idx.shape[3], _default_scale(sm_scale), _ptr(workspace),
                         workspace.numel(), _stream(dev))
    _check("vsa_fwd_lse", st)
    return out, lse


def vsa_merge(o1, lse1, o2, lse2, out=None, lse_out=None):
    """Combine two partial results over disjoint key sets (C ABI vsa_merge)."""
    lib = load_library()
    dev = o1.device
    B, S, H, D = o1.shape
    _need(o1, "o1", torch.bfloat16, dev)
    _need(o2, "o2", torch.bfloat16, dev, (B, S, H, D))
    _need(lse1, "lse1", torch.float32, dev, (B, H, S))
    _need(lse2, "lse2", torch.float32, dev, (B, H, S))
    if out is None:
        out = torch.empty_like(o1)
    if lse_out is None:
        lse_out = torch.empty_like(lse1)
    _need(out, "out", torch.bfloat16, dev, (B, S, H, D))
    _need(lse_out, "lse_out", torch.float32, dev, (B, H, S))
    st = lib.vsa_merge(_ptr(o1), _ptr(lse1), _ptr(o2), _ptr(lse2), _ptr(out), _ptr(lse_out),
                       B, S, H, D, _stream(dev))
    _check("vsa_merge", st)
    return out, lse_out


def _proxy_common(q, k, v, vbs, kmean, vsum, out):
    dev = q.device
    B, S, H, D = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, dev, (B, S, H, D))
    nblk = S // BLOCK
    _need(vbs, "vbs", torch.int32, dev, (nblk,))
    _need(kmean, "kmean", torch.bfloat16, dev, (B, nblk, H, D))
    _need(vsum, "vsum", torch.bfloat16, dev, (B, nblk, H, D))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, dev, (B, S, H, D))
    return dev, B, S, H, D, out


def vsa_fwd_proxy_bitmask(q, k, v, sel_mask, vbs, kmean, vsum, prefix_len, expected_sel,
                          sm_scale=None, out=None, workspace=None):
    """Proxy forward with a bitmask selection (C ABI vsa_fwd_proxy_bitmask).

    sel_mask: int32 or uint32-valued tensor [B, H, Nv, ceil(Nv/32)] (int32 storage)."""
    lib = load_library()
    dev, B, S, H, D, out = _proxy_common(q, k, v, vbs, kmean, vsum, out)
    nv = (S - prefix_len) // BLOCK
    _need(sel_mask, "sel_mask", torch.int32, dev, (B, H, nv, (nv + 31) // 32))
    nbytes = proxy_workspace_size(B, S, prefix_len, H, D)
    if workspace is None:
        workspace = _workspace(dev, max(nbytes, 1))
    st = lib.vsa_fwd_proxy_bitmask(_ptr(q), _ptr(k), _ptr(v), _ptr(sel_mask), _ptr(vbs), _ptr(kmean),
                                   _ptr(vsum), _ptr(out), B, S, prefix_len, H, D, int(expected_sel),
                                   _default_scale(sm_scale), _ptr(workspace), workspace.numel(),
                                   _stream(dev))
    _check("vsa_fwd_proxy_bitmask", st)
    return out


def vsa_fwd_proxy_bsr(q, k, v, sel_indptr, sel_indices, vbs, kmean, vsum, prefix_len, expected_sel,
                      sm_scale=None, out=None, workspace=None):
    """Proxy forward with a BSR selection (C ABI vsa_fwd_proxy_bsr)."""
    lib = load_library()
    dev, B, S, H, D, out = _proxy_common(q, k, v, vbs, kmean, vsum, out)
    nv = (S - prefix_len) // BLOCK
    _need(sel_indptr, "sel_indptr", torch.int32, dev, (B * H * nv + 1,))
    _need(sel_indices, "sel_indices", torch.int32, dev)
    nbytes = proxy_workspace_size(B, S, prefix_len, H, D)
    if workspace is None:
        workspace = _workspace(dev, max(nbytes, 1))
    st = lib.vsa_fwd_proxy_bsr(_ptr(q), _ptr(k), _ptr(v), _ptr(sel_indptr), _ptr(sel_indices),
                               int(sel_indices.numel()), _ptr(vbs), _ptr(kmean), _ptr(vsum), _ptr(out),
                               B, S, prefix_len, H, D, int(expected_sel), _default_scale(sm_scale),
                               _ptr(workspace), workspace.numel(), _stream(dev))
    _check("vsa_fwd_proxy_bsr", st)
    return out


def route_workspace_size(batch: int, num_blocks: int, heads: int) -> int:
    """Bytes of the fp64 score workspace vsa_route_topk needs (C ABI vsa_route_workspace_size)."""
    return int(load_library().vsa_route_workspace_size(batch, num_blocks, heads))


def vsa_route_topk(qmean, kmean, vbs, topk: int, out=None, workspace=None):
    """Top-k key blocks per query block by block-mean scores (C ABI vsa_route_topk).

    `workspace` (uint8, on the device) may be passed to reuse one allocation
    across calls; it is allocated here otherwise.
    """
    lib = load_library()
    dev = qmean.device
    B, nb, H, D = qmean.shape
    _need(qmean, "qmean", torch.bfloat16, dev)
    _need(kmean, "kmean", torch.bfloat16, dev, (B, nb, H, D))
    _need(vbs, "vbs", torch.int32, dev, (nb,))
    if out is None:
        out = torch.empty((B, H, nb, topk), dtype=torch.int32, device=dev)
    _need(out, "topk_idx", torch.int32, dev, (B, H, nb, topk))
    nbytes = route_workspace_size(B, nb, H)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    _check("vsa_route_topk", lib.vsa_route_topk(_ptr(qmean), _ptr(kmean), _ptr(vbs), _ptr(out), B, nb, H,
                                                D, topk, _ptr(workspace), workspace.numel(),
                                                _stream(dev)))
    return out
