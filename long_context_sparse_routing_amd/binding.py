"""Thin ctypes binding over libclsa.so (argument marshalling only).

Every step of routing and attention runs in the HIP kernels of libclsa;
PyTorch only provides device memory and the current stream.  If the built
library is missing, every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libclsa.so")

CLSA_F32 = 0
CLSA_BF16 = 1
MAX_LAYERS = 64

_STATUS = {0: "ok", -1: "invalid argument", -2: "workspace too small",
           -3: "unsupported dtype", -4: "HIP launch failure"}


class ClsaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)} (status {status})")
        self.status = status


_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libclsa.so (torch is imported first so that the HIP runtime
    torch already loaded is the one the library binds to)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"libclsa.so not found at {p}; build it with "
            "`python -m long_context_sparse_routing_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(p)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.clsa_version.restype = i32
    lib.clsa_version.argtypes = []
    lib.clsa_status_string.restype = ctypes.c_char_p
    lib.clsa_status_string.argtypes = [i32]
    lib.clsa_route_workspace_size.restype = sz
    lib.clsa_route_workspace_size.argtypes = [i32, i32, i32, i64, i32, i32, i32]
    lib.clsa_route.restype = i32
    lib.clsa_route.argtypes = [vp, vp, i32, i32, i32, i64, vp, i64, i32, i32, vp, vp, i32, vp,
                               sz, vp]
    lib.clsa_route_threshold_workspace_size.restype = sz
    lib.clsa_route_threshold_workspace_size.argtypes = [i32, i32, i32, i64, i32, i32]
    lib.clsa_route_threshold.restype = i32
    lib.clsa_route_threshold.argtypes = [vp, vp, i32, i32, i32, i64, vp, i64, vp, i32, vp, vp,
                                         i32, vp, sz, vp]
    lib.clsa_sparse_attn_workspace_size.restype = sz
    lib.clsa_sparse_attn_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
    lib.clsa_sparse_attn.restype = i32
    lib.clsa_sparse_attn.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, i64, vp, vp, i32,
                                     ctypes.c_float, i32, vp, vp, vp, sz, vp]
    lib.clsa_kv_append.restype = i32
    lib.clsa_kv_append.argtypes = [i32, i32, i32, i32, i32, i64, vp, vp, vp, vp, vp, vp, vp, i32,
                                   vp]
    if path is None:
        _lib = lib
    return lib


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return CLSA_F32
    if t.dtype == torch.bfloat16:
        return CLSA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(None)


def _stream(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check_dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("all tensors must be on the GPU")
            if not t.is_contiguous():
                raise ValueError("all tensors must be contiguous")


def _workspace(nbytes: int, device, ws: torch.Tensor | None) -> torch.Tensor:
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace has {ws.numel() * ws.element_size()} bytes, "
                             f"needs {nbytes}")
        return ws
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


class Prepared:
    """A library call with every argument marshalled in advance (pointers,
    sizes, stream).  Calling it only crosses into libclsa: meant for decode
    loops that repeat the same call on the same buffers."""

    def __init__(self, name: str, fn, args: tuple, result=None, keep=()):
        self.name, self.fn, self.args, self.result = name, fn, args, result
        self._keep = keep  # objects whose memory the pointers refer to

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise ClsaError(self.name, st)
        return self.result


def route_workspace_size(B, M, d, n_cap, k, cap, dtype) -> int:
    return int(load_library().clsa_route_workspace_size(B, M, d, n_cap, k, cap,
                                                         _dt(torch.empty(0, dtype=dtype))))


def route_threshold_workspace_size(B, M, d, n_cap, cap, dtype) -> int:
    return int(load_library().clsa_route_threshold_workspace_size(
        B, M, d, n_cap, cap, _dt(torch.empty(0, dtype=dtype))))


def sparse_attn_workspace_size(L, B, M, Hq, Hkv, D, cap, dtype) -> int:
    return int(load_library().clsa_sparse_attn_workspace_size(
        L, B, M, Hq, Hkv, D, cap, _dt(torch.empty(0, dtype=dtype))))


def prepare_route(q_idx: torch.Tensor, K_idx: torch.Tensor, k: int,
                  n_ctx: torch.Tensor | None = None, q_pos0: int = -1, cap: int | None = None,
                  idx: torch.Tensor | None = None, counts: torch.Tensor | None = None,
                  ws: torch.Tensor | None = None, stream=None) -> Prepared:
    """clsa_route, marshalled: calling the result returns (idx, counts)."""
    lib = load_library()
    B, M, d = q_idx.shape
    n_cap = K_idx.shape[1]
    cap = k if cap is None else cap
    dev = q_idx.device
    if idx is None:
        idx = torch.empty((B, M, cap), dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty((B, M), dtype=torch.int32, device=dev)
    _check_dev(q_idx, K_idx, n_ctx, idx, counts)
    dt = _dt(q_idx)
    need = lib.clsa_route_workspace_size(B, M, d, n_cap, k, cap, dt)
    ws = _workspace(need, dev, ws)
    args = (_ptr(q_idx), _ptr(K_idx), B, M, d, n_cap, _ptr(n_ctx), q_pos0, k, dt, _ptr(idx),
            _ptr(counts), cap, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    return Prepared("clsa_route", lib.clsa_route, args, (idx, counts),
                    (q_idx, K_idx, n_ctx, idx, counts, ws))


def route(q_idx: torch.Tensor, K_idx: torch.Tensor, k: int, n_ctx: torch.Tensor | None = None,
          q_pos0: int = -1, cap: int | None = None, idx: torch.Tensor | None = None,
          counts: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None):
    """clsa_route: q_idx [B, M, d], K_idx [B, n_cap, d] -> (idx [B, M, cap], counts [B, M])."""
    return prepare_route(q_idx, K_idx, k, n_ctx, q_pos0, cap, idx, counts, ws, stream)()


def prepare_route_threshold(q_idx: torch.Tensor, K_idx: torch.Tensor, tau: torch.Tensor,
                            cap: int, n_ctx: torch.Tensor | None = None, q_pos0: int = -1,
                            idx: torch.Tensor | None = None, counts: torch.Tensor | None = None,
                            ws: torch.Tensor | None = None, stream=None) -> Prepared:
    """clsa_route_threshold, marshalled: calling the result returns (idx, counts)."""
    lib = load_library()
    B, M, d = q_idx.shape
    n_cap = K_idx.shape[1]
    dev = q_idx.device
    if idx is None:
        idx = torch.empty((B, M, cap), dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty((B, M), dtype=torch.int32, device=dev)
    if tau.dtype != torch.float32:
        raise TypeError("tau must be float32")
    _check_dev(q_idx, K_idx, tau, n_ctx, idx, counts)
    dt = _dt(q_idx)
    need = lib.clsa_route_threshold_workspace_size(B, M, d, n_cap, cap, dt)
    ws = _workspace(need, dev, ws)
    args = (_ptr(q_idx), _ptr(K_idx), B, M, d, n_cap, _ptr(n_ctx), q_pos0, _ptr(tau), dt,
            _ptr(idx), _ptr(counts), cap, _ptr(ws), ws.numel() * ws.element_size(),
            _stream(stream))
    return Prepared("clsa_route_threshold", lib.clsa_route_threshold, args, (idx, counts),
                    (q_idx, K_idx, tau, n_ctx, idx, counts, ws))


def route_threshold(q_idx: torch.Tensor, K_idx: torch.Tensor, tau: torch.Tensor, cap: int,
                    n_ctx: torch.Tensor | None = None, q_pos0: int = -1,
                    idx: torch.Tensor | None = None, counts: torch.Tensor | None = None,
                    ws: torch.Tensor | None = None, stream=None):
    """clsa_route_threshold: tau [B, M] float32 -> (idx [B, M, cap], true counts [B, M])."""
    return prepare_route_threshold(q_idx, K_idx, tau, cap, n_ctx, q_pos0, idx, counts, ws,
                                   stream)()


def _layers(x) -> list:
    if isinstance(x, torch.Tensor):
        return [x[i] for i in range(x.shape[0])]
    return list(x)


def prepare_sparse_attn(q, K, V, idx: torch.Tensor, counts: torch.Tensor, scale: float = 0.0,
                        out=None, want_lse: bool = False, ws: torch.Tensor | None = None,
                        stream=None) -> Prepared:
    """clsa_sparse_attn, marshalled: calling the result returns (out, lse)."""
    lib = load_library()
    ql, Kl, Vl = _layers(q), _layers(K), _layers(V)
    L = len(ql)
    if not (len(Kl) == len(Vl) == L) or L < 1 or L > MAX_LAYERS:
        raise ValueError("q, K and V need the same number of layers (1..64)")
    B, M, Hq, D = ql[0].shape
    _, n_cap, Hkv, _ = Kl[0].shape
    cap = idx.shape[-1]
    dev = ql[0].device
    dt = _dt(ql[0])
    for t in ql + Kl + Vl:
        if t.dtype != ql[0].dtype:
            raise TypeError("q, K and V must share one dtype")
    _check_dev(*ql, *Kl, *Vl, idx, counts)
    if out is None:
        out = torch.empty((L, B, M, Hq, D), dtype=ql[0].dtype, device=dev)
    outl = _layers(out)
    _check_dev(*outl)
    lse = torch.empty((L, B, M, Hq), dtype=torch.float32, device=dev) if want_lse else None
    need = lib.clsa_sparse_attn_workspace_size(L, B, M, Hq, Hkv, D, cap, dt)
    ws = _workspace(need, dev, ws)
    arr = ctypes.c_void_p * L
    qa = arr(*[t.data_ptr() for t in ql])
    ka = arr(*[t.data_ptr() for t in Kl])
    va = arr(*[t.data_ptr() for t in Vl])
    oa = arr(*[t.data_ptr() for t in outl])
    args = (L, B, M, Hq, Hkv, D, qa, ka, va, n_cap, _ptr(idx), _ptr(counts), cap, float(scale),
            dt, oa, _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    return Prepared("clsa_sparse_attn", lib.clsa_sparse_attn, args, (out, lse),
                    (ql, Kl, Vl, idx, counts, out, lse, ws))


def sparse_attn(q, K, V, idx: torch.Tensor, counts: torch.Tensor, scale: float = 0.0,
                out=None, want_lse: bool = False, ws: torch.Tensor | None = None, stream=None):
    """clsa_sparse_attn over L layers.

    q: [L, B, M, Hq, D] tensor or list of L [B, M, Hq, D]; K, V: [L, B, n_cap,
    Hkv, D] or lists of [B, n_cap, Hkv, D].  Returns (out [L, B, M, Hq, D],
    lse [L, B, M, Hq] or None).
    """
    return prepare_sparse_attn(q, K, V, idx, counts, scale, out, want_lse, ws, stream)()


def prepare_kv_append(pos: torch.Tensor, src_idx=None, dst_idx=None, src_k=None, K=None,
                      src_v=None, V=None, stream=None) -> Prepared:
    """clsa_kv_append, marshalled.  pos [B] int32; src_idx [B, d] ->
    dst_idx [B, n_cap, d]; src_k/src_v [L, B, Hkv, D] (or lists) -> K/V
    [L, B, n_cap, Hkv, D] (or lists)."""
    lib = load_library()
    B = pos.shape[0]
    ks = _layers(src_k) if src_k is not None else []
    vs = _layers(src_v) if src_v is not None else []
    Kd = _layers(K) if K is not None else []
    Vd = _layers(V) if V is not None else []
    L = len(ks)
    if not (len(vs) == len(Kd) == len(Vd) == L):
        raise ValueError("src_k, K, src_v and V need the same number of layers")
    ref = dst_idx if dst_idx is not None else Kd[0]
    n_cap = ref.shape[1]
    d = dst_idx.shape[2] if dst_idx is not None else 0
    Hkv, D = (Kd[0].shape[2], Kd[0].shape[3]) if L else (0, 0)
    _check_dev(pos, src_idx, dst_idx, *ks, *vs, *Kd, *Vd)
    dt = _dt(ref)
    arr = ctypes.c_void_p * max(L, 1)
    mk = lambda ts: arr(*[t.data_ptr() for t in ts]) if ts else None  # noqa: E731
    args = (L, B, Hkv, D, d, n_cap, _ptr(pos), _ptr(src_idx), _ptr(dst_idx), mk(ks), mk(Kd),
            mk(vs), mk(Vd), dt, _stream(stream))
    return Prepared("clsa_kv_append", lib.clsa_kv_append, args, None,
                    (pos, src_idx, dst_idx, ks, vs, Kd, Vd))


def kv_append(pos, src_idx=None, dst_idx=None, src_k=None, K=None, src_v=None, V=None,
              stream=None):
    prepare_kv_append(pos, src_idx, dst_idx, src_k, K, src_v, V, stream)()
