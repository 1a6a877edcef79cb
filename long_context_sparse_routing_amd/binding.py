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
           -3: "unsupported dtype", -4: "HIP launch failure",
           -5: "shapes exceed the static scratch array"}


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
    lib.clsa_route_static.restype = i32
    lib.clsa_route_static.argtypes = [vp, vp, i32, i32, i32, i64, vp, i64, i32, i32, vp, vp, i32,
                                      vp]
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
    lib.clsa_louver_index_bytes.restype = sz
    lib.clsa_louver_index_bytes.argtypes = [i32, i32, i64, i32, i32]
    lib.clsa_louver_build_workspace_size.restype = sz
    lib.clsa_louver_build_workspace_size.argtypes = [i32, i32, i64, i32, i32]
    lib.clsa_louver_build.restype = i32
    lib.clsa_louver_build.argtypes = [vp, i32, i32, i64, i32, i32, i32, i64, i32, vp, vp, sz, vp,
                                      sz, vp]
    lib.clsa_louver_query_workspace_size.restype = sz
    lib.clsa_louver_query_workspace_size.argtypes = [i32, i32, i64, i32, i32, i64, i32, vp]
    lib.clsa_louver_query.restype = i32
    lib.clsa_louver_query.argtypes = [vp, vp, i32, i32, i64, vp, vp, i32, i32, i32, i64, i32, vp,
                                      vp, i32, vp, vp, i32, vp, vp, sz, vp]
    lib.clsa_route_aggregated_workspace_size.restype = sz
    lib.clsa_route_aggregated_workspace_size.argtypes = [i32, i32, i32, i32, i64, i32, i32, i32]
    lib.clsa_route_aggregated.restype = i32
    lib.clsa_route_aggregated.argtypes = [i32, vp, vp, i32, i32, i32, i64, vp, i64, i32, i32, vp,
                                          vp, i32, vp, sz, vp]
    lib.clsa_csa_build_workspace_size.restype = sz
    lib.clsa_csa_build_workspace_size.argtypes = [i32, i32, i32, i64, i32, i32]
    lib.clsa_csa_build.restype = i32
    lib.clsa_csa_build.argtypes = [vp, vp, i32, i32, i32, i64, vp, i32, i32, i32, i32, vp, vp, vp,
                                   sz, vp]
    lib.clsa_csa_route_workspace_size.restype = sz
    lib.clsa_csa_route_workspace_size.argtypes = [i32, i32, i64, i32, i32, i32]
    lib.clsa_csa_route.restype = i32
    lib.clsa_csa_route.argtypes = [vp, vp, i32, i32, i64, vp, vp, vp, i32, i32, i64, i32, i32, i32,
                                   vp, vp, i32, vp, sz, vp]
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


def _need(cond: bool, msg: str, exc=ValueError):
    if not cond:
        raise exc(msg)


def _check_shape(t: torch.Tensor, shape: tuple, name: str):
    _need(tuple(t.shape) == tuple(shape), f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_i32(t: torch.Tensor | None, shape: tuple, name: str):
    """int32 tensor of exactly `shape` (the library reads and writes it as such)."""
    if t is None:
        return
    _need(t.dtype == torch.int32, f"{name} must be int32, got {t.dtype}", TypeError)
    _check_shape(t, shape, name)


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _workspace(nbytes: int, device, ws: torch.Tensor | None) -> torch.Tensor:
    if ws is not None:
        _check_dev(ws)
        if _nbytes(ws) < nbytes:
            raise ValueError(f"workspace has {_nbytes(ws)} bytes, "
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
    B, M, d, n_cap = _route_shapes(q_idx, K_idx)
    cap = k if cap is None else cap
    dev = q_idx.device
    if idx is None:
        idx = torch.empty((B, M, cap), dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty((B, M), dtype=torch.int32, device=dev)
    _check_route_io(B, M, cap, n_ctx, idx, counts)
    _check_dev(q_idx, K_idx, n_ctx, idx, counts)
    dt = _dt(q_idx)
    need = lib.clsa_route_workspace_size(B, M, d, n_cap, k, cap, dt)
    ws = _workspace(need, dev, ws)
    args = (_ptr(q_idx), _ptr(K_idx), B, M, d, n_cap, _ptr(n_ctx), q_pos0, k, dt, _ptr(idx),
            _ptr(counts), cap, _ptr(ws), _nbytes(ws), _stream(stream))
    return Prepared("clsa_route", lib.clsa_route, args, (idx, counts),
                    (q_idx, K_idx, n_ctx, idx, counts, ws))


def _route_shapes(q_idx: torch.Tensor, K_idx: torch.Tensor):
    """(B, M, d, n_cap) of a routing call; q_idx [B, M, d] and K_idx
    [B, n_cap, d] must agree in B, d and dtype."""
    _need(q_idx.dim() == 3, f"q_idx must be [B, M, d], got shape {tuple(q_idx.shape)}")
    _need(K_idx.dim() == 3, f"K_idx must be [B, n_cap, d], got shape {tuple(K_idx.shape)}")
    B, M, d = q_idx.shape
    _need(K_idx.shape[0] == B and K_idx.shape[2] == d,
          f"K_idx {tuple(K_idx.shape)} does not match q_idx {tuple(q_idx.shape)}")
    _need(K_idx.dtype == q_idx.dtype, f"K_idx is {K_idx.dtype}, q_idx {q_idx.dtype}", TypeError)
    _dt(q_idx)
    return B, M, d, K_idx.shape[1]


def _check_route_io(B, M, cap, n_ctx, idx, counts):
    _check_i32(n_ctx, (B,), "n_ctx")
    _check_i32(idx, (B, M, cap), "idx")
    _check_i32(counts, (B, M), "counts")


def route(q_idx: torch.Tensor, K_idx: torch.Tensor, k: int, n_ctx: torch.Tensor | None = None,
          q_pos0: int = -1, cap: int | None = None, idx: torch.Tensor | None = None,
          counts: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None):
    """clsa_route: q_idx [B, M, d], K_idx [B, n_cap, d] -> (idx [B, M, cap], counts [B, M])."""
    return prepare_route(q_idx, K_idx, k, n_ctx, q_pos0, cap, idx, counts, ws, stream)()


def prepare_route_static(q_idx: torch.Tensor, K_idx: torch.Tensor, k: int,
                         n_ctx: torch.Tensor | None = None, q_pos0: int = -1,
                         cap: int | None = None, idx: torch.Tensor | None = None,
                         counts: torch.Tensor | None = None, stream=None) -> Prepared:
    """clsa_route_static, marshalled: the routing of clsa_route on the
    library's fixed device scratch array, so the call itself allocates
    nothing (pass idx and counts to keep the binding from allocating them).
    Calls on one GPU share that array: order them on one stream."""
    lib = load_library()
    B, M, d, n_cap = _route_shapes(q_idx, K_idx)
    cap = k if cap is None else cap
    dev = q_idx.device
    if idx is None:
        idx = torch.empty((B, M, cap), dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty((B, M), dtype=torch.int32, device=dev)
    _check_route_io(B, M, cap, n_ctx, idx, counts)
    _check_dev(q_idx, K_idx, n_ctx, idx, counts)
    dt = _dt(q_idx)
    args = (_ptr(q_idx), _ptr(K_idx), B, M, d, n_cap, _ptr(n_ctx), q_pos0, k, dt, _ptr(idx),
            _ptr(counts), cap, _stream(stream))
    return Prepared("clsa_route_static", lib.clsa_route_static, args, (idx, counts),
                    (q_idx, K_idx, n_ctx, idx, counts))


def route_static(q_idx: torch.Tensor, K_idx: torch.Tensor, k: int,
                 n_ctx: torch.Tensor | None = None, q_pos0: int = -1, cap: int | None = None,
                 idx: torch.Tensor | None = None, counts: torch.Tensor | None = None,
                 stream=None):
    """clsa_route_static: as route(), with no workspace argument."""
    return prepare_route_static(q_idx, K_idx, k, n_ctx, q_pos0, cap, idx, counts, stream)()


def prepare_route_threshold(q_idx: torch.Tensor, K_idx: torch.Tensor, tau: torch.Tensor,
                            cap: int, n_ctx: torch.Tensor | None = None, q_pos0: int = -1,
                            idx: torch.Tensor | None = None, counts: torch.Tensor | None = None,
                            ws: torch.Tensor | None = None, stream=None) -> Prepared:
    """clsa_route_threshold, marshalled: calling the result returns (idx, counts)."""
    lib = load_library()
    B, M, d, n_cap = _route_shapes(q_idx, K_idx)
    dev = q_idx.device
    if idx is None:
        idx = torch.empty((B, M, cap), dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty((B, M), dtype=torch.int32, device=dev)
    if tau.dtype != torch.float32:
        raise TypeError("tau must be float32")
    _check_shape(tau, (B, M), "tau")
    _check_route_io(B, M, cap, n_ctx, idx, counts)
    _check_dev(q_idx, K_idx, tau, n_ctx, idx, counts)
    dt = _dt(q_idx)
    need = lib.clsa_route_threshold_workspace_size(B, M, d, n_cap, cap, dt)
    ws = _workspace(need, dev, ws)
    args = (_ptr(q_idx), _ptr(K_idx), B, M, d, n_cap, _ptr(n_ctx), q_pos0, _ptr(tau), dt,
            _ptr(idx), _ptr(counts), cap, _ptr(ws), _nbytes(ws),
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
    _need(ql[0].dim() == 4, f"q[l] must be [B, M, Hq, D], got shape {tuple(ql[0].shape)}")
    _need(Kl[0].dim() == 4, f"K[l] must be [B, n_cap, Hkv, D], got shape {tuple(Kl[0].shape)}")
    B, M, Hq, D = ql[0].shape
    _, n_cap, Hkv, _ = Kl[0].shape
    _need(idx.dim() == 3, f"idx must be [B, M, cap], got shape {tuple(idx.shape)}")
    cap = idx.shape[-1]
    dev = ql[0].device
    dt = _dt(ql[0])
    for t in ql + Kl + Vl:
        if t.dtype != ql[0].dtype:
            raise TypeError("q, K and V must share one dtype")
    for l in range(L):
        _check_shape(ql[l], (B, M, Hq, D), f"q[{l}]")
        _check_shape(Kl[l], (B, n_cap, Hkv, D), f"K[{l}]")
        _check_shape(Vl[l], (B, n_cap, Hkv, D), f"V[{l}]")
    _check_i32(idx, (B, M, cap), "idx")
    _check_i32(counts, (B, M), "counts")
    if out is None:
        out = torch.empty((L, B, M, Hq, D), dtype=ql[0].dtype, device=dev)
    outl = _layers(out)
    _need(len(outl) == L, f"out has {len(outl)} layers, expected {L}")
    for l in range(L):
        _check_shape(outl[l], (B, M, Hq, D), f"out[{l}]")
        _need(outl[l].dtype == ql[0].dtype, f"out[{l}] is {outl[l].dtype}, q {ql[0].dtype}",
              TypeError)
    _check_dev(*ql, *Kl, *Vl, idx, counts, *outl)
    lse = torch.empty((L, B, M, Hq), dtype=torch.float32, device=dev) if want_lse else None
    need = lib.clsa_sparse_attn_workspace_size(L, B, M, Hq, Hkv, D, cap, dt)
    ws = _workspace(need, dev, ws)
    arr = ctypes.c_void_p * L
    qa = arr(*[t.data_ptr() for t in ql])
    ka = arr(*[t.data_ptr() for t in Kl])
    va = arr(*[t.data_ptr() for t in Vl])
    oa = arr(*[t.data_ptr() for t in outl])
    args = (L, B, M, Hq, Hkv, D, qa, ka, va, n_cap, _ptr(idx), _ptr(counts), cap, float(scale),
            dt, oa, _ptr(lse), _ptr(ws), _nbytes(ws), _stream(stream))
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
    _need(L > 0 or dst_idx is not None, "nothing to append")
    _need((src_idx is None) == (dst_idx is None), "src_idx and dst_idx go together")
    _check_i32(pos, (B,), "pos")
    ref = dst_idx if dst_idx is not None else Kd[0]
    n_cap = ref.shape[1]
    d = dst_idx.shape[2] if dst_idx is not None else 0
    Hkv, D = (Kd[0].shape[2], Kd[0].shape[3]) if L else (0, 0)
    if dst_idx is not None:
        _check_shape(dst_idx, (B, n_cap, d), "dst_idx")
        _check_shape(src_idx, (B, d), "src_idx")
    for l in range(L):
        _check_shape(Kd[l], (B, n_cap, Hkv, D), f"K[{l}]")
        _check_shape(Vd[l], (B, n_cap, Hkv, D), f"V[{l}]")
        _check_shape(ks[l], (B, Hkv, D), f"src_k[{l}]")
        _check_shape(vs[l], (B, Hkv, D), f"src_v[{l}]")
    for t in [src_idx, dst_idx, *ks, *vs, *Kd, *Vd]:
        if t is not None and t.dtype != ref.dtype:
            raise TypeError("appended rows and caches must share one dtype")
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


class LouverIndex:
    """A Louver index (clsa_louver_build / clsa_louver_query) over the routing
    keys of B sequences: the device buffer and the host table of segment
    bounds that every call passes.  build(K_idx, end) clusters positions
    [last end, end) into a new segment; query(...) is the threshold
    selection of clsa_route_threshold through the index."""

    def __init__(self, B: int, d: int, n_max: int, S: int = 1, r: int = 64, device="cuda"):
        lib = load_library()
        nbytes = lib.clsa_louver_index_bytes(B, d, n_max, S, r)
        if nbytes == 0:
            raise ValueError(f"unsupported Louver index shape B={B} d={d} n_max={n_max} S={S} r={r}")
        self.B, self.d, self.n_max, self.S, self.r = B, d, n_max, S, r
        # zeroed once, so that two indexes built from the same keys compare
        # equal byte for byte (the build writes every part a query reads)
        self.buf = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        self.bounds: list[int] = [0]

    @property
    def indexed(self) -> int:
        """Positions covered by the index; later ones are the buffer."""
        return self.bounds[-1]

    def _bounds(self, extra=None):
        b = self.bounds + ([extra] if extra is not None else [])
        return (ctypes.c_int64 * len(b))(*b), len(b) - 1

    def build(self, K_idx: torch.Tensor, end: int, ws: torch.Tensor | None = None, stream=None):
        lib = load_library()
        _need(K_idx.dim() == 3 and K_idx.shape[0] == self.B and K_idx.shape[2] == self.d,
              f"K_idx {tuple(K_idx.shape)} does not match the index (B={self.B}, d={self.d})")
        _need(K_idx.dtype == torch.bfloat16, "the Louver index takes bfloat16 keys", TypeError)
        _need(self.indexed < end <= min(self.n_max, K_idx.shape[1]),
              f"segment end {end} must lie in ({self.indexed}, {min(self.n_max, K_idx.shape[1])}]")
        _check_dev(K_idx)
        arr, nseg = self._bounds(end)
        need = lib.clsa_louver_build_workspace_size(self.B, self.d, self.n_max, self.S, self.r)
        ws = _workspace(need, K_idx.device, ws)
        st = lib.clsa_louver_build(_ptr(K_idx), self.B, self.d, K_idx.shape[1], CLSA_BF16, self.S,
                                   self.r, self.n_max, nseg, arr, _ptr(self.buf),
                                   self.buf.numel(), _ptr(ws), _nbytes(ws), _stream(stream))
        if st != 0:
            raise ClsaError("clsa_louver_build", st)
        self.bounds.append(int(end))
        self._keep = ws  # the build runs asynchronously on the stream

    def prepare_query(self, q_idx: torch.Tensor, K_idx: torch.Tensor, tau: torch.Tensor,
                      cap: int, mode: int = 1, n_ctx: torch.Tensor | None = None,
                      idx: torch.Tensor | None = None, counts: torch.Tensor | None = None,
                      checked: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                      stream=None) -> Prepared:
        """clsa_louver_query, marshalled: calling the result returns
        (idx [B, 1, cap], true counts [B, 1], checked [B] or None)."""
        lib = load_library()
        B, M, d, n_cap = _route_shapes(q_idx, K_idx)
        _need(B == self.B and d == self.d and M == 1,
              f"q_idx {tuple(q_idx.shape)} does not match the index (B={self.B}, d={self.d}, M=1)")
        _need(self.indexed > 0, "the index has no segment yet")
        if tau.dtype != torch.float32:
            raise TypeError("tau must be float32")
        _check_shape(tau, (B, 1), "tau")
        dev = q_idx.device
        if idx is None:
            idx = torch.empty((B, 1, cap), dtype=torch.int32, device=dev)
        if counts is None:
            counts = torch.empty((B, 1), dtype=torch.int32, device=dev)
        _check_route_io(B, 1, cap, n_ctx, idx, counts)
        if checked is not None:
            _check_shape(checked, (B,), "checked")
            _need(checked.dtype == torch.int32, "checked must be int32", TypeError)
        _check_dev(q_idx, K_idx, tau, n_ctx, idx, counts, checked)
        arr, nseg = self._bounds()
        need = lib.clsa_louver_query_workspace_size(B, d, n_cap, self.S, self.r, self.n_max, nseg,
                                                    arr)
        ws = _workspace(need, dev, ws)
        args = (_ptr(q_idx), _ptr(K_idx), B, d, n_cap, _ptr(n_ctx), _ptr(tau), _dt(q_idx), self.S,
                self.r, self.n_max, nseg, arr, _ptr(self.buf), mode, _ptr(idx), _ptr(counts), cap,
                _ptr(checked), _ptr(ws), _nbytes(ws), _stream(stream))
        return Prepared("clsa_louver_query", lib.clsa_louver_query, args, (idx, counts, checked),
                        (q_idx, K_idx, tau, n_ctx, idx, counts, checked, ws, arr, self.buf))

    def query(self, q_idx, K_idx, tau, cap, mode=1, n_ctx=None, idx=None, counts=None,
              checked=None, ws=None, stream=None):
        return self.prepare_query(q_idx, K_idx, tau, cap, mode, n_ctx, idx, counts, checked, ws,
                                  stream)()


def prepare_route_aggregated(q_idx, K_idx, k: int, n_ctx: torch.Tensor | None = None,
                             q_pos0: int = -1, cap: int | None = None,
                             idx: torch.Tensor | None = None, counts: torch.Tensor | None = None,
                             ws: torch.Tensor | None = None, stream=None) -> Prepared:
    """clsa_route_aggregated, marshalled.  q_idx: [H, B, M, d] tensor or list
    of H [B, M, d]; K_idx: [H, B, n_cap, d] or list of H [B, n_cap, d].
    Calling the result returns (idx [B, M, cap], counts [B, M])."""
    lib = load_library()
    ql, Kl = _layers(q_idx), _layers(K_idx)
    H = len(ql)
    _need(1 <= H <= MAX_LAYERS and len(Kl) == H, "q_idx and K_idx need the same 1..64 heads")
    B, M, d, n_cap = _route_shapes(ql[0], Kl[0])
    for h in range(H):
        _check_shape(ql[h], (B, M, d), f"q_idx[{h}]")
        _check_shape(Kl[h], (B, n_cap, d), f"K_idx[{h}]")
        _need(ql[h].dtype == ql[0].dtype and Kl[h].dtype == ql[0].dtype,
              "every head shares one dtype", TypeError)
    cap = k if cap is None else cap
    dev = ql[0].device
    if idx is None:
        idx = torch.empty((B, M, cap), dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty((B, M), dtype=torch.int32, device=dev)
    _check_route_io(B, M, cap, n_ctx, idx, counts)
    _check_dev(*ql, *Kl, n_ctx, idx, counts)
    dt = _dt(ql[0])
    ws = _workspace(lib.clsa_route_aggregated_workspace_size(H, B, M, d, n_cap, k, cap, dt), dev,
                    ws)
    arr = ctypes.c_void_p * H
    qa = arr(*[t.data_ptr() for t in ql])
    ka = arr(*[t.data_ptr() for t in Kl])
    args = (H, qa, ka, B, M, d, n_cap, _ptr(n_ctx), q_pos0, k, dt, _ptr(idx), _ptr(counts), cap,
            _ptr(ws), _nbytes(ws), _stream(stream))
    return Prepared("clsa_route_aggregated", lib.clsa_route_aggregated, args, (idx, counts),
                    (ql, Kl, n_ctx, idx, counts, ws, qa, ka))


def route_aggregated(q_idx, K_idx, k: int, **kw):
    return prepare_route_aggregated(q_idx, K_idx, k, **kw)()


def csa_build(q_prefill: torch.Tensor, K_idx: torch.Tensor, C: int, T: int, rounds: int = 10,
              n_ctx: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None):
    """clsa_csa_build: q_prefill [B, M, d], K_idx [B, n_cap, d] (bf16) ->
    (centroids [B, C, d] bf16, table [B, C, T] int32)."""
    lib = load_library()
    B, M, d, n_cap = _route_shapes(q_prefill, K_idx)
    _need(q_prefill.dtype == torch.bfloat16, "the centroid table router takes bfloat16", TypeError)
    _check_i32(n_ctx, (B,), "n_ctx")
    _check_dev(q_prefill, K_idx, n_ctx)
    dev = q_prefill.device
    cent = torch.empty((B, C, d), dtype=torch.bfloat16, device=dev)
    table = torch.empty((B, C, T), dtype=torch.int32, device=dev)
    need = lib.clsa_csa_build_workspace_size(B, M, d, n_cap, C, T)
    _need(need > 0, f"unsupported centroid table shape B={B} M={M} d={d} C={C} T={T}")
    ws = _workspace(need, dev, ws)
    st = lib.clsa_csa_build(_ptr(q_prefill), _ptr(K_idx), B, M, d, n_cap, _ptr(n_ctx), C, rounds,
                            T, CLSA_BF16, _ptr(cent), _ptr(table), _ptr(ws), _nbytes(ws),
                            _stream(stream))
    if st != 0:
        raise ClsaError("clsa_csa_build", st)
    return cent, table


def prepare_csa_route(q_idx: torch.Tensor, K_idx: torch.Tensor, centroids: torch.Tensor,
                      table: torch.Tensor, n_table: int, P: int, k: int,
                      n_ctx: torch.Tensor | None = None, cap: int | None = None,
                      idx: torch.Tensor | None = None, counts: torch.Tensor | None = None,
                      ws: torch.Tensor | None = None, stream=None) -> Prepared:
    """clsa_csa_route, marshalled: q_idx [B, 1, d]; calling the result
    returns (idx [B, 1, cap], counts [B, 1])."""
    lib = load_library()
    B, M, d, n_cap = _route_shapes(q_idx, K_idx)
    _need(M == 1, "the centroid table router takes one query row per sequence")
    _need(centroids.dim() == 3 and table.dim() == 3, "centroids [B, C, d] and table [B, C, T]")
    C, T = centroids.shape[1], table.shape[2]
    _check_shape(centroids, (B, C, d), "centroids")
    _need(centroids.dtype == torch.bfloat16 and q_idx.dtype == torch.bfloat16,
          "the centroid table router takes bfloat16", TypeError)
    _check_i32(table, (B, C, T), "table")
    cap = k if cap is None else cap
    dev = q_idx.device
    if idx is None:
        idx = torch.empty((B, 1, cap), dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty((B, 1), dtype=torch.int32, device=dev)
    _check_route_io(B, 1, cap, n_ctx, idx, counts)
    _check_dev(q_idx, K_idx, centroids, table, n_ctx, idx, counts)
    ws = _workspace(lib.clsa_csa_route_workspace_size(B, d, n_cap, C, T, P), dev, ws)
    args = (_ptr(q_idx), _ptr(K_idx), B, d, n_cap, _ptr(n_ctx), _ptr(centroids), _ptr(table), C, T,
            n_table, P, k, CLSA_BF16, _ptr(idx), _ptr(counts), cap, _ptr(ws), _nbytes(ws),
            _stream(stream))
    return Prepared("clsa_csa_route", lib.clsa_csa_route, args, (idx, counts),
                    (q_idx, K_idx, centroids, table, n_ctx, idx, counts, ws))


def csa_route(q_idx, K_idx, centroids, table, n_table: int, P: int, k: int, **kw):
    return prepare_csa_route(q_idx, K_idx, centroids, table, n_table, P, k, **kw)()
