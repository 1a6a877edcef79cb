"""Shared helpers for the GPU parity tests: acceptance rules and lazy row
gathers that let the CPU oracle read only the K/V rows it needs."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from oracle import clsa_oracle as O

# Acceptance rules (all stated with the tests that use them):
#  * top-k sets: equal counts; positions that differ must have oracle scores
#    within TOPK_REL * |s_(c)| of the oracle's c-th largest score s_(c)
#    (fp32 accumulation on the GPU vs exact fp64 scores in the oracle);
#  * threshold sets: identical (inputs keep every score >= 1e-4 from tau);
#  * attention: max |out - oracle| <= 2e-2 for bf16 K/V, <= 1e-4 for fp32.
TOPK_REL = 1e-5
ATOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def check_list_shape(idx_row: np.ndarray, count: int, cap: int, n_vis: int):
    """Ascending valid positions first, then -1 padding."""
    n = min(count, cap)
    head = idx_row[:n]
    assert np.all(head >= 0) and np.all(head < n_vis), "index out of the visible range"
    assert np.all(np.diff(head) > 0), "indices not strictly ascending"
    assert np.all(idx_row[n:] == -1), "padding is not -1"


def check_topk_row(g_idx: np.ndarray, g_cnt: int, o_idx: np.ndarray, o_cnt: int,
                   scores: np.ndarray, cap: int) -> int:
    """Returns the number of boundary-pair differences (0 when identical)."""
    assert g_cnt == o_cnt, (g_cnt, o_cnt)
    check_list_shape(g_idx, g_cnt, cap, scores.shape[0])
    gs = set(g_idx[:g_cnt].tolist())
    os_ = set(o_idx[:o_cnt].tolist())
    diff = gs ^ os_
    if diff:
        sc = np.sort(scores)[::-1][o_cnt - 1]
        for j in diff:
            assert abs(scores[j] - sc) <= TOPK_REL * abs(sc), (j, scores[j], sc)
    return len(diff)


class _Rows:
    """K/V rows of one (layer, sequence), gathered on demand as float64
    (widened exactly: bf16 -> fp32 on the device, fp32 -> fp64 on the host)."""

    def __init__(self, t: torch.Tensor):
        self.t = t

    def __getitem__(self, sel):
        s = torch.as_tensor(np.asarray(sel, dtype=np.int64), device=self.t.device)
        return self.t[s].float().cpu().numpy().astype(np.float64)


class _Layer:
    def __init__(self, t: torch.Tensor):  # [B, n_cap, Hkv, D]
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, b):
        return _Rows(self.t[b])


def lazy_layers(cache: torch.Tensor):
    """[L, B, n_cap, Hkv, D] device tensor -> list of lazily gathered layers."""
    return [_Layer(cache[l]) for l in range(cache.shape[0])]


class _QLayer:
    """Queries of one layer [B, M, Hq, D], one (b, m) row fetched on demand."""

    def __init__(self, t: torch.Tensor):
        self.t = t
        self.shape = tuple(t.shape)
        self._rows = {}

    def __getitem__(self, key):
        b, m, h = key
        if (b, m) not in self._rows:
            self._rows[(b, m)] = f64(self.t[b, m])
        return self._rows[(b, m)][h]


def lazy_queries(q: torch.Tensor):
    """[L, B, M, Hq, D] device tensor -> list of lazily read query layers."""
    return [_QLayer(q[l]) for l in range(q.shape[0])]


def host_threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def check_topk_rows(g_idx: torch.Tensor, g_counts: torch.Tensor, q_idx: torch.Tensor,
                    K_idx: torch.Tensor, n_vis, k: int, cap: int, rows) -> int:
    """Every listed (b, m) row of the GPU's routing against the oracle's exact
    top-k (check_topk_row), rows spread over host threads (NumPy's matrix
    product and sort run without the interpreter lock).  n_vis(b, m) gives
    the row's visible keys.  Returns the total of boundary-pair differences."""
    gi, gc = g_idx.cpu().numpy(), g_counts.cpu().numpy()
    q_np = f64(q_idx)
    seqs = sorted({b for b, _ in rows})
    K_np = {b: f64(K_idx[b]) for b in seqs}

    def one(bm):
        b, m = bm
        nv = n_vis(b, m)
        s = O.route_scores(q_np[b, m], K_np[b], nv)
        sel = O.topk_select(s, k)
        o_idx = np.full(cap, -1, dtype=np.int64)
        o_idx[: len(sel)] = sel
        return check_topk_row(gi[b, m], int(gc[b, m]), o_idx, len(sel), s, cap)

    with ThreadPoolExecutor(host_threads()) as ex:
        return sum(ex.map(one, list(rows)))


def attn_vs_oracle(q, Kc, Vc, g_idx, g_counts, out, rows, layers, cap, atol=None):
    """The GPU's attention output against the oracle's attention over the
    GPU's own index lists, element by element, for every listed (b, m) row
    in every listed layer: a check that holds whatever routing chose, so it
    always runs.  q [L, B, M, Hq, D], Kc/Vc [L, B, n_cap, Hkv, D] and out
    [L, B, M, Hq, D] are device tensors.  Returns (max error, pairs compared)."""
    rows, layers = list(rows), list(layers)
    assert rows and layers, "nothing to compare"
    gi, gc = g_idx.cpu().numpy(), g_counts.cpu().numpy()
    o_out, _ = O.sparse_attn(lazy_queries(q), lazy_layers(Kc), lazy_layers(Vc), gi, gc, cap,
                             rows=rows, layers=layers)
    tol = ATOL[q.dtype] if atol is None else atol
    err, n = 0.0, 0
    for l in layers:
        for b, m in rows:
            e = float(np.max(np.abs(f64(out[l, b, m]) - o_out[l, b, m])))
            assert e <= tol, (l, b, m, e)
            err = max(err, e)
            n += 1
    assert n == len(rows) * len(layers) >= 1
    return err, n
