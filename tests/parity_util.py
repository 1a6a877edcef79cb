"""Shared helpers for the GPU parity tests: acceptance rules and lazy row
gathers that let the CPU oracle read only the K/V rows it needs."""
from __future__ import annotations

import numpy as np
import torch

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
    """K/V rows of one (layer, sequence), gathered on demand as float64."""

    def __init__(self, t: torch.Tensor):
        self.t = t

    def __getitem__(self, sel):
        s = torch.as_tensor(np.asarray(sel, dtype=np.int64), device=self.t.device)
        return f64(self.t[s])


class _Layer:
    def __init__(self, t: torch.Tensor):  # [B, n_cap, Hkv, D]
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, b):
        return _Rows(self.t[b])


def lazy_layers(cache: torch.Tensor):
    """[L, B, n_cap, Hkv, D] device tensor -> list of lazily gathered layers."""
    return [_Layer(cache[l]) for l in range(cache.shape[0])]
