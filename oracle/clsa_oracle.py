"""Plain CPU oracle for shared-routing sparse decode attention (CLSA).

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously correct
definition that the HIP path is checked against.  Only the test suite, the
smoke check and the CPU-baseline leg of the benchmark may import it; the
library and its Python binding never do, and nothing here is shared with
them (no kernels, headers, helpers, tables or pre/post-processing).

Everything is computed in float64 with NumPy.  Inputs are the exact values
the GPU receives (bf16 or fp32), widened exactly to float64 by the caller.

Sources (the pages this follows):

* CLSA explainer, ai-papers.net ("CLSAとは？ルーティング共有で128Kコンテキスト
  推論を17倍高速化するスパースアテンション"):
  - section "CLSAの仕組み": the self-decoder computes, once per query token, a
    top-k list of the KV positions that matter, and every cross-decoder layer
    attends over exactly that list;
  - same section: k = 2048 tokens is the operating point;
  - section "計算コストの削減効果": routing is paid once (cost ~ N) instead of
    once per layer (~ L*N).
* Louver summary, gist.science ("技術サマリー：スパースアテンションを範囲検索問題
  として捉える", arXiv 2605.06763):
  - section "1. 半空間範囲検索への帰着": keys are points, a query q with a
    threshold tau defines the half-space {p : <q, p> >= tau}, and the answer
    is every key inside it (no false negatives).

Readings where the pages are silent (the plainest reading the rest of the
pages supports):

* R1/R2  the routing score is the raw inner product q_idx . K_idx[j] with no
         scale and no nonlinearity (one index head);
* R3     the attention logit is scaled by 1/sqrt(D) unless a scale is given;
* R4     GQA: query head h reads KV head floor(h * Hkv / Hq);
* R5     top-k ties go to the lower key index;
* R6     index lists are returned in ascending key order;
* R7     k larger than the visible context returns every visible key;
* R8     in a prefill chunk, the query at absolute position p sees keys 0..p;
* R10    threshold mode keeps s >= tau, tau given as float32 and widened;
* R11    an empty selection gives output 0 and lse = -inf;
* R12    -0.0 and +0.0 scores are equal (float64 comparison does this);
* R24    a list passed to attention is read up to min(count, cap) entries
         (a negative count reads none); entries outside [0, n_cap) are
         padding, like the -1 that pads a returned list, and take no
         part in the softmax; a position listed twice counts twice;
* R25    a context length n_ctx[b] outside [0, n_cap] is taken as the
         nearest end of that range.

Parity pins live in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "route_scores",
    "topk_select",
    "threshold_select",
    "attend_head",
    "visible_count",
    "route",
    "route_threshold",
    "sparse_attn",
]


# ---------------------------------------------------------------------------
# O1: routing score  (CLSA explainer, section "CLSAの仕組み"; Louver summary,
# section "1. 半空間範囲検索への帰着" for the raw inner product <q, p>)
# ---------------------------------------------------------------------------
def route_scores(q_idx_row, K_idx_seq, n_vis: int) -> np.ndarray:
    """s[j] = sum_i q_idx[i] * K_idx[j, i] for j < n_vis, in float64.

    q_idx_row: [d]; K_idx_seq: [n_cap, d] (rows beyond n_vis are ignored).
    The matrix-vector product is the library primitive for the sum over i.
    """
    q = np.asarray(q_idx_row, dtype=np.float64)
    K = np.asarray(K_idx_seq[:n_vis], dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(0, dtype=np.float64)
    return K @ q


# ---------------------------------------------------------------------------
# O2: exact top-k  (CLSA explainer, section "CLSAの仕組み": the k tokens with
# the highest routing scores; ties to the lower index and ascending output
# order are readings R5/R6)
# ---------------------------------------------------------------------------
def topk_select(s: np.ndarray, k: int) -> np.ndarray:
    """Indices of the min(k, len(s)) largest scores, ascending.

    Ordering key: score descending, then index ascending.  np.lexsort sorts
    by the last key first, so (j, -s) sorts by -s and breaks ties by j.
    """
    s = np.asarray(s, dtype=np.float64)
    n = s.shape[0]
    j = np.arange(n, dtype=np.int64)
    order = np.lexsort((j, -s))
    sel = order[: min(int(k), n)]
    return np.sort(sel).astype(np.int64)


# ---------------------------------------------------------------------------
# O3: exact half-space selection  (Louver summary, section
# "1. 半空間範囲検索への帰着": every key with <q, k> >= tau, none other)
# ---------------------------------------------------------------------------
def threshold_select(s: np.ndarray, tau) -> np.ndarray:
    """All j with s[j] >= tau (tau is a float32 value, widened exactly)."""
    t = np.float64(np.float32(tau))
    return np.flatnonzero(np.asarray(s, dtype=np.float64) >= t).astype(np.int64)


# ---------------------------------------------------------------------------
# O4: softmax attention over the selected rows  (CLSA explainer, section
# "CLSAの仕組み": each cross-decoder layer attends over the shared list)
# ---------------------------------------------------------------------------
def attend_head(q_h, K_sel, V_sel, scale: float, return_weights: bool = False):
    """One query head over its selected rows.

    q_h: [D]; K_sel, V_sel: [n_sel, D] (the rows of this head's KV head at
    the selected positions).  Returns (out [D], lse) and optionally the
    softmax weights p [n_sel].
    """
    q = np.asarray(q_h, dtype=np.float64)
    K = np.asarray(K_sel, dtype=np.float64)
    V = np.asarray(V_sel, dtype=np.float64)
    if K.shape[0] == 0:
        out = np.zeros(q.shape[0], dtype=np.float64)
        res = (out, -math.inf)
        return res + (np.zeros(0),) if return_weights else res
    z = (K @ q) * float(scale)
    zmax = z.max()
    e = np.exp(z - zmax)
    tot = e.sum()
    p = e / tot
    out = p @ V
    lse = float(zmax + np.log(tot))
    if return_weights:
        return out, lse, p
    return out, lse


# ---------------------------------------------------------------------------
# Batched wrappers with the library's shapes
# ---------------------------------------------------------------------------
def visible_count(n_ctx_b: int, q_pos0: int, m: int, n_cap: int | None = None) -> int:
    """Keys visible to query row m: the whole context in decode (q_pos0 < 0),
    keys 0..q_pos0+m in a prefill chunk (reading R8); a context length
    outside [0, n_cap] counts as the nearest end of that range (R25)."""
    n = max(0, int(n_ctx_b))
    if n_cap is not None:
        n = min(n, int(n_cap))
    if q_pos0 < 0:
        return n
    return int(min(n, q_pos0 + m + 1))


def route(q_idx, K_idx, n_ctx, q_pos0: int, k: int, cap: int, rows=None):
    """Top-k routing for every (b, m) row.

    q_idx: [B, M, d]; K_idx: [B, n_cap, d]; n_ctx: [B].
    Returns idx [B, M, cap] int64 (ascending, -1 padded) and counts [B, M].
    rows: optional list of (b, m) to compute (others stay -1 / 0).
    """
    B, M, _ = q_idx.shape
    idx = np.full((B, M, cap), -1, dtype=np.int64)
    counts = np.zeros((B, M), dtype=np.int64)
    todo = rows if rows is not None else [(b, m) for b in range(B) for m in range(M)]
    for b, m in todo:
        nv = visible_count(n_ctx[b], q_pos0, m, K_idx.shape[1])
        s = route_scores(q_idx[b, m], K_idx[b], nv)
        sel = topk_select(s, k)
        idx[b, m, : sel.shape[0]] = sel
        counts[b, m] = sel.shape[0]
    return idx, counts


def route_threshold(q_idx, K_idx, n_ctx, q_pos0: int, tau, cap: int, rows=None):
    """Threshold routing for every (b, m) row; tau: [B, M] float32.

    counts holds the true size of the set; only the first cap indices are
    stored (the library's capacity convention).
    """
    B, M, _ = q_idx.shape
    idx = np.full((B, M, cap), -1, dtype=np.int64)
    counts = np.zeros((B, M), dtype=np.int64)
    todo = rows if rows is not None else [(b, m) for b in range(B) for m in range(M)]
    for b, m in todo:
        nv = visible_count(n_ctx[b], q_pos0, m, K_idx.shape[1])
        s = route_scores(q_idx[b, m], K_idx[b], nv)
        sel = threshold_select(s, tau[b, m])
        w = min(cap, sel.shape[0])
        idx[b, m, :w] = sel[:w]
        counts[b, m] = sel.shape[0]
    return idx, counts


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """GQA group of query head h (reading R4)."""
    return (h * Hkv) // Hq


def sparse_attn(q, K, V, idx, counts, cap: int, scale: float = 0.0, rows=None, layers=None):
    """Sparse attention in every layer over the shared index lists.

    q: list over layers of [B, M, Hq, D]; K, V: list over layers of
    [B, n_cap, Hkv, D] (any array-like supporting fancy row indexing, so a
    caller may pass lazily gathered rows); idx [B, M, cap]; counts [B, M].
    Returns out [L, B, M, Hq, D] and lse [L, B, M, Hq] (float64).
    """
    L = len(q)
    B, M, Hq, D = q[0].shape
    n_cap, Hkv = K[0].shape[1], K[0].shape[2]
    sc = float(scale) if scale else 1.0 / math.sqrt(D)
    out = np.zeros((L, B, M, Hq, D), dtype=np.float64)
    lse = np.full((L, B, M, Hq), -math.inf, dtype=np.float64)
    todo = rows if rows is not None else [(b, m) for b in range(B) for m in range(M)]
    lays = layers if layers is not None else range(L)
    for l in lays:
        for b, m in todo:
            n = max(0, int(min(counts[b, m], cap)))
            sel = np.asarray(idx[b, m, :n], dtype=np.int64)
            sel = sel[(sel >= 0) & (sel < n_cap)]  # padding entries (R24)
            Kr = np.asarray(K[l][b][sel], dtype=np.float64)  # [n, Hkv, D]
            Vr = np.asarray(V[l][b][sel], dtype=np.float64)
            for h in range(Hq):
                g = kv_head_of(h, Hq, Hkv)
                o, s = attend_head(q[l][b, m, h], Kr[:, g, :], Vr[:, g, :], sc)
                out[l, b, m, h] = o
                lse[l, b, m, h] = s
    return out, lse
