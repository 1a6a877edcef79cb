"""Plain CPU oracle of two alternative ways to produce the shared index list.

TEST INFRASTRUCTURE ONLY, like clsa_oracle.py: only the test suite, the smoke
check and the CPU-baseline leg of the benchmark may import it; the library
never does, and nothing here is shared with it.  NumPy, float64.

1. Centroid table router.  Source: the CSAttention summary (news.neo-ai.one,
   article on CSAttention and STACK, section on CSAttention): the queries of
   a long context are not spread evenly, so clustering them into centroids
   predicts which keys matter; the heavy work runs at prefill and builds a
   fixed-size query-centroid lookup table per request; at decode the table is
   consulted instead of scanning the whole context, with the scores still
   accumulated on the GPU.
2. Cross-layer score aggregation.  Source: the CLAA abstract (fugumt.com,
   "CLAA: Cross-Layer Attention Aggregation for Accelerating LLM Prefill"):
   token importance estimated in single layers is unstable from layer to
   layer; aggregating it across layers gives a stable ranking.

Readings where the pages are silent (the plainest reading they support):
  * C1 clusters: Lloyd's k-means with squared Euclidean distance over the
    prefill's routing queries; centroid c starts at query floor(c M / C);
    each query joins its nearest centroid (ties: the lower centroid); a
    centroid becomes the mean of its queries, and one with no query keeps
    its place; a fixed number of rounds;
  * C2 table: each centroid's row of the table lists the T keys it scores
    highest (top-T by centroid . key, the routing rule: ties to the lower
    position, ascending);
  * C3 lookup: a decode query scores the C centroids, takes its P best (ties:
    the lower centroid), and the candidates are the union of their table rows
    plus every key past the positions the table covers (keys appended since
    it was built); the query's exact scores over the candidates give the
    top-k (same rule as top-k routing);
  * A1 aggregation: layer l has its own routing query and keys; a key's
    aggregated score is the sum over layers of q_l . K_l[j] (a mean ranks the
    same), and the shared list is the top-k of that sum.

Parity pins live in tests/test_router_oracle.py.
"""
from __future__ import annotations

import numpy as np

from oracle import clsa_oracle as O

__all__ = [
    "kmeans_init",
    "kmeans_round",
    "kmeans",
    "centroid_table",
    "table_route",
    "aggregated_scores",
    "aggregated_route",
]


def kmeans_init(Q, C: int) -> np.ndarray:
    """Centroid c starts at query floor(c M / C) (reading C1)."""
    Q = np.asarray(Q, dtype=np.float64)
    M = Q.shape[0]
    return Q[[(c * M) // C for c in range(C)]].copy()


def kmeans_round(Q, mu):
    """One Lloyd round (reading C1): nearest centroid by squared Euclidean
    distance (ties to the lower centroid), then the mean of each cluster
    (an empty cluster keeps its centroid).  Returns (new mu, assignment)."""
    Q = np.asarray(Q, dtype=np.float64)
    mu = np.asarray(mu, dtype=np.float64)
    d2 = ((Q[:, None, :] - mu[None, :, :]) ** 2).sum(axis=2)
    assign = np.argmin(d2, axis=1)  # first minimum: the lower centroid
    new = mu.copy()
    for c in range(mu.shape[0]):
        mem = assign == c
        if mem.any():
            new[c] = Q[mem].mean(axis=0)
    return new, assign


def kmeans(Q, C: int, rounds: int):
    mu = kmeans_init(Q, C)
    for _ in range(rounds):
        mu, _ = kmeans_round(Q, mu)
    return mu


def centroid_table(mu, K, n: int, T: int) -> np.ndarray:
    """Row c: the T keys (of positions < n) that centroid c scores highest,
    ascending, -1 padded (reading C2)."""
    mu = np.asarray(mu, dtype=np.float64)
    tab = np.full((mu.shape[0], T), -1, dtype=np.int64)
    for c in range(mu.shape[0]):
        sel = O.topk_select(O.route_scores(mu[c], K, n), T)
        tab[c, : len(sel)] = sel
    return tab


def table_route(q, K, mu, tab, n_table: int, n_vis: int, P: int, k: int):
    """Top-k of one decode query through the table (reading C3).

    Returns (ascending positions, the candidate positions, the exact scores
    of every visible key -- for the boundary rule of the tests)."""
    q = np.asarray(q, dtype=np.float64)
    cs = np.asarray(mu, dtype=np.float64) @ q
    order = np.lexsort((np.arange(len(cs)), -cs))  # best first, ties to the lower centroid
    cand = set()
    for c in order[:P]:
        cand.update(int(j) for j in tab[c] if 0 <= j < n_vis)
    cand.update(range(min(n_table, n_vis), n_vis))
    cand = np.array(sorted(cand), dtype=np.int64)
    s_all = O.route_scores(q, K, n_vis)
    if cand.size == 0:
        return cand, cand, s_all
    pick = O.topk_select(s_all[cand], k)  # ties: lower index within cand = lower position
    return np.sort(cand[pick]), cand, s_all


def aggregated_scores(q_layers, K_layers, n: int) -> np.ndarray:
    """sum_l q_l . K_l[j] for j < n (reading A1)."""
    return sum(O.route_scores(q, K, n) for q, K in zip(q_layers, K_layers))


def aggregated_route(q_layers, K_layers, n: int, k: int):
    """The shared list of cross-layer aggregation: top-k of the summed
    scores (reading A1).  Returns (ascending positions, summed scores)."""
    s = aggregated_scores(q_layers, K_layers, n)
    return O.topk_select(s, k), s
