"""Plain CPU oracle of the Louver index for threshold (half-space) selection.

TEST INFRASTRUCTURE ONLY, like clsa_oracle.py: only the test suite, the smoke
check and the CPU-baseline leg of the benchmark may import it; the library
never does, and nothing here is shared with it.  NumPy, float64.

Source: Louver summary, gist.science ("技術サマリー：スパースアテンションを範囲
検索問題として捉える", arXiv 2605.06763):
  * section "1. 半空間範囲検索への帰着": keys are points; a query q and a
    threshold tau define the half-space {p : <q, p> >= tau}; the answer is
    every key inside it, with no false negatives;
  * section "2. Louver インデックス": the d-dimensional key space is cut
    into S contiguous subspaces, each indexed on its own; inside a subspace a
    balanced PCA tree groups the keys into clusters of a fixed size r; every
    cluster is wrapped in a bounding ball (center c, radius rho); a query
    first tests each ball against its half-space and prunes clusters whose
    ball misses it, then checks the surviving keys exactly; keys added
    during decoding wait in a buffer and are clustered into the index when
    it fills, without rebuilding what is there;
  * section "クエリアルゴリズム": Query 1 prunes the clusters of each
    subspace on their own with per-subspace thresholds; Query 2 adapts the
    threshold algorithm (TA): one global threshold, clusters scanned in
    descending upper bound until a stopping rule holds.  Both return every
    key scoring >= tau.

Readings where the page is silent (the plainest reading the rest supports):
  * L1 ball test: the largest <q_s, p> over a ball is <q_s, c> + rho |q_s|
    (Cauchy-Schwarz), so a cluster can hold a key scoring >= t in subspace s
    only if that bound is >= t;
  * L2 PCA split: a node's principal axis is the top eigenvector of its
    members' covariance; members are ordered by their projection on it
    (ties by key position) and the lower part goes to the left child;
  * L3 balance: level l of a tree over n keys has 2^l nodes, node i holding
    the ordered slots floor(i n / 2^l) .. floor((i+1) n / 2^l) - 1; the tree
    has the fewest levels h with ceil(n / 2^h) <= r, so leaves hold
    floor(n / 2^h) or ceil(n / 2^h) <= r keys;
  * L4 ball: center = mean of the members, radius = largest member distance;
  * L5 Query 1 thresholds: tau_s = tau - sum over the other subspaces of
    their largest cluster bound; a key is a candidate when its cluster
    passes in every subspace;
  * L6 Query 2: per subspace the clusters in descending bound (ties by
    cluster number); the scan stops at the first depth t whose bounds sum
    below tau (the best any unseen key can score); the candidates are the
    members of every cluster of rank below t, in any subspace;
  * L7 buffer: keys at positions past the indexed ones are checked exactly;
    an index is a list of segments, each a tree over a contiguous range of
    positions, and clustering the buffer appends a segment.

Parity pins live in tests/test_louver_oracle.py.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "tree_levels",
    "build_segment",
    "cluster_bounds",
    "query_all_subspace",
    "query_ta",
]


def tree_levels(n: int, r: int) -> int:
    """Fewest levels h with ceil(n / 2^h) <= r (reading L3)."""
    h = 0
    while -(-n // (1 << h)) > r:
        h += 1
    return h


def _principal_axis(X: np.ndarray) -> np.ndarray:
    """Top eigenvector of the covariance of the rows of X (reading L2)."""
    Xc = X - X.mean(axis=0)
    w, V = np.linalg.eigh(Xc.T @ Xc)
    return V[:, np.argmax(w)]


def build_segment(K, start: int, end: int, S: int, r: int) -> dict:
    """A Louver index segment over key positions start .. end-1 of K [n, d].

    Returns {"start", "end", "S", "ds", "h", "clusters": [per subspace: list
    of position arrays], "centers": [per subspace: [C, ds]], "radii": [per
    subspace: [C]], "tree": [per subspace: list of levels, each a list of
    (left positions, right positions, axis) for the splits made there]}.
    """
    K = np.asarray(K, dtype=np.float64)
    d = K.shape[1]
    assert d % S == 0
    ds = d // S
    n = end - start
    h = tree_levels(n, r)
    seg = {"start": start, "end": end, "S": S, "ds": ds, "h": h,
           "clusters": [], "centers": [], "radii": [], "tree": []}
    for s in range(S):
        X = K[:, s * ds:(s + 1) * ds]
        order = np.arange(start, end, dtype=np.int64)  # slot -> position
        levels = []
        for lv in range(h):
            splits = []
            for i in range(1 << lv):
                lo = (i * n) >> lv
                hi = ((i + 1) * n) >> lv
                mid = ((2 * i + 1) * n) >> (lv + 1)
                mem = order[lo:hi]
                v = _principal_axis(X[mem])
                p = X[mem] @ v
                o = np.lexsort((mem, p))  # projection ascending, ties by position
                order[lo:hi] = mem[o]
                splits.append((order[lo:mid].copy(), order[mid:hi].copy(), v))
            levels.append(splits)
        C = 1 << h
        clusters = [order[(i * n) >> h:((i + 1) * n) >> h].copy() for i in range(C)]
        centers = np.stack([X[c].mean(axis=0) for c in clusters])
        radii = np.array([np.sqrt(((X[c] - centers[i]) ** 2).sum(axis=1)).max()
                          for i, c in enumerate(clusters)])
        seg["clusters"].append(clusters)
        seg["centers"].append(centers)
        seg["radii"].append(radii)
        seg["tree"].append(levels)
    return seg


def cluster_bounds(seg: dict, q) -> list:
    """Per subspace, every cluster's largest possible <q_s, p> (reading L1)."""
    q = np.asarray(q, dtype=np.float64)
    ds = seg["ds"]
    out = []
    for s in range(seg["S"]):
        qs = q[s * ds:(s + 1) * ds]
        out.append(seg["centers"][s] @ qs + seg["radii"][s] * np.linalg.norm(qs))
    return out


def _exact(K, q, cand, tau) -> np.ndarray:
    cand = np.asarray(sorted(set(int(j) for j in cand)), dtype=np.int64)
    if cand.size == 0:
        return cand
    s = np.asarray(K, dtype=np.float64)[cand] @ np.asarray(q, dtype=np.float64)
    return cand[s >= np.float64(np.float32(tau))]


def _buffer(segs, n_vis: int):
    last = max([sg["end"] for sg in segs], default=0)
    return np.arange(last, n_vis, dtype=np.int64)


def query_all_subspace(segs, K, q, tau, n_vis: int):
    """Query 1 (reading L5) over every segment, plus the exact buffer.

    Returns (ascending positions with score >= tau, number of keys checked
    exactly).  Only positions < n_vis count."""
    t = np.float64(np.float32(tau))
    cand = []
    for seg in segs:
        ub = cluster_bounds(seg, q)
        S = seg["S"]
        tops = [u.max() for u in ub]
        ok = [ub[s] >= t - (sum(tops) - tops[s]) for s in range(S)]
        passing = None
        for s in range(S):
            mem = set()
            for i in np.flatnonzero(ok[s]):
                mem.update(int(j) for j in seg["clusters"][s][i])
            passing = mem if passing is None else passing & mem
        cand.extend(j for j in passing if j < n_vis)
    cand.extend(_buffer(segs, n_vis).tolist())
    return _exact(K, q, cand, tau), len(set(cand))


def query_ta(segs, K, q, tau, n_vis: int):
    """Query 2, the threshold algorithm (reading L6), over every segment,
    plus the exact buffer.  Returns (positions, keys checked exactly)."""
    t = np.float64(np.float32(tau))
    cand = set()
    for seg in segs:
        ub = cluster_bounds(seg, q)
        S = seg["S"]
        C = len(ub[0])
        ranked = [np.lexsort((np.arange(C), -u)) for u in ub]  # descending, ties by number
        depth = C
        for dpt in range(C):
            if sum(ub[s][ranked[s][dpt]] for s in range(S)) < t:
                depth = dpt
                break
        for s in range(S):
            for i in ranked[s][:depth]:
                cand.update(int(j) for j in seg["clusters"][s][i] if j < n_vis)
    cand.update(_buffer(segs, n_vis).tolist())
    return _exact(K, q, cand, tau), len(cand)
