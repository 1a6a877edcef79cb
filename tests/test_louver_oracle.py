"""Pins of the Louver oracle (CPU only).

Louver summary, gist.science, sections "2. Louver インデックス" and
"クエリアルゴリズム": a balanced PCA tree per subspace, bounding balls, a
ball-versus-half-space filter, Query 1 (all-subspace filter) and Query 2
(threshold algorithm), both with zero false negatives.  Each pin checks the
oracle against something it does not compute itself:

* the query answer equals the exact threshold set of clsa_oracle (itself
  pinned in test_oracle_pins.py) on Gaussian, clustered and duplicated keys,
  with several segments and a buffer -- the page's zero-false-negative
  guarantee, and no false positives since survivors are checked exactly;
* the ball bound holds for every key (Cauchy-Schwarz, checked by brute
  force), and every unseen key of a TA scan is bounded below tau;
* the tree is balanced and its clusters partition the segment;
* every split orders its node along the principal axis found by an SVD
  (a different routine from the oracle's eigh);
* every ball contains its members, tightly, around their mean.
The battery is re-run against deliberately broken copies at the end.
"""
from __future__ import annotations

import math
import types

import numpy as np
import pytest

from oracle import clsa_oracle as O
from oracle import louver_oracle as LV


def _ns(**over):
    base = dict(build_segment=LV.build_segment, query_all_subspace=LV.query_all_subspace,
                query_ta=LV.query_ta, cluster_bounds=LV.cluster_bounds)
    base.update(over)
    return types.SimpleNamespace(**base)


def _gauss(n, d, seed):
    return np.random.default_rng(seed).standard_normal((n, d))


def _clustered(n, d, seed, centers=6, sigma=0.05):
    rng = np.random.default_rng(seed)
    c = rng.standard_normal((centers, d))
    return c[rng.integers(0, centers, n)] + sigma * rng.standard_normal((n, d))


def _taus(s, fracs=(0.0, 0.01, 0.1, 0.5, 1.0)):
    srt = np.sort(s)[::-1]
    out = [float(np.float32(srt[0] + 1.0)), float(np.float32(srt[-1] - 1.0))]
    for f in fracs[1:-1]:
        c = max(1, int(f * len(s)))
        out.append(float(np.float32(0.5 * (srt[c - 1] + srt[c]))))
    return out


def _cases():
    yield "gauss", _gauss(300, 32, 1)
    yield "clustered", _clustered(300, 32, 2)
    K = _gauss(40, 32, 3)
    yield "duplicated", K[np.random.default_rng(4).integers(0, 40, 300)]


# --------------------------------------------------------------------------
def pin_queries_are_the_threshold_set(o):
    rng = np.random.default_rng(11)
    for name, K in _cases():
        for S in (1, 2, 4):
            segs = [o.build_segment(K, 0, 200, S, 16), o.build_segment(K, 200, 260, S, 8)]
            for trial in range(3):
                q = rng.standard_normal(32) / math.sqrt(32)
                n_vis = 300 - 13 * trial
                s = O.route_scores(q, K, n_vis)
                for tau in _taus(s):
                    want = O.threshold_select(s, tau)
                    for qf in (o.query_all_subspace, o.query_ta):
                        got, _ = qf(segs, K, q, tau, n_vis)
                        assert np.array_equal(got, want), (name, S, qf.__name__, tau)


def pin_ball_bound_holds_for_every_key(o):
    for name, K in _cases():
        for S in (1, 2, 4):
            seg = o.build_segment(K, 0, 300, S, 16)
            q = np.random.default_rng(5).standard_normal(32)
            ub = o.cluster_bounds(seg, q)
            ds = 32 // S
            for s in range(S):
                for i, mem in enumerate(seg["clusters"][s]):
                    sc = K[mem, s * ds:(s + 1) * ds] @ q[s * ds:(s + 1) * ds]
                    assert np.all(sc <= ub[s][i] + 1e-12), (name, S, s, i)


def pin_tree_is_balanced_and_partitions(o):
    for n, r in ((300, 16), (257, 8), (64, 64), (65, 64), (5, 16), (1024, 32)):
        K = _gauss(n + 7, 16, n)
        seg = o.build_segment(K, 7, 7 + n, 2, r)
        h = seg["h"]
        assert h == (0 if n <= r else math.ceil(math.log2(n / r)))
        for s in range(2):
            cl = seg["clusters"][s]
            assert len(cl) == 1 << h
            sizes = {len(c) for c in cl}
            assert sizes <= {n // (1 << h), -(-n // (1 << h))} and max(sizes) <= r
            allpos = np.sort(np.concatenate(cl))
            assert np.array_equal(allpos, np.arange(7, 7 + n))


def pin_splits_follow_the_principal_axis(o):
    K = _gauss(256, 16, 21) * np.linspace(3.0, 0.5, 16)  # distinct variances: clear top axis
    seg = o.build_segment(K, 0, 256, 1, 16)
    for level in seg["tree"][0]:
        for left, right, v in level:
            X = K[np.concatenate([left, right])]
            _, _, Vt = np.linalg.svd(X - X.mean(axis=0), full_matrices=False)
            assert abs(abs(float(Vt[0] @ v)) - 1.0) < 1e-6
            pl, pr = K[left] @ v, K[right] @ v
            assert pl.max() <= pr.min()
            assert abs(len(left) - len(right)) <= 1


def pin_balls_are_tight(o):
    K = _clustered(300, 32, 31)
    seg = o.build_segment(K, 0, 300, 4, 16)
    for s in range(4):
        X = K[:, s * 8:(s + 1) * 8]
        for i, mem in enumerate(seg["clusters"][s]):
            c = seg["centers"][s][i]
            assert np.allclose(c, X[mem].mean(axis=0), atol=1e-12)
            dist = np.sqrt(((X[mem] - c) ** 2).sum(axis=1))
            assert abs(dist.max() - seg["radii"][s][i]) < 1e-12


def pin_ta_unseen_keys_are_below_tau(o):
    K = _gauss(400, 32, 41)
    rng = np.random.default_rng(42)
    for S in (2, 4):
        seg = o.build_segment(K, 0, 400, S, 16)
        for _ in range(4):
            q = rng.standard_normal(32)
            s = K @ q
            tau = float(np.float32(np.sort(s)[::-1][20]))
            _, ncand = o.query_ta([seg], K, q, tau, 400)
            ub = o.cluster_bounds(seg, q)
            cid = [np.empty(400, dtype=np.int64) for _ in range(S)]
            for ss in range(S):
                for i, mem in enumerate(seg["clusters"][ss]):
                    cid[ss][mem] = i
            best = sum(ub[ss][cid[ss]] for ss in range(S))  # each key's bound
            # every key the scan left unseen must be bounded below tau; the
            # scan sees exactly ncand keys, the ones with the largest bounds
            # cannot all be unseen
            assert ncand <= 400
            assert np.all(np.sort(best)[::-1][ncand:] < tau) or ncand == 400


def pin_pruning_on_clustered_keys(o):
    # tight clusters: a query's half-space misses most balls (S = 1 keeps
    # whole clusters or nothing); on these inputs the index must check
    # fewer than half of the keys, or it is not pruning at all
    K = _clustered(2048, 32, 51, centers=32, sigma=0.02)
    seg = o.build_segment(K, 0, 2048, 1, 32)
    q = np.random.default_rng(52).standard_normal(32) / math.sqrt(32)
    s = K @ q
    tau = float(np.float32(np.sort(s)[::-1][100]))
    got, ncand = o.query_all_subspace([seg], K, q, tau, 2048)
    assert np.array_equal(got, O.threshold_select(s, tau))
    assert ncand < 1024, ncand


ALL_PINS = [pin_queries_are_the_threshold_set, pin_ball_bound_holds_for_every_key,
            pin_tree_is_balanced_and_partitions, pin_splits_follow_the_principal_axis,
            pin_balls_are_tight, pin_ta_unseen_keys_are_below_tau,
            pin_pruning_on_clustered_keys]


def battery(o):
    for p in ALL_PINS:
        p(o)


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(_ns())


# --------------------------------------------------------------- mutants
def _mut_build_no_radius(K, start, end, S, r):
    seg = LV.build_segment(K, start, end, S, r)
    seg["radii"] = [0.0 * x for x in seg["radii"]]
    return seg


def _mut_build_unsorted(K, start, end, S, r):
    # splits by slot order instead of by projection
    orig = LV._principal_axis
    try:
        LV._principal_axis = lambda X: np.zeros(X.shape[1])
        return LV.build_segment(K, start, end, S, r)
    finally:
        LV._principal_axis = orig


def _mut_bounds_minus_radius(seg, q):
    q = np.asarray(q, dtype=np.float64)
    ds = seg["ds"]
    return [seg["centers"][s] @ q[s * ds:(s + 1) * ds] - seg["radii"][s]
            * np.linalg.norm(q[s * ds:(s + 1) * ds]) for s in range(seg["S"])]


def _mut_query1_own_threshold(segs, K, q, tau, n_vis):
    # prunes each subspace against tau itself, forgetting the other subspaces
    t = np.float64(np.float32(tau))
    cand = []
    for seg in segs:
        ub = LV.cluster_bounds(seg, q)
        passing = None
        for s in range(seg["S"]):
            mem = set()
            for i in np.flatnonzero(ub[s] >= t):
                mem.update(int(j) for j in seg["clusters"][s][i])
            passing = mem if passing is None else passing & mem
        cand.extend(j for j in passing if j < n_vis)
    cand.extend(range(max(sg["end"] for sg in segs), n_vis))
    return LV._exact(K, q, cand, tau), len(set(cand))


def _mut_ta_stops_early(segs, K, q, tau, n_vis):
    t = np.float64(np.float32(tau))
    cand = set()
    for seg in segs:
        ub = LV.cluster_bounds(seg, q)
        S, C = seg["S"], len(ub[0])
        ranked = [np.lexsort((np.arange(C), -u)) for u in ub]
        depth = C
        for dpt in range(C):
            if sum(ub[s][ranked[s][dpt]] for s in range(S)) < t:
                depth = dpt
                break
        depth = max(0, depth - 1)
        for s in range(S):
            for i in ranked[s][:depth]:
                cand.update(int(j) for j in seg["clusters"][s][i] if j < n_vis)
    cand.update(range(max(sg["end"] for sg in segs), n_vis))
    return LV._exact(K, q, cand, tau), len(cand)


def _mut_no_buffer(segs, K, q, tau, n_vis):
    got, n = LV.query_ta(segs, K, q, tau, max(sg["end"] for sg in segs))
    return got, n


def _mut_unbalanced(K, start, end, S, r):
    seg = LV.build_segment(K, start, end, S, r)
    for s in range(S):
        cl = seg["clusters"][s]
        if len(cl) > 1 and len(cl[0]) > 1:
            cl[1] = np.concatenate([cl[0][-1:], cl[1]])
            cl[0] = cl[0][:-1]
    return seg


MUTANTS = {
    "ball_without_radius": dict(build_segment=_mut_build_no_radius),
    "split_not_along_axis": dict(build_segment=_mut_build_unsorted),
    "bound_subtracts_radius": dict(cluster_bounds=_mut_bounds_minus_radius),
    "query1_ignores_other_subspaces": dict(query_all_subspace=_mut_query1_own_threshold),
    "ta_stops_one_depth_early": dict(query_ta=_mut_ta_stops_early),
    "buffer_not_checked": dict(query_ta=_mut_no_buffer),
    "tree_unbalanced": dict(build_segment=_mut_unbalanced),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    over = MUTANTS[name]
    for fn, impl in over.items():
        if fn == "cluster_bounds":  # the queries call the module-level helper
            monkeypatch.setattr(LV, fn, impl)
    with pytest.raises(AssertionError):
        battery(_ns(**over))
