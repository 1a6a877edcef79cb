"""Pins of the alternative-router oracle (CPU only).

Centroid table router (CSAttention summary, news.neo-ai.one) and cross-layer
score aggregation (CLAA abstract, fugumt.com).  The pages print no example
and no formula, so these routers' readings are stated in the oracle's header
and pinned here against what fixes them independently of the oracle:

* a k-means round equals brute-force loops; Lloyd rounds never raise the
  within-cluster sum of squares; with one centroid per query the centroids
  are the queries; well separated clusters are recovered;
* a table row is the library top-k (torch.topk) of the centroid's scores;
* probing every centroid of full tables, or indexing nothing (every key in
  the buffer), gives exactly the plain top-k of all keys;
* the lookup equals a loop-by-loop evaluation on tiny inputs and never
  returns a key outside its candidates;
* the aggregated score over layers equals one inner product of the
  concatenated query and key rows, and one layer is plain top-k routing.
The battery runs again against broken copies at the end.
"""
from __future__ import annotations

import types

import numpy as np
import pytest
import torch

from oracle import clsa_oracle as O
from oracle import router_oracle as RO


def _ns(**over):
    base = dict(kmeans_round=RO.kmeans_round, kmeans=RO.kmeans, centroid_table=RO.centroid_table,
                table_route=RO.table_route, aggregated_route=RO.aggregated_route)
    base.update(over)
    return types.SimpleNamespace(**base)


def _bf(shape, seed, scale=1.0):
    x = torch.from_numpy(np.random.default_rng(seed).standard_normal(shape) * scale)
    return x.to(torch.bfloat16).double().numpy()


# --------------------------------------------------------------------------
def pin_kmeans_round_brute_force(o):
    Q = _bf((40, 5), 1)
    mu = _bf((6, 5), 2)
    mu[3] = mu[1]  # equal centroids: ties go to the lower one
    new, assign = o.kmeans_round(Q, mu)
    for i in range(40):
        best, bc = None, None
        for c in range(6):
            dd = sum((Q[i, e] - mu[c, e]) ** 2 for e in range(5))
            if best is None or dd < best:
                best, bc = dd, c
        assert assign[i] == bc
    for c in range(6):
        mem = [i for i in range(40) if assign[i] == c]
        want = mu[c] if not mem else np.mean(Q[mem], axis=0)
        assert np.allclose(new[c], want, atol=1e-12)


def pin_kmeans_inertia_falls(o):
    Q = _bf((300, 8), 3)
    mu = RO.kmeans_init(Q, 7)
    prev = np.inf
    for _ in range(6):
        d2 = ((Q[:, None] - mu[None]) ** 2).sum(axis=2).min(axis=1).sum()
        assert d2 <= prev + 1e-9
        prev = d2
        mu, _ = o.kmeans_round(Q, mu)


def pin_kmeans_one_centroid_per_query(o):
    Q = _bf((12, 4), 4)
    mu = o.kmeans(Q, 12, 3)
    assert np.array_equal(mu, Q)


def pin_kmeans_separated_clusters(o):
    rng = np.random.default_rng(5)
    cent = np.array([[10.0, 0, 0], [0, 10.0, 0], [0, 0, 10.0]])
    lab = np.repeat(np.arange(3), 50)
    Q = cent[lab] + 0.1 * rng.standard_normal((150, 3))
    mu = o.kmeans(Q, 3, 5)
    for c in range(3):
        assert np.allclose(mu[c], Q[lab == c].mean(axis=0), atol=1e-12)


def pin_table_is_library_topk(o):
    K = _bf((500, 16), 6)
    mu = _bf((5, 16), 7)
    tab = o.centroid_table(mu, K, 480, 37)
    for c in range(5):
        s = torch.from_numpy(K[:480] @ mu[c])
        want = torch.topk(s, 37).indices.sort().values.numpy()
        assert np.array_equal(tab[c], want)
    tab2 = o.centroid_table(mu, K, 20, 37)  # fewer keys than T: all of them, -1 padded
    assert np.array_equal(tab2[0, :20], np.arange(20)) and np.all(tab2[0, 20:] == -1)


def pin_full_tables_are_plain_topk(o):
    K = _bf((400, 16), 8)
    Q = _bf((60, 16), 9)
    mu = o.kmeans(Q, 4, 3)
    full = o.centroid_table(mu, K, 400, 400)
    for i in range(5):
        q = Q[i]
        s = O.route_scores(q, K, 390)
        want = O.topk_select(s, 50)
        got, _, _ = o.table_route(q, K, mu, full, 400, 390, 4, 50)  # every centroid probed
        assert np.array_equal(got, want)
        got2, _, _ = o.table_route(q, K, mu, full[:, :10], 0, 390, 1, 50)  # all in the buffer
        assert np.array_equal(got2, want)


def pin_lookup_brute_force(o):
    K = _bf((60, 6), 10)
    mu = _bf((5, 6), 11)
    tab = o.centroid_table(mu, K, 50, 8)
    for t in range(6):
        q = _bf((6,), 20 + t)
        n_vis = 55 + t % 3
        cs = [sum(q[e] * mu[c, e] for e in range(6)) for c in range(5)]
        order = sorted(range(5), key=lambda c: (-cs[c], c))[:2]
        cand = sorted({int(j) for c in order for j in tab[c] if 0 <= j < n_vis} |
                      set(range(50, n_vis)))
        sc = {j: sum(q[e] * K[j, e] for e in range(6)) for j in cand}
        best = sorted(cand, key=lambda j: (-sc[j], j))[:7]
        got, gcand, _ = o.table_route(q, K, mu, tab, 50, n_vis, 2, 7)
        assert got.tolist() == sorted(best)
        assert set(got.tolist()) <= set(gcand.tolist()) == set(cand)


def pin_aggregation_is_concatenated_product(o):
    L, n, d = 4, 300, 8
    qs = [_bf((d,), 30 + l) for l in range(L)]
    Ks = [_bf((n, d), 40 + l) for l in range(L)]
    qc = np.concatenate(qs)
    Kc = np.concatenate(Ks, axis=1)
    got, s = o.aggregated_route(qs, Ks, 280, 33)
    assert np.allclose(s, Kc[:280] @ qc, atol=1e-12)
    assert np.array_equal(got, O.topk_select(O.route_scores(qc, Kc, 280), 33))
    one, _ = o.aggregated_route(qs[:1], Ks[:1], 280, 33)
    assert np.array_equal(one, O.topk_select(O.route_scores(qs[0], Ks[0], 280), 33))
    rev, _ = o.aggregated_route(qs[::-1], Ks[::-1], 280, 33)
    assert np.array_equal(rev, got)


ALL_PINS = [pin_kmeans_round_brute_force, pin_kmeans_inertia_falls,
            pin_kmeans_one_centroid_per_query, pin_kmeans_separated_clusters,
            pin_table_is_library_topk, pin_full_tables_are_plain_topk, pin_lookup_brute_force,
            pin_aggregation_is_concatenated_product]


def battery(o):
    for p in ALL_PINS:
        p(o)


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(_ns())


# --------------------------------------------------------------- mutants
def _mut_round_ties_high(Q, mu):
    Q = np.asarray(Q, dtype=np.float64)
    d2 = ((Q[:, None, :] - mu[None, :, :]) ** 2).sum(axis=2)
    assign = mu.shape[0] - 1 - np.argmin(d2[:, ::-1], axis=1)
    new = mu.copy()
    for c in range(mu.shape[0]):
        if (assign == c).any():
            new[c] = Q[assign == c].mean(axis=0)
    return new, assign


def _mut_round_empty_to_zero(Q, mu):
    new, assign = RO.kmeans_round(Q, mu)
    for c in range(mu.shape[0]):
        if not (assign == c).any():
            new[c] = 0.0
    return new, assign


def _mut_kmeans_no_update(Q, C, rounds):
    return RO.kmeans_init(Q, C)


def _mut_table_off_by_one(mu, K, n, T):
    return RO.centroid_table(mu, K, n - 1, T)


def _mut_lookup_no_buffer(q, K, mu, tab, n_table, n_vis, P, k):
    return RO.table_route(q, K, mu, tab, n_table, min(n_vis, n_table), P, k)


def _mut_lookup_one_probe_less(q, K, mu, tab, n_table, n_vis, P, k):
    return RO.table_route(q, K, mu, tab, n_table, n_vis, max(P - 1, 1), k)


def _mut_aggregate_max(q_layers, K_layers, n, k):
    s = np.max([O.route_scores(q, K, n) for q, K in zip(q_layers, K_layers)], axis=0)
    return O.topk_select(s, k), s


MUTANTS = {
    "kmeans_ties_to_higher_centroid": dict(kmeans_round=_mut_round_ties_high),
    "kmeans_empty_cluster_to_zero": dict(kmeans_round=_mut_round_empty_to_zero),
    "kmeans_never_updates": dict(kmeans=_mut_kmeans_no_update),
    "table_misses_last_key": dict(centroid_table=_mut_table_off_by_one),
    "lookup_skips_buffer": dict(table_route=_mut_lookup_no_buffer),
    "lookup_probes_one_less": dict(table_route=_mut_lookup_one_probe_less),
    "aggregate_max_not_sum": dict(aggregated_route=_mut_aggregate_max),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    with pytest.raises(AssertionError):
        battery(_ns(**MUTANTS[name]))
