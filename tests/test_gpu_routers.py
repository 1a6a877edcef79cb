"""GPU parity of the two alternative routers against the CPU oracle
(oracle/router_oracle.py).

* Cross-layer aggregation (CLAA abstract, fugumt.com): clsa_route_aggregated
  against the top-k of the oracle's summed scores, with the top-k rule of
  the other routing tests (sets equal up to boundary pairs within 1e-5
  relative of the k-th score); with one head it must equal clsa_route.
* Centroid table router (CSAttention summary, news.neo-ai.one): the k-means
  rounds are followed exactly on well separated queries (centroids within
  one bf16 rounding of the oracle's); the table and the lookup are compared
  with the oracle run on the GPU's own centroids and table, so the
  comparison holds whatever rounding did to the clustering.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from long_context_sparse_routing_amd import binding as clsa
from long_context_sparse_routing_amd import inputs as gen
from oracle import clsa_oracle as O
from oracle import router_oracle as RO
from tests.parity_util import check_topk_row, f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _g(seed):
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def _check_rows(gi, gc, cap, rows):
    """rows: (b, selected oracle set, scores over the visible keys)."""
    nd = 0
    for b, sel, s in rows:
        o_idx = np.full(cap, -1, dtype=np.int64)
        o_idx[: len(sel)] = sel
        nd += check_topk_row(gi[b, 0], int(gc[b, 0]), o_idx, len(sel), s, cap)
    return nd


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("H,d", [(1, 64), (3, 32), (16, 64), (4, 128)])
def test_aggregated_routing(dtype, H, d):
    g = _g(700 + H + d)
    B, n, k = 3, 9000, 700
    n_ctx = [9000, 8999, 4321]
    K = torch.randn((H, B, n, d), generator=g).to(dtype)
    q = (torch.randn((H, B, 1, d), generator=g) / math.sqrt(d)).to(dtype)
    nc = torch.tensor(n_ctx, dtype=torch.int32, device=DEV)
    idx, counts = clsa.route_aggregated(q.to(DEV), K.to(DEV), k, n_ctx=nc, cap=k + 5)
    torch.cuda.synchronize()
    rows = []
    for b in range(B):
        sel, s = RO.aggregated_route([f64(q[h, b, 0]) for h in range(H)],
                                     [f64(K[h, b]) for h in range(H)], n_ctx[b], k)
        rows.append((b, sel, s))
    _check_rows(idx.cpu().numpy(), counts.cpu().numpy(), k + 5, rows)
    if H == 1:
        ref = clsa.route(q[0].to(DEV), K[0].to(DEV), k, n_ctx=nc, cap=k + 5)
        assert torch.equal(idx, ref[0]) and torch.equal(counts, ref[1])


def _clustered_queries(B, M, d, centers, seed, sigma=0.02):
    g = _g(seed)
    cent = torch.randn((B, centers, d), generator=g)
    lab = torch.randint(0, centers, (B, M), generator=g)
    q = torch.gather(cent, 1, lab[..., None].expand(-1, -1, d))
    return (q + sigma * torch.randn((B, M, d), generator=g)).to(torch.bfloat16)


@pytest.mark.parametrize("d,C,T", [(64, 16, 256), (128, 64, 512), (32, 8, 100)])
def test_centroid_table_build(d, C, T):
    B, M, n = 2, 640, 7000
    g = _g(720 + d)
    q = _clustered_queries(B, M, d, C, 730 + d)
    K = torch.randn((B, n, d), generator=g).to(torch.bfloat16)
    n_ctx = [7000, 6001]
    cent, table = clsa.csa_build(q.to(DEV), K.to(DEV), C, T, rounds=6,
                                 n_ctx=torch.tensor(n_ctx, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    gc = f64(cent)
    for b in range(B):
        mu = RO.kmeans(f64(q[b]), C, 6)
        assert np.max(np.abs(gc[b] - mu)) <= 2.0 ** -8 * (1.0 + np.abs(mu).max())
        tab = table[b].cpu().numpy()
        for c in range(C):  # the table rows of the GPU's own centroids
            s = O.route_scores(gc[b, c], f64(K[b]), n_ctx[b])
            sel = O.topk_select(s, T)
            o = np.full(T, -1, dtype=np.int64)
            o[: len(sel)] = sel
            check_topk_row(tab[c], len(sel), o, len(sel), s, T)


@pytest.mark.parametrize("P", [1, 4])
def test_centroid_table_lookup_buffer_ragged(P):
    B, M, n, d, C, T, k = 3, 512, 6000, 64, 32, 512, 300
    g = _g(740 + P)
    q = _clustered_queries(B, M, d, C, 750)
    K = torch.randn((B, n, d), generator=g).to(torch.bfloat16)
    n_table = 5000  # keys 5000 .. are the buffer of appended keys
    nt = torch.full((B,), n_table, dtype=torch.int32, device=DEV)
    cent, table = clsa.csa_build(q.to(DEV), K.to(DEV), C, T, rounds=4, n_ctx=nt)
    qd = q[:, ::97][:, :1].contiguous()  # decode queries: prompt queries of the clusters
    qd = (f64(qd) + 0.05 * torch.randn((B, 1, d), generator=g).double().numpy())
    qd = torch.from_numpy(qd).to(torch.bfloat16)
    n_ctx = [6000, 5500, 4800]  # the last row ends inside the table's range
    nc = torch.tensor(n_ctx, dtype=torch.int32, device=DEV)
    idx, counts = clsa.csa_route(qd.to(DEV), K.to(DEV), cent, table, n_table, P, k, n_ctx=nc,
                                 cap=k + 7)
    torch.cuda.synchronize()
    gcent, gtab = f64(cent), table.cpu().numpy()
    rows = []
    for b in range(B):
        sel, cand, s_all = RO.table_route(f64(qd)[b, 0], f64(K[b]), gcent[b], gtab[b], n_table,
                                          n_ctx[b], P, k)
        assert counts[b, 0].item() == len(sel)
        # the boundary rule over the candidates' scores
        s = np.full(n_ctx[b], -np.inf)
        s[cand] = s_all[cand]
        rows.append((b, sel, s))
    _check_rows(idx.cpu().numpy(), counts.cpu().numpy(), k + 7, rows)


@pytest.mark.timeout(600)
def test_centroid_table_decode_workload():
    """The headline decode shapes (8 x 128K keys, d_idx 64, k 2048): a table
    of 64 centroids x 2048 keys from 4096 prompt queries per sequence, probed
    at P = 3, against the oracle on the GPU's centroids and table; recall
    against the exact top-k is printed (a diagnostic, not parity)."""
    wl = gen.WORKLOADS["decode_128k_b8"]
    K_idx, u, planted = gen.gen_routing_keys(wl, DEV)
    qp = gen.gen_prompt_routing_queries(wl, u, 4096, DEV)
    n = wl.n_ctx
    nc = torch.full((wl.B,), n, dtype=torch.int32, device=DEV)
    cent, table = clsa.csa_build(qp, K_idx, 64, 2048, rounds=8, n_ctx=nc)
    q_idx = gen.gen_routing_query(wl, u, 0, DEV)
    idx, counts = clsa.csa_route(q_idx, K_idx, cent, table, n, 3, wl.k, n_ctx=nc)
    ex_idx, _ = clsa.route(q_idx, K_idx, wl.k, n_ctx=nc)
    torch.cuda.synchronize()
    gcent, gtab, gi = f64(cent), table.cpu().numpy(), idx.cpu().numpy()
    rows, recall = [], []
    for b in range(wl.B):
        Kb = f64(K_idx[b])
        sel, cand, s_all = RO.table_route(f64(q_idx)[b, 0], Kb, gcent[b], gtab[b], n, n, 3, wl.k)
        s = np.full(n, -np.inf)
        s[cand] = s_all[cand]
        rows.append((b, sel, s))
        ex = set(ex_idx[b, 0].cpu().tolist())
        recall.append(len(ex & set(gi[b, 0, : counts[b, 0].item()].tolist())) / wl.k)
    _check_rows(gi, counts.cpu().numpy(), wl.k, rows)
    print(f"centroid table router: recall of the exact top-{wl.k} per sequence "
          f"{[round(r, 3) for r in recall]} (diagnostic)", flush=True)
    del K_idx
    torch.cuda.empty_cache()


def test_router_edge_cases():
    """Degenerate sizes: a lookup whose candidates are fewer than k (every
    candidate returned, count = candidates), a build with no k-means round
    (centroids are the starting queries), aggregated routing with k at or
    above the visible keys and a sequence with no visible key."""
    g = _g(790)
    B, M, n, d, C, T = 2, 128, 3000, 32, 8, 40
    q = _clustered_queries(B, M, d, C, 791)
    K = torch.randn((B, n, d), generator=g).to(torch.bfloat16)
    cent, table = clsa.csa_build(q.to(DEV), K.to(DEV), C, T, rounds=0)
    torch.cuda.synchronize()
    first = q[:, [(c * M) // C for c in range(C)]]  # rounds = 0: the starting queries
    assert torch.equal(cent.cpu(), first)
    qd = q[:, :1].contiguous()
    idx, counts = clsa.csa_route(qd.to(DEV), K.to(DEV), cent, table, n, 1, 100, cap=110)
    torch.cuda.synchronize()
    gcent, gtab = f64(cent), table.cpu().numpy()
    rows = []
    for b in range(B):
        sel, cand, s_all = RO.table_route(f64(qd)[b, 0], f64(K[b]), gcent[b], gtab[b], n, n, 1,
                                          100)
        assert len(sel) == T and counts[b, 0].item() == T  # every candidate, fewer than k
        s = np.full(n, -np.inf)
        s[cand] = s_all[cand]
        rows.append((b, sel, s))
    _check_rows(idx.cpu().numpy(), counts.cpu().numpy(), 110, rows)
    # aggregated: k above the visible keys, and a sequence with none
    H = 3
    Ka = torch.randn((H, 3, 500, 64), generator=g).to(torch.bfloat16)
    qa = (torch.randn((H, 3, 1, 64), generator=g) / 8).to(torch.bfloat16)
    nc = torch.tensor([500, 37, 0], dtype=torch.int32, device=DEV)
    ia, ca = clsa.route_aggregated(qa.to(DEV), Ka.to(DEV), 64, n_ctx=nc, cap=64)
    torch.cuda.synchronize()
    assert ca[:, 0].cpu().tolist() == [64, 37, 0]
    assert ia[1, 0, :37].cpu().tolist() == list(range(37)) and bool((ia[1, 0, 37:] == -1).all())
    assert bool((ia[2, 0] == -1).all())
    sel, s = RO.aggregated_route([f64(qa[h, 0, 0]) for h in range(H)],
                                 [f64(Ka[h, 0]) for h in range(H)], 500, 64)
    _check_rows(ia.cpu().numpy(), ca.cpu().numpy(), 64, [(0, sel, s)])
