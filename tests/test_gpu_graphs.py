"""The library's calls under HIP graph capture.

Every call takes its workspace from the caller, clears what must start at
zero with kernels (no memset nodes) and never synchronizes, so a step can be
captured once and replayed.  Each test captures a step, replays it several
times with other eager calls and synchronizations in between, clears the
outputs before each replay, and checks every replay bit for bit against the
same calls run eagerly: the kernels and inputs are the same, so the results
must be identical.  Covered: the decode step (append, sampled-filter
routing, a multi-layer attention call and single-layer calls, both with
split lists and the combine kernel), block routing of a prefill chunk,
threshold routing, and the allocation-free routing call.
"""
from __future__ import annotations

import pytest
import torch

from long_context_sparse_routing_amd import binding as clsa
from long_context_sparse_routing_amd import inputs as gen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REPLAYS = 3


def _capture(calls, stream):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in calls:
            c()
    return g


def _eager(calls, stream):
    with torch.cuda.stream(stream):
        for c in calls:
            c()
    stream.synchronize()


def _replays_match(g, stream, outputs, ref, between):
    for i in range(REPLAYS):
        for t in outputs:  # the replay must write every output again
            t.fill_(-7 if t.dtype == torch.int32 else 0)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        stream.synchronize()
        for t, r in zip(outputs, ref):
            assert torch.equal(t, r), f"replay {i} differs from the eager run"
        between()  # the program's own eager work between replays
        torch.cuda.synchronize()


def test_decode_step_graph_replays():
    wl = gen.WORKLOADS["decode_32k"].with_(B=4, n_ctx=20000, n_cap=20008, L=4, k=2048,
                                           planted=64)
    K_idx, u, _ = gen.gen_routing_keys(wl, DEV)
    Kc, Vc = gen.gen_kv(wl, DEV)
    new_kidx, new_k, new_v = gen.gen_append_rows(wl, 1, DEV)
    n_ctx = [20001, 19000, 12345, 4097]
    nc = torch.tensor(n_ctx, dtype=torch.int32, device=DEV)
    pos = torch.tensor([n - 1 for n in n_ctx], dtype=torch.int32, device=DEV)
    q_idx = gen.gen_routing_query(wl, u, 0, DEV)
    q = gen.gen_attn_query(wl, q_idx, 0, DEV)
    s = torch.cuda.Stream()
    idx = torch.empty((wl.B, 1, wl.k), dtype=torch.int32, device=DEV)
    counts = torch.empty((wl.B, 1), dtype=torch.int32, device=DEV)
    out_all = torch.empty((wl.L, wl.B, 1, wl.Hq, wl.D), dtype=torch.bfloat16, device=DEV)
    out_one = torch.empty_like(out_all)
    # the whole-step call and one call per layer (both split each list over
    # several workgroups and merge them with the combine kernel)
    ws_one = torch.empty(max(1, clsa.sparse_attn_workspace_size(1, wl.B, 1, wl.Hq, wl.Hkv, wl.D,
                                                                 wl.k, torch.bfloat16)),
                         dtype=torch.uint8, device=DEV)
    calls = [clsa.prepare_kv_append(pos, new_kidx[0], K_idx, new_k[0], Kc, new_v[0], Vc, stream=s),
             clsa.prepare_route(q_idx, K_idx, wl.k, n_ctx=nc, idx=idx, counts=counts, stream=s),
             clsa.prepare_sparse_attn(q, Kc, Vc, idx, counts, out=out_all, stream=s)]
    calls += [clsa.prepare_sparse_attn([q[l]], [Kc[l]], [Vc[l]], idx, counts, out=[out_one[l]],
                                       ws=ws_one, stream=s) for l in range(wl.L)]
    _eager(calls, s)
    ref = [idx.clone(), counts.clone(), out_all.clone(), out_one.clone()]
    assert int(counts.min()) == wl.k
    g = _capture(calls, s)
    other_q = gen.gen_routing_query(wl, u, 5, DEV)

    def between():  # a different routing call on other buffers, eagerly
        clsa.route(other_q, K_idx, wl.k, n_ctx=nc)
        torch.cuda.synchronize()

    _replays_match(g, s, [idx, counts, out_all, out_one], ref, between)
    del K_idx, Kc, Vc


def test_block_and_threshold_routing_graph_replays():
    g0 = torch.Generator()
    g0.manual_seed(71)
    B, M, n, d = 1, 256, 9000, 64
    K = torch.randn((B, n, d), generator=g0).to(torch.bfloat16).to(DEV)
    Q = (torch.randn((B, M, d), generator=g0) / 8).to(torch.bfloat16).to(DEV)
    tau = torch.full((B, M), 0.25, dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    idx_b = torch.empty((B, M, 512), dtype=torch.int32, device=DEV)
    cnt_b = torch.empty((B, M), dtype=torch.int32, device=DEV)
    idx_t = torch.empty((B, M, 4096), dtype=torch.int32, device=DEV)
    cnt_t = torch.empty((B, M), dtype=torch.int32, device=DEV)
    calls = [clsa.prepare_route(Q, K, 512, q_pos0=n - M, idx=idx_b, counts=cnt_b, stream=s),
             clsa.prepare_route_threshold(Q, K, tau, 4096, q_pos0=n - M, idx=idx_t, counts=cnt_t,
                                          stream=s)]
    _eager(calls, s)
    ref = [idx_b.clone(), cnt_b.clone(), idx_t.clone(), cnt_t.clone()]
    g = _capture(calls, s)
    Q2 = (torch.randn((B, M, d), generator=g0) / 8).to(torch.bfloat16).to(DEV)

    def between():
        clsa.route(Q2, K, 512, q_pos0=n - M)
        torch.cuda.synchronize()

    _replays_match(g, s, [idx_b, cnt_b, idx_t, cnt_t], ref, between)


def test_static_routing_graph_replays():
    # the allocation-free call is the one meant for capture: its scratch is
    # the library's own array, so nothing is allocated while capturing
    wl = gen.WORKLOADS["decode_32k"].with_(B=3, n_ctx=30000, n_cap=30000, L=1, planted=32)
    K_idx, u, _ = gen.gen_routing_keys(wl, DEV)
    q_idx = gen.gen_routing_query(wl, u, 0, DEV)
    nc = torch.tensor([30000, 22222, 5000], dtype=torch.int32, device=DEV)
    s = torch.cuda.Stream()
    idx = torch.empty((wl.B, 1, wl.k), dtype=torch.int32, device=DEV)
    counts = torch.empty((wl.B, 1), dtype=torch.int32, device=DEV)
    calls = [clsa.prepare_route_static(q_idx, K_idx, wl.k, n_ctx=nc, idx=idx, counts=counts,
                                       stream=s)]
    _eager(calls, s)
    ref = [idx.clone(), counts.clone()]
    want, _ = clsa.route(q_idx, K_idx, wl.k, n_ctx=nc)
    torch.cuda.synchronize()
    assert torch.equal(ref[0], want)
    g = _capture(calls, s)
    q2 = gen.gen_routing_query(wl, u, 3, DEV)

    def between():  # another static call overwrites the shared scratch array
        clsa.route_static(q2, K_idx, wl.k, n_ctx=nc)
        torch.cuda.synchronize()

    _replays_match(g, s, [idx, counts], ref, between)
    del K_idx
