"""Independent calls on two streams at once.

The library keeps no state between calls: every call works in the
caller's workspace and writes only its own outputs.  So calls with their
own buffers may run concurrently on different streams.  Two decode steps
(routing, then attention over the lists), a prefill-chunk routing call and
a threshold routing call are launched on two streams with no
synchronization between them, three times over, and every output must
equal the same calls run one after another on one stream, bit for bit.
"""
from __future__ import annotations

import pytest
import torch

from long_context_sparse_routing_amd import binding as clsa
from long_context_sparse_routing_amd import inputs as gen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _decode_calls(seed, B, n, L, k):
    wl = gen.WORKLOADS["decode_32k"].with_(B=B, n_ctx=n, n_cap=n, L=L, k=k, planted=32)
    K_idx, u, _ = gen.gen_routing_keys(wl, DEV, seed=seed)
    Kc, Vc = gen.gen_kv(wl, DEV, seed=seed + 1)
    q_idx = gen.gen_routing_query(wl, u, 0, DEV, seed=seed + 2)
    q = gen.gen_attn_query(wl, q_idx, 0, DEV, seed=seed + 3)
    nc = torch.tensor([n - 7 * b for b in range(B)], dtype=torch.int32, device=DEV)
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
    counts = torch.empty((B, 1), dtype=torch.int32, device=DEV)
    out = torch.empty((L, B, 1, wl.Hq, wl.D), dtype=torch.bfloat16, device=DEV)
    keep = (K_idx, Kc, Vc, q_idx, q, nc)

    def calls(stream):
        return [clsa.prepare_route(q_idx, K_idx, k, n_ctx=nc, idx=idx, counts=counts,
                                   stream=stream),
                clsa.prepare_sparse_attn(q, Kc, Vc, idx, counts, out=out, stream=stream)]
    return calls, [idx, counts, out], keep


def _prefill_calls(seed):
    g = torch.Generator()
    g.manual_seed(seed)
    B, M, n, d, k = 1, 256, 12000, 64, 1024
    K = torch.randn((B, n, d), generator=g).to(torch.bfloat16).to(DEV)
    Q = (torch.randn((B, M, d), generator=g) / 8).to(torch.bfloat16).to(DEV)
    idx = torch.empty((B, M, k), dtype=torch.int32, device=DEV)
    counts = torch.empty((B, M), dtype=torch.int32, device=DEV)

    def calls(stream):
        return [clsa.prepare_route(Q, K, k, q_pos0=n - M, idx=idx, counts=counts, stream=stream)]
    return calls, [idx, counts], (K, Q)


def _threshold_calls(seed):
    g = torch.Generator()
    g.manual_seed(seed)
    B, n, d, cap = 4, 40000, 128, 4096
    K = torch.randn((B, n, d), generator=g).to(torch.bfloat16).to(DEV)
    q = (torch.randn((B, 1, d), generator=g) / 11).to(torch.bfloat16).to(DEV)
    tau = torch.tensor([[1.6], [1.8], [2.0], [2.2]], dtype=torch.float32, device=DEV)
    idx = torch.empty((B, 1, cap), dtype=torch.int32, device=DEV)
    counts = torch.empty((B, 1), dtype=torch.int32, device=DEV)

    def calls(stream):
        return [clsa.prepare_route_threshold(q, K, tau, cap, idx=idx, counts=counts,
                                             stream=stream)]
    return calls, [idx, counts], (K, q, tau)


def test_two_streams_match_one_stream():
    jobs = [_decode_calls(11, 3, 20000, 4, 2048), _decode_calls(21, 2, 30000, 2, 1024),
            _prefill_calls(31), _threshold_calls(41)]
    s0 = torch.cuda.current_stream()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    # the calls are prepared (buffers and workspaces allocated) before any
    # of them runs; each job keeps its buffers for every run
    one = [mk(s0) for mk, _, _ in jobs]
    two = [mk(sa if i % 2 == 0 else sb) for i, (mk, _, _) in enumerate(jobs)]
    for cs in one:
        for c in cs:
            c()
    torch.cuda.synchronize()
    ref = [[t.clone() for t in outs] for _, outs, _ in jobs]
    assert int(ref[0][1].min()) == 2048 and int(ref[1][1].min()) == 1024
    for rep in range(3):
        for _, outs, _ in jobs:
            for t in outs:
                t.fill_(-7 if t.dtype == torch.int32 else 0)
        torch.cuda.synchronize()
        # interleave the jobs' launches over the two streams
        for step in range(2):
            for cs in two:
                if step < len(cs):
                    cs[step]()
        torch.cuda.synchronize()
        for j, (_, outs, _) in enumerate(jobs):
            for t, r in zip(outs, ref[j]):
                assert torch.equal(t, r), f"run {rep}: job {j} differs from the one-stream run"
