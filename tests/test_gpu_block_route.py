"""GPU parity of block routing (many query rows per sequence, bf16, scores on
the matrix cores) against the CPU oracle.

Acceptance (as for the one-query path): equal counts, ascending lists with
-1 padding, index sets identical except at boundary pairs whose oracle
scores lie within 1e-5 relative of the c-th largest score; where identical
key rows create exact ties the sets must be identical.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from long_context_sparse_routing_amd import binding as clsa
from oracle import clsa_oracle as O
from tests.parity_util import check_topk_row, f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _gen(seed):
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def _check(idx, counts, q, K, n_ctx, q_pos0, k, cap, rows=None):
    q_np, K_np = f64(q), f64(K)
    B, M = q.shape[0], q.shape[1]
    rows = rows if rows is not None else [(b, m) for b in range(B) for m in range(M)]
    gi, gc = idx.cpu().numpy(), counts.cpu().numpy()
    ndiff = 0
    for b, m in rows:
        nv = O.visible_count(n_ctx[b], q_pos0, m)
        s = O.route_scores(q_np[b, m], K_np[b], nv)
        sel = O.topk_select(s, k)
        o_idx = np.full(cap, -1)
        o_idx[: len(sel)] = sel
        ndiff += check_topk_row(gi[b, m], int(gc[b, m]), o_idx, len(sel), s, cap)
    return ndiff


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("M,n,k,q_pos0", [
    (64, 100, 1, -1),         # one chunk, ragged tail
    (64, 5000, 256, -1),      # several chunks
    (100, 3000, 300, 2950),   # causal: row m sees min(n_ctx, 2951 + m) keys
    (100, 5000, 50, 0),       # causal from position 0: early rows take every key
    (130, 20000, 2048, 19900),
    (300, 70001, 2048, -1),   # several filter workgroups per chunk column
])
def test_block_route_shapes(d, M, n, k, q_pos0):
    g = _gen(100 + d + M + n + k)
    B = 2
    n_ctx = [n, n - 37]
    K = torch.randn((B, n, d), generator=g).to(torch.bfloat16)
    q = (torch.randn((B, M, d), generator=g) / math.sqrt(d)).to(torch.bfloat16)
    nc = torch.tensor(n_ctx, dtype=torch.int32, device=DEV)
    cap = k + 5
    idx, counts = clsa.route(q.to(DEV), K.to(DEV), k, n_ctx=nc, q_pos0=q_pos0, cap=cap)
    torch.cuda.synchronize()
    rows = None
    if n * M > 2_000_000:  # sampled rows: edges, slab boundaries, the ragged tail
        ms = sorted({0, 1, 31, 32, 63, 64, 255, 256, M // 2, M - 2, M - 1} & set(range(M)))
        rows = [(b, m) for b in range(B) for m in ms]
    _check(idx, counts, q, K, n_ctx, q_pos0, k, cap, rows)


def test_block_route_exact_ties_lower_index_wins():
    g = _gen(201)
    base = torch.randn((29, 64), generator=g).to(torch.bfloat16)
    K = base[torch.randint(0, 29, (1, 30000), generator=g)]
    q = (torch.randn((1, 96, 64), generator=g) / 8).to(torch.bfloat16)
    for k in (1, 700, 2048):
        idx, counts = clsa.route(q.to(DEV), K.to(DEV), k)
        assert _check(idx, counts, q, K, [30000], -1, k, k) == 0


@pytest.mark.parametrize("n", [3000, 20000])
def test_block_route_zero_query_takes_lowest_positions(n):
    # every score is exactly 0: all keys are candidates (n = 3000 fits the
    # candidate buffer, n = 20000 overflows it and is rescanned)
    K = torch.randn((1, n, 32), generator=_gen(202)).to(torch.bfloat16)
    q = torch.zeros((1, 64, 32), dtype=torch.bfloat16)
    for k in (100, 2048):
        idx, counts = clsa.route(q.to(DEV), K.to(DEV), k)
        gi = idx.cpu().numpy()
        assert np.all(counts.cpu().numpy() == k)
        assert np.all(gi[0, :, :k] == np.arange(k)[None, :])


def test_block_route_sampled_keys_outliers_force_rescan():
    # keys at the sampled positions (multiples of 32) score far above all
    # others, so the sampled threshold keeps fewer than k keys and every
    # row falls back to the exact rescan
    g = _gen(203)
    n, d, M = 40000, 64, 64
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    K = 0.05 * torch.randn((1, n, d), generator=g)
    K[0, ::32] = 3.0 * u + 0.2 * torch.randn((len(range(0, n, 32)), d), generator=g)
    q = (u[None, None, :] + 0.1 * torch.randn((1, M, d), generator=g)).to(torch.bfloat16)
    K = K.to(torch.bfloat16)
    idx, counts = clsa.route(q.to(DEV), K.to(DEV), 2048)
    assert _check(idx, counts, q, K, [n], -1, 2048, 2048) <= 4 * M


def test_block_route_run_twice_bitwise_identical():
    g = _gen(204)
    K = torch.randn((2, 50000, 128), generator=g).to(torch.bfloat16).to(DEV)
    q = (torch.randn((2, 200, 128), generator=g) / 11).to(torch.bfloat16).to(DEV)
    a = [t.clone() for t in clsa.route(q, K, 2048, q_pos0=49800)]
    b = [t.clone() for t in clsa.route(q, K, 2048, q_pos0=49800)]
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("d,M,n,k,q_pos0", [
    (64, 65, 2047, 100, -1),      # one key short of a full sub-chunk; 65 rows: a partial slab
    (64, 130, 2048, 2048, -1),    # k = n: every key, exactly one sub-chunk
    (64, 64, 2049, 300, -1),      # one key into the next sub-chunk
    (64, 96, 8193, 1000, 8150),   # one key into the next segment chunk; causal tail
    (32, 200, 5000, 2048, 1000),  # causal from mid-chunk: early rows see < k keys
    (128, 70, 3000, 64, 2930),    # d = 128 (256-key sub-chunks)
])
def test_block_route_chunk_edges(d, M, n, k, q_pos0):
    g = _gen(400 + d + M + n)
    B = 3
    n_ctx = [n, max(n - 5, 1), n // 2 + 1]
    K = torch.randn((B, n, d), generator=g).to(torch.bfloat16)
    q = (torch.randn((B, M, d), generator=g) / math.sqrt(d)).to(torch.bfloat16)
    nc = torch.tensor(n_ctx, dtype=torch.int32, device=DEV)
    idx, counts = clsa.route(q.to(DEV), K.to(DEV), k, n_ctx=nc, q_pos0=q_pos0, cap=k + 1)
    torch.cuda.synchronize()
    rows = [(b, m) for b in range(B) for m in sorted({0, 1, 31, 32, 63, 64, M // 2, M - 1})
            if m < M]
    _check(idx, counts, q, K, n_ctx, q_pos0, k, k + 1, rows)


def test_block_route_workload_rows_sampled_across_the_chunk():
    # the benchmark's prefill configuration: rows from every 512-row group
    from long_context_sparse_routing_amd import inputs as gen
    wl = gen.WORKLOADS["prefill_128k_c4096"]
    K_idx, u, _ = gen.gen_routing_keys(wl, DEV)
    q_idx = gen.gen_routing_query(wl, u, 0, DEV)
    idx, counts = clsa.route(q_idx, K_idx, wl.k, q_pos0=wl.q_pos0)
    torch.cuda.synchronize()
    rows = [(0, m) for m in range(3, wl.M, 509)]
    nd = _check(idx, counts, q_idx.cpu(), K_idx.cpu(), [wl.n_ctx], wl.q_pos0, wl.k, wl.k, rows)
    assert nd <= 2 * len(rows)
    del K_idx
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M", [1, 64])
def test_route_empty_middle_segments(M):
    # keys in the middle of the context score about 0, far below every row's
    # threshold, so the chunks there hold no candidates and the select walks
    # its candidate runs across several empty segments (M = 1: decode rows,
    # 256-key chunks; M = 64: block routing, 2048-key chunks)
    g = _gen(500 + M)
    B, n, d, k = 2, 20000, 64, 512
    K = torch.randn((B, n, d), generator=g)
    K[:, 6000:14500] *= 1e-3
    K = K.to(torch.bfloat16)
    q = (torch.randn((B, M, d), generator=g) / math.sqrt(d)).to(torch.bfloat16)
    idx, counts = clsa.route(q.to(DEV), K.to(DEV), k)
    torch.cuda.synchronize()
    _check(idx, counts, q, K, [n, n], -1, k, k)
    assert not bool(((idx >= 6000) & (idx < 14500)).any())


def test_block_route_most_rows():
    # B*M = 65535 rows, the call's limit, in one causal block from position
    # 0: early rows keep every visible key, rows past 8191 the top 64 of 8192
    g = _gen(600)
    M, n, d, k = 65535, 8192, 64, 64
    K = torch.randn((1, n, d), generator=g).to(torch.bfloat16)
    q = (torch.randn((1, M, d), generator=g) / math.sqrt(d)).to(torch.bfloat16)
    idx, counts = clsa.route(q.to(DEV), K.to(DEV), k, q_pos0=0)
    torch.cuda.synchronize()
    assert counts[0, :64].cpu().tolist() == list(range(1, 65))
    ms = sorted({0, 1, 62, 63, 64, 255, 256, 8190, 8191, 8192, M - 2, M - 1,
                 *range(5, M, 997)})
    _check(idx, counts, q, K, [n], 0, k, k, [(0, m) for m in ms])


def test_block_route_context_lengths_outside_the_cache():
    # a block of causal rows whose sequences report context lengths below 0
    # (no key) or above n_cap (every key up to the row's position), as the
    # oracle's reading R25 takes them
    g = _gen(700)
    B, M, n, d, k = 3, 64, 5000, 64, 300
    n_ctx = [-7, n + 1000, 2 ** 31 - 1]
    K = torch.randn((B, n, d), generator=g).to(torch.bfloat16)
    q = (torch.randn((B, M, d), generator=g) / math.sqrt(d)).to(torch.bfloat16)
    nc = torch.tensor(n_ctx, dtype=torch.int32, device=DEV)
    idx, counts = clsa.route(q.to(DEV), K.to(DEV), k, n_ctx=nc, q_pos0=4950, cap=k)
    torch.cuda.synchronize()
    assert bool((counts[0] == 0).all()) and bool((idx[0] == -1).all())
    _check(idx, counts, q, K, n_ctx, 4950, k, k)
