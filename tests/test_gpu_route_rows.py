"""GPU parity of routing for rows whose keys no other row shares (bf16,
k <= 2048, up to 512K keys: a sampled per-row lower bound of the k-th
score, one filtered scan, the exact select of the candidates) at the edges
of that path, against the CPU oracle.

Acceptance as in test_gpu_parity: equal counts, ascending lists with -1
padding, index sets identical except at boundary pairs whose oracle scores
lie within 1e-5 relative of the c-th largest score.
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
    for b, m in rows:
        nv = O.visible_count(n_ctx[b], q_pos0, m)
        s = O.route_scores(q_np[b, m], K_np[b], nv)
        sel = O.topk_select(s, k)
        o_idx = np.full(cap, -1)
        o_idx[: len(sel)] = sel
        check_topk_row(gi[b, m], int(gc[b, m]), o_idx, len(sel), s, cap)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("k", [300, 2048])
def test_causal_query_rows_below_block_size(d, k):
    # 16 causal query rows per sequence (a few tokens decoded at once):
    # fewer than a matrix-core block, so every row is routed on its own
    g = _gen(500 + d + k)
    B, M, n = 2, 16, 20000
    n_ctx = [n, n - 9]
    K = torch.randn((B, n, d), generator=g).to(torch.bfloat16)
    q = (torch.randn((B, M, d), generator=g) / math.sqrt(d)).to(torch.bfloat16)
    nc = torch.tensor(n_ctx, dtype=torch.int32, device=DEV)
    idx, counts = clsa.route(q.to(DEV), K.to(DEV), k, n_ctx=nc, q_pos0=n - M, cap=k + 4)
    torch.cuda.synchronize()
    _check(idx, counts, q, K, n_ctx, n - M, k, k + 4)


@pytest.mark.parametrize("n", [2049, 2100, 4095, 4096, 4097, 8191, 8193])
def test_context_lengths_around_the_sample_size(n):
    # every key is a sample up to 4096 keys, then evenly spaced samples;
    # just above k the bound keeps every key
    g = _gen(600 + n)
    K = torch.randn((3, n, 64), generator=g).to(torch.bfloat16)
    q = (torch.randn((3, 1, 64), generator=g) / 8).to(torch.bfloat16)
    n_ctx = [n, n - 1, n // 2 + 1]
    nc = torch.tensor(n_ctx, dtype=torch.int32, device=DEV)
    idx, counts = clsa.route(q.to(DEV), K.to(DEV), 2048, n_ctx=nc)
    torch.cuda.synchronize()
    _check(idx, counts, q, K, n_ctx, -1, 2048, 2048)


@pytest.mark.parametrize("n_cap", [524288, 524289])
def test_largest_context_of_the_path_and_past_it(n_cap):
    # 512K keys is the largest context the sampled path takes; one more key
    # goes to the exhaustive path.  Both must agree with the oracle.
    g = _gen(700 + n_cap % 7)
    K = torch.randn((1, n_cap, 64), generator=g).to(torch.bfloat16)
    q = (torch.randn((1, 1, 64), generator=g) / 8).to(torch.bfloat16)
    idx, counts = clsa.route(q.to(DEV), K.to(DEV), 2048)
    torch.cuda.synchronize()
    _check(idx, counts, q, K, [n_cap], -1, 2048, 2048)


def test_many_sequences_one_launch():
    # 40 sequences of different lengths in one call
    g = _gen(800)
    B, n = 40, 12000
    n_ctx = [n - 250 * b for b in range(B)]
    K = torch.randn((B, n, 64), generator=g).to(torch.bfloat16)
    q = (torch.randn((B, 1, 64), generator=g) / 8).to(torch.bfloat16)
    nc = torch.tensor(n_ctx, dtype=torch.int32, device=DEV)
    idx, counts = clsa.route(q.to(DEV), K.to(DEV), 1024, n_ctx=nc)
    torch.cuda.synchronize()
    _check(idx, counts, q, K, n_ctx, -1, 1024, 1024, rows=[(b, 0) for b in range(0, B, 3)])


def test_many_sequences_take_the_longest_chunks():
    # 32 sequences x 64K keys: enough rows for the score pass to take its
    # longest chunks (2048 keys); ragged contexts end inside a chunk, on a
    # chunk boundary and one key past it
    g = _gen(900)
    B, n = 32, 65536
    n_ctx = [n - 977 * (b % 7) for b in range(B)]
    n_ctx[3], n_ctx[4] = 6 * 2048, 6 * 2048 + 1
    K = torch.randn((B, n, 64), generator=g).to(torch.bfloat16)
    q = (torch.randn((B, 1, 64), generator=g) / 8).to(torch.bfloat16)
    nc = torch.tensor(n_ctx, dtype=torch.int32, device=DEV)
    idx, counts = clsa.route(q.to(DEV), K.to(DEV), 2048, n_ctx=nc)
    torch.cuda.synchronize()
    for b in (0, 3, 4, 13, 31):  # one sequence at a time: the host copy stays small
        _check(idx[b:b + 1], counts[b:b + 1], q[b:b + 1], K[b:b + 1], [n_ctx[b]], -1, 2048, 2048)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_empty_and_tiny_contexts(dtype):
    # contexts of 0 and 1 keys, one below, at and above k, and a long one,
    # in one call (the sampled path for bf16, the exhaustive one for fp32);
    # then k = 1
    g = _gen(950)
    n = 50000
    n_ctx = [0, 1, 2047, 2048, 2049, n]
    B = len(n_ctx)
    K = torch.randn((B, n, 64), generator=g).to(dtype)
    q = (torch.randn((B, 1, 64), generator=g) / 8).to(dtype)
    nc = torch.tensor(n_ctx, dtype=torch.int32, device=DEV)
    idx, counts = clsa.route(q.to(DEV), K.to(DEV), 2048, n_ctx=nc, cap=2050)
    torch.cuda.synchronize()
    assert counts[:, 0].cpu().tolist() == [0, 1, 2047, 2048, 2048, 2048]
    assert bool((idx[0] == -1).all()) and idx[1, 0, 0].item() == 0
    _check(idx, counts, q, K, n_ctx, -1, 2048, 2050)
    idx1, counts1 = clsa.route(q.to(DEV), K.to(DEV), 1, n_ctx=nc, cap=3)
    torch.cuda.synchronize()
    assert counts1[:, 0].cpu().tolist() == [0, 1, 1, 1, 1, 1]
    _check(idx1, counts1, q, K, n_ctx, -1, 1, 3)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_most_sequences_one_call(dtype):
    # B = 65535 sequences of one query each, the call's row limit, with
    # contexts of 0 .. 300 keys (below, at and above k); checked on the
    # first, the last and a spread of sequences between
    gd = torch.Generator(device=DEV)
    gd.manual_seed(970)
    B, n, d, k = 65535, 300, 32, 16
    K = torch.randn((B, n, d), generator=gd, device=DEV).to(dtype)
    q = (torch.randn((B, 1, d), generator=gd, device=DEV) / 6).to(dtype)
    n_ctx = [b % (n + 1) for b in range(B)]
    nc = torch.tensor(n_ctx, dtype=torch.int32, device=DEV)
    idx, counts = clsa.route(q, K, k, n_ctx=nc)
    torch.cuda.synchronize()
    bs = sorted({0, 1, 15, 16, 17, 300, 301, B - 2, B - 1, *range(7, B, 613)})
    sel = torch.tensor(bs, device=DEV)
    _check(idx[sel], counts[sel], q[sel].cpu(), K[sel].cpu(), [n_ctx[b] for b in bs], -1, k, k)
    assert len(bs) >= 100


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_context_lengths_outside_the_cache(dtype):
    # context lengths below 0 see no key and lengths above n_cap every key
    # (the oracle's reading R25), in one call with ordinary ones
    g = _gen(980)
    n = 9000
    n_ctx = [-1, -(2 ** 31), n + 1, 2 ** 31 - 1, 0, n]
    B = len(n_ctx)
    K = torch.randn((B, n, 64), generator=g).to(dtype)
    q = (torch.randn((B, 1, 64), generator=g) / 8).to(dtype)
    nc = torch.tensor(n_ctx, dtype=torch.int32, device=DEV)
    idx, counts = clsa.route(q.to(DEV), K.to(DEV), 2048, n_ctx=nc, cap=2050)
    torch.cuda.synchronize()
    assert counts[:, 0].cpu().tolist() == [0, 0, 2048, 2048, 0, 2048]
    _check(idx, counts, q, K, n_ctx, -1, 2048, 2050)
