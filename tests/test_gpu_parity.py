"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Acceptance rules:
  * top-k index sets: equal counts, ascending, -1 padded; sets identical
    except at boundary pairs whose oracle scores are within 1e-5 relative
    of the c-th largest score (GPU scores accumulate in fp32, the oracle's
    are exact in fp64);
  * threshold sets: identical, zero false negatives (inputs keep every
    score at least 1e-4 away from tau);
  * attention: max abs error <= 2e-2 for bf16 K/V and <= 1e-4 for fp32,
    with the oracle attending over the GPU's own index lists (so the check
    runs whatever routing chose at near-ties); the full workloads also
    compare a few rows end to end on the oracle's own lists.
Small cases are compared element by element; the full-size workloads run
in the benchmark's launch configuration and are compared on every routed
row and, for attention, on every row of decode steps and 64 rows of the
prefill chunk, in all 16 layers.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from long_context_sparse_routing_amd import binding as clsa
from long_context_sparse_routing_amd import inputs as gen
from oracle import clsa_oracle as O
from tests.parity_util import (ATOL, attn_vs_oracle, check_topk_row, check_topk_rows, f64,
                               lazy_layers)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _cpu_gen(seed):
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def _oracle_topk_rows(q_np, K_np, n_ctx, q_pos0, k, cap, rows):
    res = {}
    for b, m in rows:
        nv = O.visible_count(n_ctx[b], q_pos0, m)
        s = O.route_scores(q_np[b, m], K_np[b], nv)
        sel = O.topk_select(s, k)
        res[(b, m)] = (sel, s)
    return res


def _check_route(idx, counts, q, K, n_ctx, q_pos0, k, cap, rows=None):
    q_np, K_np = f64(q), f64(K)
    B, M = q.shape[0], q.shape[1]
    rows = rows if rows is not None else [(b, m) for b in range(B) for m in range(M)]
    gi = idx.cpu().numpy()
    gc = counts.cpu().numpy()
    ndiff = 0
    for (b, m), (sel, s) in _oracle_topk_rows(q_np, K_np, n_ctx, q_pos0, k, cap, rows).items():
        o_idx = np.full(cap, -1)
        o_idx[: len(sel)] = sel
        ndiff += check_topk_row(gi[b, m], int(gc[b, m]), o_idx, len(sel), s, cap)
    return ndiff


# ------------------------------------------------------------------ routing
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("n,k", [(1, 1), (17, 5), (5000, 256), (70001, 2048)])
def test_route_topk_shapes(dtype, d, n, k):
    g = _cpu_gen(7 + d + n)
    B = 3
    n_ctx = [n, max(n - 3, 0), n // 2]
    K = torch.randn((B, n, d), generator=g).to(dtype)
    q = (torch.randn((B, 1, d), generator=g) / math.sqrt(d)).to(dtype)
    nc = torch.tensor(n_ctx, dtype=torch.int32)
    idx, counts = clsa.route(q.to(DEV), K.to(DEV), k, n_ctx=nc.to(DEV), cap=k + 3)
    torch.cuda.synchronize()
    _check_route(idx, counts, q, K, n_ctx, -1, k, k + 3)


def test_route_exact_ties_lower_index_wins():
    g = _cpu_gen(11)
    base = torch.randn((37, 64), generator=g).to(torch.bfloat16)
    pick = torch.randint(0, 37, (2, 20000), generator=g)
    K = base[pick]  # [2, 20000, 64]: many identical rows, so exact score ties
    q = (torch.randn((2, 1, 64), generator=g) / 8).to(torch.bfloat16)
    for k in (1, 999, 1000, 7777):
        idx, counts = clsa.route(q.to(DEV), K.to(DEV), k)
        ndiff = _check_route(idx, counts, q, K, [20000, 20000], -1, k, k)
        assert ndiff == 0  # identical rows score identically: the tie rule decides


def test_route_zero_query_takes_lowest_positions():
    K = torch.randn((2, 3000, 32), generator=_cpu_gen(12))
    q = torch.zeros((2, 1, 32))
    q[1, 0, 0] = -0.0
    idx, counts = clsa.route(q.to(DEV), K.to(DEV), 100, cap=128)
    gi = idx.cpu().numpy()
    for b in range(2):
        assert gi[b, 0, :100].tolist() == list(range(100))
        assert np.all(gi[b, 0, 100:] == -1)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_route_degenerate_bucket_uses_global_select(dtype):
    # every score lies in one histogram bucket ([2, 2.5)), with only 64 distinct
    # bf16 values: more candidates than the LDS select holds, and exact ties
    g = _cpu_gen(17)
    B, N = 2, 20000
    K = torch.zeros((B, N, 32))
    K[:, :, 0] = 2.0 + 0.49 * torch.rand((B, N), generator=g)
    K[:, :, 1:] = 0.01 * torch.randn((B, N, 31), generator=g)
    K = K.to(torch.bfloat16).to(dtype)
    q = torch.zeros((B, 1, 32), dtype=dtype)
    q[:, 0, 0] = 1.0
    for k in (1, 2048, 9999):
        idx, counts = clsa.route(q.to(DEV), K.to(DEV), k)
        assert _check_route(idx, counts, q, K, [N, N], -1, k, k) == 0  # exact scores
    q0 = torch.zeros((B, 1, 32), dtype=dtype)  # all scores exactly 0
    idx, counts = clsa.route(q0.to(DEV), K.to(DEV), 7000)
    assert idx.cpu()[:, 0].tolist() == [list(range(7000))] * B


@pytest.mark.parametrize("n", [3000, 20000])
def test_route_bf16_zero_query_takes_lowest_positions(n):
    # bf16 decode rows with k <= 2048 take the sampled-threshold path; every
    # score is exactly 0, so every key passes the threshold (n = 3000 fits
    # the select, n = 20000 overflows it and the row is rescanned)
    K = torch.randn((2, n, 64), generator=_cpu_gen(15)).to(torch.bfloat16)
    q = torch.zeros((2, 1, 64), dtype=torch.bfloat16)
    for k in (100, 2048):
        idx, counts = clsa.route(q.to(DEV), K.to(DEV), k, cap=k + 2)
        gi = idx.cpu().numpy()
        assert np.all(counts.cpu().numpy() == k)
        assert np.all(gi[:, 0, :k] == np.arange(k)[None, :])
        assert np.all(gi[:, 0, k:] == -1)


def test_route_decode_sampled_outliers_force_rescan():
    # the keys the threshold samples (positions floor(i n / 4096)) score far
    # above the rest, so the sampled bound keeps fewer than k keys and each
    # row is redone by the exact rescan
    g = _cpu_gen(16)
    B, n, d = 2, 40000, 64
    at = torch.arange(4096, dtype=torch.int64) * n // 4096
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    K = 0.05 * torch.randn((B, n, d), generator=g)
    K[:, at] = 3.0 * u + 0.2 * torch.randn((B, len(at), d), generator=g)
    q = (u[None, None, :] + 0.1 * torch.randn((B, 1, d), generator=g)).to(torch.bfloat16)
    K = K.to(torch.bfloat16)
    idx, counts = clsa.route(q.to(DEV), K.to(DEV), 2048)
    assert _check_route(idx, counts, q, K, [n, n], -1, 2048, 2048) <= 4


def test_route_prefill_causal_rows():
    g = _cpu_gen(13)
    K = torch.randn((2, 3000, 64), generator=g).to(torch.bfloat16)
    q = (torch.randn((2, 70, 64), generator=g) / 8).to(torch.bfloat16)
    n_ctx = [3000, 2950]
    nc = torch.tensor(n_ctx, dtype=torch.int32, device=DEV)
    idx, counts = clsa.route(q.to(DEV), K.to(DEV), 300, n_ctx=nc, q_pos0=2900, cap=300)
    _check_route(idx, counts, q, K, n_ctx, 2900, 300, 300)


def test_route_run_twice_bitwise_identical():
    g = _cpu_gen(14)
    K = torch.randn((4, 50000, 64), generator=g).to(torch.bfloat16).to(DEV)
    q = (torch.randn((4, 1, 64), generator=g) / 8).to(torch.bfloat16).to(DEV)
    a = [t.clone() for t in clsa.route(q, K, 2048)]
    b = [t.clone() for t in clsa.route(q, K, 2048)]
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ---------------------------------------------------------------- threshold
def _tau_with_margin(s, c, margin=1e-4):
    srt = np.sort(s)[::-1]
    for cc in range(c, len(srt)):
        t = np.float32(0.5 * (srt[cc - 1] + srt[cc])) if cc > 0 else np.float32(srt[0] + 1)
        if np.min(np.abs(s - float(t))) >= margin:
            return t
    return np.float32(srt[-1] - 1)


def test_threshold_sets_and_overflow():
    g = _cpu_gen(15)
    B, N, d = 5, 9000, 64
    K = torch.randn((B, N, d), generator=g).to(torch.bfloat16)
    q = (torch.randn((B, 1, d), generator=g) / 8).to(torch.bfloat16)
    q_np, K_np = f64(q), f64(K)
    targets = [0, 1, 500, 3000, N]
    tau = np.zeros((B, 1), dtype=np.float32)
    for b in range(B):
        s = O.route_scores(q_np[b, 0], K_np[b], N)
        tau[b, 0] = np.float32(s.max() + 1) if targets[b] == 0 else (
            np.float32(s.min() - 1) if targets[b] == N else _tau_with_margin(s, targets[b]))
    tau_t = torch.from_numpy(tau).to(DEV)
    for cap in (N, 400):
        idx, counts = clsa.route_threshold(q.to(DEV), K.to(DEV), tau_t, cap)
        o_idx, o_cnt = O.route_threshold(q_np, K_np, [N] * B, -1, tau, cap)
        assert np.array_equal(counts.cpu().numpy(), o_cnt)  # true counts, even past cap
        assert np.array_equal(idx.cpu().numpy(), o_idx)


@pytest.mark.parametrize("dtype,d", [(torch.float32, 32), (torch.float32, 128),
                                     (torch.bfloat16, 32)])
def test_threshold_dtypes_and_index_widths(dtype, d):
    # fp32 keys and the narrowest index head, with a context that ends
    # inside a scan chunk
    g = _cpu_gen(17 + d)
    B, N = 3, 7001
    K = torch.randn((B, N, d), generator=g).to(dtype)
    q = (torch.randn((B, 1, d), generator=g) / math.sqrt(d)).to(dtype)
    q_np, K_np = f64(q), f64(K)
    n_ctx = [N, 5000, 1]
    tau = np.zeros((B, 1), dtype=np.float32)
    for b in range(B):
        s = O.route_scores(q_np[b, 0], K_np[b], n_ctx[b])
        tau[b, 0] = _tau_with_margin(s, min(200, n_ctx[b])) if n_ctx[b] > 1 else np.float32(s[0] - 1)
    nc = torch.tensor(n_ctx, dtype=torch.int32, device=DEV)
    for cap in (1024, 100):
        idx, counts = clsa.route_threshold(q.to(DEV), K.to(DEV), torch.from_numpy(tau).to(DEV),
                                           cap, n_ctx=nc)
        o_idx, o_cnt = O.route_threshold(q_np, K_np, n_ctx, -1, tau, cap)
        assert np.array_equal(counts.cpu().numpy(), o_cnt)
        assert np.array_equal(idx.cpu().numpy(), o_idx)


def test_threshold_ragged_context_and_prefill():
    g = _cpu_gen(16)
    B, M, N, d = 2, 9, 4100, 128
    K = torch.randn((B, N, d), generator=g).to(torch.bfloat16)
    q = (torch.randn((B, M, d), generator=g) / 11).to(torch.bfloat16)
    q_np, K_np = f64(q), f64(K)
    n_ctx = [4100, 3333]
    tau = np.zeros((B, M), dtype=np.float32)
    for b in range(B):
        for m in range(M):
            s = O.route_scores(q_np[b, m], K_np[b], O.visible_count(n_ctx[b], 4000, m))
            tau[b, m] = _tau_with_margin(s, 40 + 7 * m)
    nc = torch.tensor(n_ctx, dtype=torch.int32, device=DEV)
    idx, counts = clsa.route_threshold(q.to(DEV), K.to(DEV), torch.from_numpy(tau).to(DEV), 512,
                                       n_ctx=nc, q_pos0=4000)
    o_idx, o_cnt = O.route_threshold(q_np, K_np, n_ctx, 4000, tau, 512)
    assert np.array_equal(counts.cpu().numpy(), o_cnt)
    assert np.array_equal(idx.cpu().numpy(), o_idx)


# ---------------------------------------------------------------- attention
def _random_lists(g, B, M, n_cap, cap, counts_choice):
    idx = torch.full((B, M, cap), -1, dtype=torch.int32)
    counts = torch.zeros((B, M), dtype=torch.int32)
    i = 0
    for b in range(B):
        for m in range(M):
            c = counts_choice[i % len(counts_choice)]
            i += 1
            sel = torch.randperm(n_cap, generator=g)[:c].sort().values
            idx[b, m, :c] = sel.to(torch.int32)
            counts[b, m] = c
    return idx, counts


def _attn_case(dtype, L, B, M, Hq, Hkv, D, n_cap, cap, counts_choice, seed, qscale=1.0):
    g = _cpu_gen(seed)
    q = (torch.randn((L, B, M, Hq, D), generator=g) * qscale).to(dtype)
    K = torch.randn((L, B, n_cap, Hkv, D), generator=g).to(dtype)
    V = torch.randn((L, B, n_cap, Hkv, D), generator=g).to(dtype)
    idx, counts = _random_lists(g, B, M, n_cap, cap, counts_choice)
    return q, K, V, idx, counts


def _check_attn(q, K, V, idx, counts, scale=0.0, lse_check=True):
    dtype = q.dtype
    out, lse = clsa.sparse_attn(q.to(DEV), K.to(DEV), V.to(DEV), idx.to(DEV), counts.to(DEV),
                                scale=scale, want_lse=True)
    L = q.shape[0]
    o_out, o_lse = O.sparse_attn([f64(q[l]) for l in range(L)], [f64(K[l]) for l in range(L)],
                                 [f64(V[l]) for l in range(L)], idx.numpy(), counts.numpy(),
                                 idx.shape[-1], scale)
    err = np.max(np.abs(f64(out) - o_out))
    assert err <= ATOL[dtype], err
    if lse_check:
        gl = f64(lse)
        fin = np.isfinite(o_lse)
        assert np.array_equal(np.isfinite(gl), fin)
        assert np.max(np.abs(gl[fin] - o_lse[fin]), initial=0.0) <= 1e-3
    return err


def test_attn_fp32_generic():
    case = _attn_case(torch.float32, 2, 2, 3, 4, 2, 64, 600, 300, [0, 1, 64, 65, 300, 129], 21)
    _check_attn(*case)


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (8, 8, 128), (16, 8, 64), (32, 4, 128),
                                      (64, 4, 64), (16, 1, 128), (16, 2, 256), (8, 8, 256)])
def test_attn_bf16_fast_shapes(Hq, Hkv, D):
    case = _attn_case(torch.bfloat16, 2, 2, 2, Hq, Hkv, D, 5000, 700, [0, 1, 700, 65], 22 + Hq)
    _check_attn(*case)


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (16, 8, 64), (64, 4, 64), (16, 2, 256)])
def test_attn_bf16_rows_sharing_positions(Hq, Hkv, D):
    # 48 query rows of one sequence pick 160 of 1500 positions each, so every
    # K/V row is read about five times per layer: the launch keeps gathered
    # rows in the caches instead of streaming them
    case = _attn_case(torch.bfloat16, 2, 1, 48, Hq, Hkv, D, 1500, 160, [160, 97, 1, 0], 31 + D)
    _check_attn(*case)


def test_attn_bf16_generic_head_dim():
    case = _attn_case(torch.bfloat16, 2, 2, 2, 8, 2, 96, 3000, 300, [300, 17, 0, 64], 23)
    _check_attn(*case)


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 2, 256), (16, 1, 256), (4, 4, 8), (2, 1, 16)])
def test_attn_bf16_shapes_outside_the_fast_kernel(Hq, Hkv, D):
    # group sizes the bf16 fast kernel does not take at D = 256 (16 query
    # heads per KV head), and the smallest head dims, on the generic kernel
    case = _attn_case(torch.bfloat16, 2, 2, 2, Hq, Hkv, D, 2500, 400, [400, 63, 1, 0], 27 + D)
    _check_attn(*case)


def test_attn_large_logits_stable():
    case = _attn_case(torch.bfloat16, 1, 2, 2, 32, 8, 128, 3000, 512, [512, 100], 24, qscale=40.0)
    _check_attn(*case)


def test_attn_explicit_scale_and_fp32_mfma_free_path():
    case = _attn_case(torch.float32, 1, 1, 2, 8, 8, 128, 2000, 256, [256, 3], 25)
    _check_attn(*case, scale=0.05)


def test_attn_out_of_range_entries_are_skipped():
    q, K, V, idx, counts = _attn_case(torch.bfloat16, 1, 1, 2, 32, 8, 128, 3000, 256, [200, 256],
                                      26)
    bad = idx.clone()
    bad[0, 0, 5] = -1
    bad[0, 1, 7] = 3000  # == n_cap
    out, _ = clsa.sparse_attn(q.to(DEV), K.to(DEV), V.to(DEV), bad.to(DEV), counts.to(DEV))
    for m, j in ((0, 5), (1, 7)):
        keep = [i for i in range(int(counts[0, m])) if i != j]
        ref_idx = torch.full((1, 1, 256), -1, dtype=torch.int32)
        ref_idx[0, 0, : len(keep)] = idx[0, m, keep]
        ref_cnt = torch.tensor([[len(keep)]], dtype=torch.int32)
        o_out, _ = O.sparse_attn([f64(q[0][:, m:m + 1])], [f64(K[0])], [f64(V[0])],
                                 ref_idx.numpy(), ref_cnt.numpy(), 256)
        assert np.max(np.abs(f64(out[0, 0, m]) - o_out[0, 0, 0])) <= 2e-2


@pytest.mark.parametrize("dtype,Hq,Hkv,D", [(torch.bfloat16, 32, 8, 128),
                                            (torch.bfloat16, 16, 8, 64),
                                            (torch.float32, 4, 2, 64)])
def test_attn_duplicate_and_unordered_entries(dtype, Hq, Hkv, D):
    # a list is a sequence, not a set: a position listed twice takes two
    # softmax terms, and the order of the entries does not matter.  Row
    # lengths cover one ragged tile, several tiles and a split row.
    g = _cpu_gen(29)
    L, B, M, n_cap, cap = 2, 2, 3, 700, 2048
    q = torch.randn((L, B, M, Hq, D), generator=g).to(dtype)
    K = torch.randn((L, B, n_cap, Hkv, D), generator=g).to(dtype)
    V = torch.randn((L, B, n_cap, Hkv, D), generator=g).to(dtype)
    idx = torch.full((B, M, cap), -1, dtype=torch.int32)
    counts = torch.zeros((B, M), dtype=torch.int32)
    lens = [37, 300, 2048, 129, 1500, 1]
    for r, c in enumerate(lens):
        b, m = divmod(r, M)
        # positions drawn with replacement from a small pool, so many repeat
        pool = torch.randperm(n_cap, generator=g)[: max(1, c // 3)]
        sel = pool[torch.randint(0, pool.numel(), (c,), generator=g)]
        idx[b, m, :c] = sel.to(torch.int32)
        counts[b, m] = c
    assert any(torch.unique(idx[b, m, : counts[b, m]]).numel() < int(counts[b, m])
               for b in range(B) for m in range(M) if counts[b, m] > 1)
    _check_attn(q, K, V, idx, counts)
    # the same multiset in ascending order gives the same output within
    # rounding of the summation order
    srt = idx.clone()
    for b in range(B):
        for m in range(M):
            c = int(counts[b, m])
            srt[b, m, :c] = idx[b, m, :c].sort().values
    a, _ = clsa.sparse_attn(q.to(DEV), K.to(DEV), V.to(DEV), idx.to(DEV), counts.to(DEV))
    s, _ = clsa.sparse_attn(q.to(DEV), K.to(DEV), V.to(DEV), srt.to(DEV), counts.to(DEV))
    assert np.max(np.abs(f64(a) - f64(s))) <= ATOL[dtype]


@pytest.mark.parametrize("dtype,Hq,Hkv,D", [(torch.bfloat16, 32, 8, 128),
                                            (torch.float32, 8, 2, 64)])
def test_attn_padding_entries_and_odd_counts(dtype, Hq, Hkv, D):
    # lists built outside the routing calls (reading R24 of the oracle):
    # padding entries (-1, n_cap, the int32 extremes) inside the counted
    # prefix, repeated positions, negative counts, counts past cap; the
    # oracle reads the same lists by the same rules, and rows split
    g = _cpu_gen(34)
    L, B, M, n_cap, cap = 2, 2, 4, 900, 600
    q = torch.randn((L, B, M, Hq, D), generator=g).to(dtype)
    K = torch.randn((L, B, n_cap, Hkv, D), generator=g).to(dtype)
    V = torch.randn((L, B, n_cap, Hkv, D), generator=g).to(dtype)
    idx = torch.randint(0, n_cap, (B, M, cap), generator=g, dtype=torch.int32)
    pad = torch.rand((B, M, cap), generator=g) < 0.1
    vals = torch.tensor([-1, n_cap, 2 ** 31 - 1, -2 ** 31], dtype=torch.int32)
    idx[pad] = vals[torch.randint(0, 4, (int(pad.sum()),), generator=g)]
    idx[1, 1, 0] = -1  # a count of 1 over padding only: an empty row
    counts = torch.tensor([[600, -1, 257, 10 ** 6], [-2 ** 31, 1, 599, 0]], dtype=torch.int32)
    _check_attn(q, K, V, idx, counts)


def _vector_lists(g, R, n_cap, cap, counts):
    """R ascending lists of `cap` distinct positions (all slots filled)."""
    sel = torch.rand((R, n_cap), generator=g).argsort(dim=1)[:, :cap].sort(dim=1).values
    return sel.to(torch.int32), torch.as_tensor(counts, dtype=torch.int32)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_attn_most_layers(dtype):
    # L = 64, the most layers one call takes; two rows, one split per row
    # and one list that splits
    g = _cpu_gen(30)
    L, B, M, Hq, Hkv, D, n_cap, cap = 64, 1, 2, 8, 2, 64, 3000, 1500
    q = torch.randn((L, B, M, Hq, D), generator=g).to(dtype)
    K = torch.randn((L, B, n_cap, Hkv, D), generator=g).to(dtype)
    V = torch.randn((L, B, n_cap, Hkv, D), generator=g).to(dtype)
    idx, counts = _vector_lists(g, B * M, n_cap, cap, [1500, 200])
    _check_attn(q, K, V, idx.view(B, M, cap), counts.view(B, M))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_attn_most_rows(dtype):
    # B*M = 65535 rows, the grid's limit; checked on the first, the last and
    # a spread of rows between
    g = _cpu_gen(31)
    L, B, M, Hq, Hkv, D, n_cap, cap = 2, 5, 13107, 4, 1, 64, 96, 24
    R = B * M
    q = torch.randn((L, B, M, Hq, D), generator=g).to(dtype)
    K = torch.randn((L, B, n_cap, Hkv, D), generator=g).to(dtype)
    V = torch.randn((L, B, n_cap, Hkv, D), generator=g).to(dtype)
    cnt = torch.randint(0, cap + 1, (R,), generator=g)
    cnt[-1] = cap
    idx, counts = _vector_lists(g, R, n_cap, cap, cnt)
    idx, counts = idx.view(B, M, cap), counts.view(B, M)
    out, lse = clsa.sparse_attn(q.to(DEV), K.to(DEV), V.to(DEV), idx.to(DEV), counts.to(DEV),
                                want_lse=True)
    picks = sorted({0, 1, R - 2, R - 1, *range(0, R, 331)})
    rows = [divmod(r, M) for r in picks]
    o_out, o_lse = O.sparse_attn([f64(q[l]) for l in range(L)], [f64(K[l]) for l in range(L)],
                                 [f64(V[l]) for l in range(L)], idx.numpy(), counts.numpy(), cap,
                                 rows=rows)
    go, gl = f64(out), f64(lse)
    for b, m in rows:
        assert np.max(np.abs(go[:, b, m] - o_out[:, b, m])) <= ATOL[dtype], (b, m)
        fin = np.isfinite(o_lse[:, b, m])
        assert np.array_equal(np.isfinite(gl[:, b, m]), fin)
        assert np.max(np.abs(gl[:, b, m][fin] - o_lse[:, b, m][fin]), initial=0.0) <= 1e-3
    assert len(rows) >= 200


@pytest.mark.parametrize("dtype,Hq,Hkv,D", [(torch.bfloat16, 64, 64, 128),
                                            (torch.float32, 64, 64, 128),
                                            (torch.bfloat16, 32, 4, 256),
                                            (torch.float32, 32, 4, 256)])
def test_attn_widest_heads(dtype, Hq, Hkv, D):
    # Hq * D = 8192, the widest query a call takes: 64 heads of 128 (every
    # query head its own KV head) and 32 heads of 256 in groups of 8
    g = _cpu_gen(32)
    L, B, M, n_cap, cap = 2, 2, 2, 1200, 700
    q = torch.randn((L, B, M, Hq, D), generator=g).to(dtype)
    K = torch.randn((L, B, n_cap, Hkv, D), generator=g).to(dtype)
    V = torch.randn((L, B, n_cap, Hkv, D), generator=g).to(dtype)
    idx, counts = _vector_lists(g, B * M, n_cap, cap, [700, 1, 333, 0])
    _check_attn(q, K, V, idx.view(B, M, cap), counts.view(B, M))


def test_attn_counts_past_cap_use_the_first_cap_entries():
    # a threshold list longer than cap reports its true size; attention
    # takes the first cap entries, as for counts == cap
    g = _cpu_gen(33)
    L, B, M, Hq, Hkv, D, n_cap, cap = 2, 1, 3, 32, 8, 128, 5000, 640
    q = torch.randn((L, B, M, Hq, D), generator=g).to(torch.bfloat16)
    K = torch.randn((L, B, n_cap, Hkv, D), generator=g).to(torch.bfloat16)
    V = torch.randn((L, B, n_cap, Hkv, D), generator=g).to(torch.bfloat16)
    idx, _ = _vector_lists(g, M, n_cap, cap, [0, 0, 0])
    idx = idx.view(B, M, cap)
    over = torch.tensor([[641, 100000, 2 ** 31 - 1]], dtype=torch.int32)
    at = torch.full((B, M), cap, dtype=torch.int32)
    a, la = clsa.sparse_attn(q.to(DEV), K.to(DEV), V.to(DEV), idx.to(DEV), over.to(DEV),
                             want_lse=True)
    b_, lb = clsa.sparse_attn(q.to(DEV), K.to(DEV), V.to(DEV), idx.to(DEV), at.to(DEV),
                              want_lse=True)
    assert torch.equal(a, b_) and torch.equal(la, lb)
    _check_attn(q, K, V, idx, at)


def test_attn_split_rows_with_empty_splits():
    # one query row per layer is split 8 ways (256 entries each); in row 0
    # the second half of the list is -1, so four splits hold nothing and the
    # merge must ignore them; row 1 holds only -1 entries (out 0, lse -inf)
    q, K, V, idx, counts = _attn_case(torch.bfloat16, 2, 1, 2, 32, 8, 128, 5000, 2048, [2048],
                                      28)
    idx[0, 0, 1024:] = -1
    idx[0, 1, :] = -1
    out, lse = clsa.sparse_attn(q.to(DEV), K.to(DEV), V.to(DEV), idx.to(DEV), counts.to(DEV),
                                want_lse=True)
    # the oracle takes the valid entries only: row 0's first 1024, none of row 1's
    o_cnt = counts.numpy().copy()
    o_cnt[0, 0], o_cnt[0, 1] = 1024, 0
    o_out, o_lse = O.sparse_attn([f64(q[l]) for l in range(2)], [f64(K[l]) for l in range(2)],
                                 [f64(V[l]) for l in range(2)], idx.numpy(), o_cnt, 2048)
    assert np.max(np.abs(f64(out) - o_out)) <= ATOL[torch.bfloat16]
    gl = f64(lse)
    assert np.all(np.isneginf(gl[:, 0, 1])) and np.all(np.isneginf(o_lse[:, 0, 1]))
    assert np.all(f64(out)[:, 0, 1] == 0.0)
    fin = np.isfinite(o_lse)
    assert np.array_equal(np.isfinite(gl), fin)
    assert np.max(np.abs(gl[fin] - o_lse[fin])) <= 1e-3


def test_attn_split_and_single_pass_agree():
    # one row per layer is split across workgroups; 4096 rows are not
    q, K, V, idx, counts = _attn_case(torch.bfloat16, 1, 1, 1, 32, 8, 128, 8000, 2048, [2048], 27)
    out1, _ = clsa.sparse_attn(q.to(DEV), K.to(DEV), V.to(DEV), idx.to(DEV), counts.to(DEV))
    qq = q.expand(1, 1, 4096, 32, 128).contiguous()
    ii = idx.expand(1, 4096, 2048).contiguous()
    cc = counts.expand(1, 4096).contiguous()
    out2, _ = clsa.sparse_attn(qq.to(DEV), K.to(DEV), V.to(DEV), ii.to(DEV), cc.to(DEV))
    d = (out1[0, 0, 0].float() - out2[0, 0, 4095].float()).abs().max().item()
    assert d <= 1e-2
    _check_attn(q, K, V, idx, counts)


# ------------------------------------------------------- full-size workloads
def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _oracle_lists(q_idx, K_idx, n_ctx, q_pos0, k, rows):
    q_np = f64(q_idx)
    out = {}
    for b, m in rows:
        Kb = f64(K_idx[b])
        nv = O.visible_count(n_ctx[b], q_pos0, m)
        out[(b, m)] = O.topk_select(O.route_scores(q_np[b, m], Kb, nv), k)
    return out


def _attn_oracle_lists_uploaded(q, Kc, Vc, o_lists, layers, cap):
    """End to end: the oracle's own lists, uploaded as the GPU path's input,
    row by row, against the oracle's attention over them."""
    err = 0.0
    for (b, m), sel in o_lists.items():
        oi = torch.full((1, 1, cap), -1, dtype=torch.int32)
        oi[0, 0, : len(sel)] = torch.from_numpy(np.asarray(sel, dtype=np.int32))
        oc = torch.tensor([[len(sel)]], dtype=torch.int32)
        qs = torch.stack([q[l, b:b + 1, m:m + 1] for l in layers])
        Ks = torch.stack([Kc[l, b:b + 1] for l in layers])
        Vs = torch.stack([Vc[l, b:b + 1] for l in layers])
        out, _ = clsa.sparse_attn(qs, Ks, Vs, oi.to(DEV), oc.to(DEV))
        o_out, _ = O.sparse_attn([f64(qs[i]) for i in range(len(layers))], lazy_layers(Ks),
                                 lazy_layers(Vs), oi.numpy(), oc.numpy(), cap)
        err = max(err, float(np.max(np.abs(f64(out) - o_out))))
        del Ks, Vs
    assert err <= ATOL[q.dtype], err
    return err


def _decode_workload(name, steps):
    """The benchmark's decode loop on the full workload: every step appends
    one row per sequence (routing key, and K/V in every layer), routes once
    and attends in all layers in one launch.  The first and the last step
    are checked in full: every sequence's routing against the oracle's exact
    top-k over the cache as that step left it, and the attention output of
    every sequence in every layer against the oracle's attention over the
    GPU's own lists (the very launch the benchmark times)."""
    base = gen.WORKLOADS[name]
    wl = base.with_(n_cap=base.n_ctx + steps)
    K_idx, u, planted = gen.gen_routing_keys(wl, DEV)
    Kc, Vc = gen.gen_kv(wl, DEV)
    new_kidx, new_k, new_v = gen.gen_append_rows(wl, steps, DEV)
    idx = torch.empty((wl.B, 1, wl.k), dtype=torch.int32, device=DEV)
    counts = torch.empty((wl.B, 1), dtype=torch.int32, device=DEV)
    out = torch.empty((wl.L, wl.B, 1, wl.Hq, wl.D), dtype=torch.bfloat16, device=DEV)
    rows = [(b, 0) for b in range(wl.B)]
    layers = list(range(wl.L))
    for t in range(steps):
        n = wl.n_ctx + t + 1
        nc = torch.full((wl.B,), n, dtype=torch.int32, device=DEV)
        q_idx = gen.gen_routing_query(wl, u, t, DEV)
        q = gen.gen_attn_query(wl, q_idx, t, DEV)
        clsa.kv_append(nc - 1, new_kidx[t], K_idx, new_k[t], Kc, new_v[t], Vc)
        clsa.route(q_idx, K_idx, wl.k, n_ctx=nc, idx=idx, counts=counts)
        clsa.sparse_attn(q, Kc, Vc, idx, counts, out=out)
        if t not in (0, steps - 1):
            continue
        torch.cuda.synchronize()
        print(f"{name}: checking step {t} (n = {n})", flush=True)
        ndiff = check_topk_rows(idx, counts, q_idx, K_idx, lambda b, m: n, wl.k, wl.k, rows)
        err, npairs = attn_vs_oracle(q, Kc, Vc, idx, counts, out, rows, layers, wl.k)
        msg = f"{name} step {t}: boundary diffs={ndiff} attention pairs={npairs} err={err:.3g}"
        if t == 0:
            o_lists = _oracle_lists(q_idx, K_idx, [n] * wl.B, -1, wl.k, rows[:2])
            err2 = _attn_oracle_lists_uploaded(q, Kc, Vc, o_lists, [0, wl.L - 1], wl.k)
            gi = idx.cpu().numpy()
            hits = sum(len(set(gi[b, 0].tolist()) & set(planted[b].tolist()))
                       for b in range(wl.B))
            msg += f" oracle-list err={err2:.3g} planted routed={hits}/{planted.numel()} (diagnostic)"
        print(msg, flush=True)
    del K_idx, Kc, Vc, out
    _free()


def test_workload_tiny_fp32():
    wl = gen.WORKLOADS["tiny_fp32_4k"]
    K_idx, u, planted = gen.gen_routing_keys(wl, DEV)
    Kc, Vc = gen.gen_kv(wl, DEV)
    q_idx = gen.gen_routing_query(wl, u, 0, DEV)
    q = gen.gen_attn_query(wl, q_idx, 0, DEV)
    idx, counts = clsa.route(q_idx, K_idx, wl.k)
    out, lse = clsa.sparse_attn(q, Kc, Vc, idx, counts, want_lse=True)
    torch.cuda.synchronize()
    assert _check_route(idx, counts, q_idx, K_idx, [wl.n_ctx], -1, wl.k, wl.k) == 0
    o_idx, o_cnt = O.route(f64(q_idx), f64(K_idx), [wl.n_ctx], -1, wl.k, wl.k)
    o_out, o_lse = O.sparse_attn([f64(q[0])], [f64(Kc[0])], [f64(Vc[0])], o_idx, o_cnt, wl.k)
    assert np.max(np.abs(f64(out) - o_out)) <= 1e-4
    assert np.max(np.abs(f64(lse) - o_lse)) <= 1e-4


@pytest.mark.timeout(600)
def test_workload_decode_32k():
    _decode_workload("decode_32k", 64)


@pytest.mark.timeout(600)
def test_workload_decode_128k_b8():
    _decode_workload("decode_128k_b8", 64)


@pytest.mark.timeout(900)
def test_workload_prefill_128k():
    """All 4096 rows of the chunk's routing against the oracle; the chunk's
    16-layer attention launch on 64 rows spread over the chunk, in every
    layer, against the oracle over the GPU's lists; and 3 rows end to end
    on the oracle's own lists."""
    wl = gen.WORKLOADS["prefill_128k_c4096"]
    K_idx, u, _ = gen.gen_routing_keys(wl, DEV)
    q_idx = gen.gen_routing_query(wl, u, 0, DEV)
    idx, counts = clsa.route(q_idx, K_idx, wl.k, q_pos0=wl.q_pos0)
    torch.cuda.synchronize()
    print("prefill_128k: routing of all rows against the oracle", flush=True)
    nd = check_topk_rows(idx, counts, q_idx, K_idx,
                         lambda b, m: O.visible_count(wl.n_ctx, wl.q_pos0, m), wl.k, wl.k,
                         [(0, m) for m in range(wl.M)])
    assert nd <= 2 * wl.M
    Kc, Vc = gen.gen_kv(wl, DEV)
    q = gen.gen_attn_query(wl, q_idx, 0, DEV)
    out, _ = clsa.sparse_attn(q, Kc, Vc, idx, counts)  # the full 4096-row launch
    torch.cuda.synchronize()
    rows = [(0, int(m)) for m in np.linspace(0, wl.M - 1, 64).round().astype(int)]
    print("prefill_128k: attention of 64 rows in 16 layers against the oracle", flush=True)
    err, npairs = attn_vs_oracle(q, Kc, Vc, idx, counts, out, rows, range(wl.L), wl.k)
    o_lists = _oracle_lists(q_idx, K_idx, [wl.n_ctx], wl.q_pos0, wl.k, rows[:3])
    _attn_oracle_lists_uploaded(q, Kc, Vc, o_lists, [0, 15], wl.k)
    print(f"prefill_128k: boundary diffs={nd} attention pairs={npairs} err={err:.3g}", flush=True)
    del Kc, Vc, q, out, K_idx
    _free()


@pytest.mark.timeout(600)
def test_workload_threshold_128k_b16():
    wl = gen.WORKLOADS["threshold_128k_b16"]
    K_cpu, q_cpu, tau = gen.gen_threshold_inputs(
        wl, lambda qq, KK: O.route_scores(qq, KK, KK.shape[0]))
    K_idx, q_idx, tau_d = K_cpu.to(DEV), q_cpu.to(DEV), tau.to(DEV)
    for cap in (16384, 4096):
        idx, counts = clsa.route_threshold(q_idx, K_idx, tau_d, cap)
        o_idx, o_cnt = O.route_threshold(f64(q_cpu), f64(K_cpu), [wl.n_ctx] * wl.B, -1,
                                         tau.numpy(), cap)
        assert np.array_equal(counts.cpu().numpy(), o_cnt)  # true counts, zero misses
        assert np.array_equal(idx.cpu().numpy(), o_idx)
    assert o_cnt.min() >= 200 and o_cnt.max() <= 9000
    cap = 16384
    idx, counts = clsa.route_threshold(q_idx, K_idx, tau_d, cap)
    Kc, Vc = gen.gen_kv(wl, DEV)
    q = gen.gen_attn_query(wl, q_idx, 0, DEV)
    out, _ = clsa.sparse_attn(q, Kc, Vc, idx, counts)
    torch.cuda.synchronize()
    # the lists equal the oracle's (asserted above), so this is end to end too
    rows = [(b, 0) for b in (0, 5, 10, 15)]
    err, npairs = attn_vs_oracle(q, Kc, Vc, idx, counts, out, rows, range(wl.L), cap)
    print(f"threshold_128k: attention pairs={npairs} err={err:.3g}", flush=True)
    del Kc, Vc, q, out, K_idx
    _free()


def test_kv_append_writes_each_sequence_slot():
    g = _cpu_gen(31)
    L, B, n_cap, Hkv, D, d = 3, 5, 50, 8, 128, 64
    K = torch.randn((L, B, n_cap, Hkv, D), generator=g).to(torch.bfloat16).to(DEV)
    V = torch.randn((L, B, n_cap, Hkv, D), generator=g).to(torch.bfloat16).to(DEV)
    Ki = torch.randn((B, n_cap, d), generator=g).to(torch.bfloat16).to(DEV)
    nk = torch.randn((L, B, Hkv, D), generator=g).to(torch.bfloat16).to(DEV)
    nv = torch.randn((L, B, Hkv, D), generator=g).to(torch.bfloat16).to(DEV)
    ni = torch.randn((B, d), generator=g).to(torch.bfloat16).to(DEV)
    pos = torch.tensor([0, 17, 49, 50, -1], dtype=torch.int32, device=DEV)  # 50, -1: outside
    K0, V0, Ki0 = K.clone(), V.clone(), Ki.clone()
    clsa.kv_append(pos, ni, Ki, nk, K, nv, V)
    torch.cuda.synchronize()
    for b, p in enumerate([0, 17, 49]):
        K0[:, b, p] = nk[:, b]
        V0[:, b, p] = nv[:, b]
        Ki0[b, p] = ni[b]
    assert torch.equal(K, K0) and torch.equal(V, V0) and torch.equal(Ki, Ki0)


def test_decode_steps_append_route_attend():
    # the benchmark's step, three times in a row on a small decode shape:
    # each step appends one row per sequence (its routing key, and K/V in
    # every layer) with clsa_kv_append, routes over the grown context and
    # attends.  Each step is checked against the oracle on the caches as
    # that step left them.  One context grows through 4096 keys, where the
    # routing sample starts to skip keys.
    wl = gen.WORKLOADS["decode_32k"].with_(B=3, n_ctx=6000, n_cap=6008, L=3, k=1024,
                                           planted=32)
    K_idx, u, _ = gen.gen_routing_keys(wl, DEV)
    Kc, Vc = gen.gen_kv(wl, DEV)
    steps = 3
    new_kidx, new_k, new_v = gen.gen_append_rows(wl, steps, DEV)
    n0 = [6000, 5000, 4094]
    for t in range(steps):
        n_ctx = [n + t + 1 for n in n0]
        pos = torch.tensor([n - 1 for n in n_ctx], dtype=torch.int32, device=DEV)
        nc = torch.tensor(n_ctx, dtype=torch.int32, device=DEV)
        q_idx = gen.gen_routing_query(wl, u, t, DEV)
        q = gen.gen_attn_query(wl, q_idx, t, DEV)
        clsa.kv_append(pos, new_kidx[t], K_idx, new_k[t], Kc, new_v[t], Vc)
        idx, counts = clsa.route(q_idx, K_idx, wl.k, n_ctx=nc)
        out, _ = clsa.sparse_attn(q, Kc, Vc, idx, counts)
        torch.cuda.synchronize()
        for b in range(wl.B):  # the step's rows sit where it appended them
            assert torch.equal(K_idx[b, n_ctx[b] - 1], new_kidx[t, b])
            assert torch.equal(Kc[:, b, n_ctx[b] - 1], new_k[t, :, b])
            assert torch.equal(Vc[:, b, n_ctx[b] - 1], new_v[t, :, b])
        _check_route(idx, counts, q_idx, K_idx, n_ctx, -1, wl.k, wl.k)
        rows = [(b, 0) for b in range(wl.B)]
        attn_vs_oracle(q, Kc, Vc, idx, counts, out, rows, range(wl.L), wl.k)
    del K_idx, Kc, Vc
    _free()


def test_attn_headline_launch_shape_small_context():
    # the headline's attention launch shape (16 layers x 8 sequences x 8 KV
    # heads = 1024 workgroups, each streaming one unsplit 2048-entry list)
    # at a context the oracle reads in full: every output element compared
    q, K, V, idx, counts = _attn_case(torch.bfloat16, 16, 8, 1, 32, 8, 128, 9000, 2048,
                                      [2048], 41)
    assert clsa.sparse_attn_workspace_size(16, 8, 1, 32, 8, 128, 2048, torch.bfloat16) == 0
    _check_attn(q, K, V, idx, counts)
