"""Pins of the CPU oracle to facts outside itself (CPU only).

Each pin checks the oracle against something it does not compute itself: a
hand-worked example, exact rational arithmetic, closed forms, exhaustive
brute force on tiny inputs, library routines (torch.matmul, torch.topk,
scaled_dot_product_attention) and invariants of the definitions:

* routing score: raw inner product (CLSA explainer, ai-papers.net, section
  "CLSAの仕組み"; Louver summary, gist.science, section
  "1. 半空間範囲検索への帰着");
* top-k: the k highest scores, ties to the lower index, ascending
  (same CLSA section; tie rule and order are readings);
* threshold: every key with score >= tau and no other (Louver summary,
  same section: zero false negatives);
* attention: softmax over the selected rows (CLSA explainer, "CLSAの仕組み").

The pins are collected in `battery(o)` so that the mutation tests at the end
can re-run all of them against deliberately broken copies of the oracle and
show that each plausible mistake is caught.
"""
from __future__ import annotations

import itertools
import json
import math
import os
import types
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import clsa_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def _ns(**over):
    base = dict(
        route_scores=O.route_scores,
        topk_select=O.topk_select,
        threshold_select=O.threshold_select,
        attend_head=O.attend_head,
        sparse_attn=O.sparse_attn,
        route=O.route,
        visible_count=O.visible_count,
    )
    base.update(over)
    return types.SimpleNamespace(**base)


ORACLE = _ns()
# originals, for mutants that wrap them (the mutation tests patch the module)
_SCORES, _TOPK, _ATTEND = O.route_scores, O.topk_select, O.attend_head
_SPARSE = O.sparse_attn


def _bf16_values(shape, rng, scale=1.0):
    x = torch.from_numpy(rng.standard_normal(shape) * scale).to(torch.bfloat16)
    return x.to(torch.float64).numpy()


# --------------------------------------------------------------------------
# individual pins (each raises AssertionError on failure)
# --------------------------------------------------------------------------
def pin_golden(o):
    with open(os.path.join(HERE, "golden", "hand_route.json")) as f:
        g = json.load(f)
    r = g["route"]
    q = np.array(r["q_idx"])
    K = np.array(r["K_idx"])
    s = o.route_scores(q, K, K.shape[0])
    assert np.array_equal(s, np.array(r["scores"])), s
    for k, want in r["topk"].items():
        got = o.topk_select(s, int(k)).tolist()
        assert got == want, (k, got, want)
    for t, want in r["threshold"].items():
        got = o.threshold_select(s, float(t)).tolist()
        assert got == want, (t, got, want)
    a = g["attention"]
    out, lse, p = o.attend_head(np.array(a["q"]), np.array(a["K"]), np.array(a["V"]),
                                a["scale"], return_weights=True)
    assert np.allclose(p, a["weights"], rtol=0, atol=1e-14), p
    assert np.allclose(out, a["out"], rtol=0, atol=1e-13), out
    assert abs(lse - a["lse"]) < 1e-13, lse


def pin_scores_exact(o):
    rng = np.random.default_rng(11)
    # small integers: every product and partial sum is exact in float64
    for d in (1, 3, 32, 64, 128):
        q = rng.integers(-8, 9, size=d).astype(np.float64)
        K = rng.integers(-8, 9, size=(9, d)).astype(np.float64)
        s = o.route_scores(q, K, 9)
        for j in range(9):
            exact = sum(int(q[i]) * int(K[j, i]) for i in range(d))
            assert s[j] == exact, (d, j, s[j], exact)
    # bf16-valued Gaussians: compare with exact rational sums
    for d in (32, 64, 128):
        q = _bf16_values(d, rng)
        K = _bf16_values((12, d), rng)
        s = o.route_scores(q, K, 12)
        for j in range(12):
            exact = sum(Fraction(float(q[i])) * Fraction(float(K[j, i])) for i in range(d))
            mag = sum(abs(Fraction(float(q[i])) * Fraction(float(K[j, i]))) for i in range(d))
            assert abs(Fraction(float(s[j])) - exact) <= mag * Fraction(1, 2**50), (d, j)


def pin_scores_closed_form(o):
    rng = np.random.default_rng(12)
    for d in (4, 32):
        q = rng.standard_normal(d)
        s = o.route_scores(q, np.eye(d), d)
        assert np.array_equal(s, q)
        s = o.route_scores(q, 2.0 * np.eye(d)[::-1], d)
        assert np.array_equal(s, 2.0 * q[::-1])
        # only the visible prefix is scored
        s = o.route_scores(q, np.eye(d), d // 2)
        assert s.shape == (d // 2,) and np.array_equal(s, q[: d // 2])
    q = rng.standard_normal(16)
    K = rng.standard_normal((40, 16))
    ref = torch.matmul(torch.from_numpy(K), torch.from_numpy(q)).numpy()
    assert np.allclose(o.route_scores(q, K, 40), ref, rtol=1e-14, atol=1e-14)


def _brute_topk(s, k):
    n = len(s)
    kk = min(k, n)
    valid = []
    for S in itertools.combinations(range(n), kk):
        inS = set(S)
        ok = all((s[i] > s[j]) or (s[i] == s[j] and i < j)
                 for i in inS for j in range(n) if j not in inS)
        if ok:
            valid.append(list(S))
    assert len(valid) == 1, valid  # the ordering is total, so exactly one set
    return valid[0]


def pin_topk_bruteforce(o):
    rng = np.random.default_rng(13)
    for _ in range(60):
        n = int(rng.integers(0, 10))
        s = rng.integers(-2, 3, size=n).astype(np.float64)  # many exact ties
        for k in range(0, n + 3):
            want = _brute_topk(s, k)
            got = o.topk_select(s, k).tolist()
            assert got == want, (s.tolist(), k, got, want)


def pin_topk_library(o):
    rng = np.random.default_rng(14)
    s = rng.standard_normal(1000)  # continuous: ties have probability 0
    for k in (1, 10, 500, 999, 1000):
        got = o.topk_select(s, k)
        ref = torch.topk(torch.from_numpy(s), k).indices.numpy()
        assert np.array_equal(got, np.sort(ref)), k
        assert np.all(np.diff(got) > 0)


def pin_topk_ties_signed_zero(o):
    s = np.array([0.0, -0.0, 0.0, -0.0, 1.0, -1.0])
    assert o.topk_select(s, 3).tolist() == [0, 1, 4]
    assert o.topk_select(s, 4).tolist() == [0, 1, 2, 4]
    s = np.zeros(50)
    assert o.topk_select(s, 7).tolist() == list(range(7))
    assert o.topk_select(s, 0).tolist() == []


def pin_threshold(o):
    rng = np.random.default_rng(15)
    s = rng.standard_normal(2000)
    srt = np.sort(s)[::-1]
    for c in (0, 1, 17, 1000, 1999):
        tau = np.float32(0.5 * (srt[c - 1] + srt[c])) if c > 0 else np.float32(srt[0] + 1.0)
        if c > 0 and not (srt[c - 1] > float(tau) > srt[c]):
            continue
        got = o.threshold_select(s, tau)
        assert np.array_equal(got, o.topk_select(s, c)), c
    tau = np.float32(0.25)
    got = set(o.threshold_select(s, tau).tolist())
    for j in range(len(s)):
        assert (j in got) == (s[j] >= float(tau))
    # ">=" keeps equality, and -0.0 equals +0.0
    assert o.threshold_select(np.array([0.0, -0.0, -1e-30, 1e-30]), -0.0).tolist() == [0, 1, 3]
    assert o.threshold_select(np.array([1.5, 1.5, 2.0]), 1.5).tolist() == [0, 1, 2]


def _sdpa_ref(q, K, V, idx_rows, scale):
    """Dense SDPA (float64, CPU) with -inf outside each row's selected set."""
    L = len(q)
    B, M, Hq, D = q[0].shape
    Hkv = K[0].shape[2]
    N = K[0].shape[1]
    G = Hq // Hkv
    out = np.zeros((L, B, M, Hq, D))
    for l in range(L):
        for b in range(B):
            qq = torch.from_numpy(q[l][b]).permute(1, 0, 2)[None]  # [1,Hq,M,D]
            kk = torch.from_numpy(K[l][b]).permute(1, 0, 2).repeat_interleave(G, 0)[None]
            vv = torch.from_numpy(V[l][b]).permute(1, 0, 2).repeat_interleave(G, 0)[None]
            mask = torch.full((1, Hq, M, N), -math.inf, dtype=torch.float64)
            for m in range(M):
                mask[0, :, m, idx_rows[b][m]] = 0.0
            o_ = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask,
                                                                  scale=scale)
            out[l, b] = o_[0].permute(1, 0, 2).numpy()
    return out


def _rand_attn_case(rng, L=2, B=2, M=3, Hq=8, Hkv=2, D=16, N=37):
    q = [rng.standard_normal((B, M, Hq, D)) for _ in range(L)]
    K = [rng.standard_normal((B, N, Hkv, D)) for _ in range(L)]
    V = [rng.standard_normal((B, N, Hkv, D)) for _ in range(L)]
    return q, K, V


def pin_attention_dense(o):
    rng = np.random.default_rng(16)
    q, K, V = _rand_attn_case(rng)
    B, M, N = 2, 3, 37
    idx = np.tile(np.arange(N), (B, M, 1))
    counts = np.full((B, M), N)
    out, lse = o.sparse_attn(q, K, V, idx, counts, N)
    ref = _sdpa_ref(q, K, V, [[np.arange(N)] * M] * B, 1.0 / math.sqrt(16))
    assert np.max(np.abs(out - ref)) < 1e-12


def pin_attention_masked(o):
    rng = np.random.default_rng(17)
    q, K, V = _rand_attn_case(rng)
    B, M, N, cap = 2, 3, 37, 20
    idx = np.full((B, M, cap), -1)
    counts = np.zeros((B, M), dtype=np.int64)
    rows = [[None] * M for _ in range(B)]
    for b in range(B):
        for m in range(M):
            c = int(rng.integers(1, cap + 1))
            sel = np.sort(rng.choice(N, size=c, replace=False))
            idx[b, m, :c] = sel
            counts[b, m] = c
            rows[b][m] = sel
    out, lse = o.sparse_attn(q, K, V, idx, counts, cap, scale=0.37)
    ref = _sdpa_ref(q, K, V, rows, 0.37)
    assert np.max(np.abs(out - ref)) < 1e-12
    # lse = log sum exp of the scaled logits
    for b in range(B):
        for m in range(M):
            for h in range(8):
                g = (h * 2) // 8
                z = (K[0][b][rows[b][m], g, :] @ q[0][b, m, h]) * 0.37
                assert abs(lse[0, b, m, h] - math.log(np.sum(np.exp(z)))) < 1e-12


def pin_softmax_weights(o):
    rng = np.random.default_rng(18)
    for n in (1, 2, 100):
        qh = rng.standard_normal(8) * 3
        Ks = rng.standard_normal((n, 8))
        Vs = rng.standard_normal((n, 8))
        out, lse, p = o.attend_head(qh, Ks, Vs, 0.5, return_weights=True)
        assert abs(p.sum() - 1.0) < 1e-12 and np.all(p >= 0)
        assert np.allclose(out, p @ Vs, atol=1e-13)


def pin_attention_closed_forms(o):
    rng = np.random.default_rng(19)
    Ks = rng.standard_normal((13, 8))
    Vs = rng.standard_normal((13, 8))
    out, lse = o.attend_head(np.zeros(8), Ks, Vs, 1.0)
    assert np.allclose(out, Vs.mean(axis=0), atol=1e-14)
    assert abs(lse - math.log(13)) < 1e-14
    # one logit far above the others selects that row's value
    qh = np.zeros(8)
    qh[0] = 1.0
    Ks2 = Ks.copy()
    Ks2[:, 0] = 0.0
    Ks2[5, 0] = 2000.0
    out, lse = o.attend_head(qh, Ks2, Vs, 1.0)
    assert np.allclose(out, Vs[5], atol=1e-12) and abs(lse - 2000.0) < 1e-9
    # large logits stay finite
    out, lse = o.attend_head(qh * 1e4, Ks, Vs, 1.0)
    assert np.all(np.isfinite(out)) and math.isfinite(lse)
    # empty selection
    out, lse = o.attend_head(qh, Ks[:0], Vs[:0], 1.0)
    assert np.all(out == 0) and lse == -math.inf


def pin_attention_hull_and_order(o):
    rng = np.random.default_rng(20)
    Ks = rng.standard_normal((50, 16))
    Vs = rng.standard_normal((50, 16))
    qh = rng.standard_normal(16)
    out, _ = o.attend_head(qh, Ks, Vs, 0.25)
    assert np.all(out <= Vs.max(axis=0) + 1e-12) and np.all(out >= Vs.min(axis=0) - 1e-12)
    perm = rng.permutation(50)
    out2, _ = o.attend_head(qh, Ks[perm], Vs[perm], 0.25)
    assert np.max(np.abs(out - out2)) < 1e-13


def pin_prefill_visibility(o):
    # K_idx row j = (j+1) * e0, q = e0: the highest scores are the latest keys,
    # so causal visibility decides the selection.
    n, d = 64, 4
    K = np.zeros((1, n, d))
    K[0, :, 0] = np.arange(1, n + 1)
    qi = np.zeros((1, 5, d))
    qi[0, :, 0] = 1.0
    idx, counts = o.route(qi, K, [n], 40, 3, 6)
    for m in range(5):
        p = 40 + m
        assert counts[0, m] == 3
        assert idx[0, m].tolist() == [p - 2, p - 1, p, -1, -1, -1], (m, idx[0, m])
    idx, counts = o.route(qi, K, [n], 0, 8, 8)
    assert counts[0, 0] == 1 and idx[0, 0, 0] == 0
    assert counts[0, 4] == 5 and idx[0, 4, :5].tolist() == [0, 1, 2, 3, 4]


def pin_attention_padding_and_counts(o):
    # R24: a list is read up to min(count, cap) entries, a negative count
    # reads none, entries outside [0, n_cap) are padding, and a position
    # listed c times weighs c times in the softmax.  Reference: dense SDPA
    # with log(multiplicity) as the additive mask of each listed position.
    rng = np.random.default_rng(21)
    q, K, V = _rand_attn_case(rng, L=1, B=1, M=6)
    N, cap, sc = 37, 12, 0.3
    idx = rng.integers(0, N, size=(1, 6, cap))
    idx[0, 0, [1, 4, 7]] = -1          # padding inside the counted prefix
    idx[0, 1, [0, 11]] = N             # one past the end, and at the last slot
    idx[0, 2, :6] = [5, 5, 5, 9, 9, 2]  # repeats
    counts = np.array([[cap, cap, 6, -3, cap + 40, 4]])
    idx[0, 5, :4] = -1                 # a counted prefix of padding only
    out, lse = o.sparse_attn(q, K, V, idx, counts, cap, scale=sc)
    for m in range(6):
        n = max(0, min(int(counts[0, m]), cap))
        ent = [int(j) for j in idx[0, m, :n] if 0 <= j < N]
        if not ent:
            assert np.all(out[0, 0, m] == 0) and np.all(lse[0, 0, m] == -math.inf), m
            continue
        mult = np.bincount(ent, minlength=N)
        mask = torch.full((1, 8, 1, N), -math.inf, dtype=torch.float64)
        mask[0, :, 0, mult > 0] = torch.from_numpy(np.log(mult[mult > 0]))
        qq = torch.from_numpy(q[0][0, m:m + 1]).permute(1, 0, 2)[None]
        kk = torch.from_numpy(K[0][0]).permute(1, 0, 2).repeat_interleave(4, 0)[None]
        vv = torch.from_numpy(V[0][0]).permute(1, 0, 2).repeat_interleave(4, 0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask,
                                                               scale=sc)[0, :, 0].numpy()
        assert np.max(np.abs(out[0, 0, m] - ref)) < 1e-12, m
        for h in range(8):
            z = (K[0][0][:, h // 4, :] @ q[0][0, m, h]) * sc
            want = math.log(float(np.sum(mult * np.exp(z))))
            assert abs(lse[0, 0, m, h] - want) < 1e-12, (m, h)


def pin_context_clamp(o):
    # R25: a context length below 0 sees no key, one above n_cap every key;
    # reference: the top-k by a stable argsort of the scores over the keys
    # the clamped length leaves visible
    rng = np.random.default_rng(22)
    n_cap, d, k = 40, 8, 6
    K = rng.standard_normal((4, n_cap, d))
    qi = rng.standard_normal((4, 3, d))
    n_ctx = [-3, n_cap + 50, 5, -(2 ** 31)]
    for q_pos0 in (-1, 30):
        idx, counts = o.route(qi, K, n_ctx, q_pos0, k, k + 2)
        for b, n in enumerate(n_ctx):
            for m in range(3):
                nv = min(max(n, 0), n_cap)
                if q_pos0 >= 0:
                    nv = min(nv, q_pos0 + m + 1)
                s_ = K[b, :nv] @ qi[b, m]
                want = np.sort(np.argsort(-s_, kind="stable")[:k])
                assert counts[b, m] == len(want), (q_pos0, b, m)
                assert idx[b, m, : len(want)].tolist() == want.tolist()
                assert np.all(idx[b, m, len(want):] == -1)


ALL_PINS = [
    pin_golden,
    pin_scores_exact,
    pin_scores_closed_form,
    pin_topk_bruteforce,
    pin_topk_library,
    pin_topk_ties_signed_zero,
    pin_threshold,
    pin_attention_dense,
    pin_attention_masked,
    pin_softmax_weights,
    pin_attention_closed_forms,
    pin_attention_hull_and_order,
    pin_attention_padding_and_counts,
    pin_prefill_visibility,
    pin_context_clamp,
]


def battery(o):
    for p in ALL_PINS:
        p(o)


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(ORACLE)


# --------------------------------------------------------------------------
# property tests over random small shapes
# --------------------------------------------------------------------------
@settings(max_examples=150, deadline=None)
@given(st.lists(st.sampled_from([-2.0, -1.0, -0.0, 0.0, 0.5, 1.0, 3.0]), max_size=40),
       st.integers(min_value=0, max_value=45))
def test_topk_invariants_with_ties(vals, k):
    s = np.array(vals, dtype=np.float64)
    S = O.topk_select(s, k)
    n = len(s)
    assert len(S) == min(k, n)
    assert np.all(np.diff(S) > 0)
    inS = np.zeros(n, dtype=bool)
    inS[S] = True
    if 0 < len(S) < n:
        lo = s[inS].min()
        hi = s[~inS].max()
        assert lo >= hi
        if lo == hi:  # at the boundary value, selected indices precede unselected ones
            sel_b = np.flatnonzero(inS & (s == lo))
            uns_b = np.flatnonzero(~inS & (s == lo))
            assert sel_b.max() < uns_b.min()
    assert np.array_equal(O.topk_select(2.0 * s, k), S)


@settings(max_examples=100, deadline=None)
@given(st.integers(min_value=1, max_value=60), st.integers(min_value=0, max_value=70),
       st.integers(min_value=0, max_value=2**31 - 1))
def test_topk_permutation_equivariance(n, k, seed):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal(n)
    perm = rng.permutation(n)
    S = set(O.topk_select(s, k).tolist())
    Sp = set(O.topk_select(s[perm], k).tolist())
    assert {int(perm[i]) for i in Sp} == S


@settings(max_examples=100, deadline=None)
@given(st.integers(min_value=0, max_value=80), st.floats(min_value=-3, max_value=3),
       st.integers(min_value=0, max_value=2**31 - 1))
def test_threshold_definition(n, tau, seed):
    rng = np.random.default_rng(seed)
    s = np.round(rng.standard_normal(n), 1)  # ties with tau happen
    S = O.threshold_select(s, tau)
    t = float(np.float32(tau))
    assert S.tolist() == [j for j in range(n) if s[j] >= t]


# --------------------------------------------------------------------------
# mutation tests: each plausible mistake, planted in a copy of the oracle on
# the CPU, makes at least one pin fail
# --------------------------------------------------------------------------
def _mut_scores_drop_last(q, K, n):
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K[:n], dtype=np.float64)
    return K[:, :-1] @ q[:-1] if K.shape[0] else np.zeros(0)


def _mut_scores_off_by_one(q, K, n):
    return _SCORES(q, K, max(n - 1, 0))


def _mut_scores_transposed(q, K, n):
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K[:n], dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(0)
    return (K.T @ K @ q)[: K.shape[0]] if K.shape[0] <= K.shape[1] else K @ q[::-1]


def _mut_topk_high_tie(s, k):
    s = np.asarray(s, dtype=np.float64)
    j = np.arange(len(s))
    return np.sort(np.lexsort((-j, -s))[: min(k, len(s))])


def _mut_topk_unsorted(s, k):
    s = np.asarray(s, dtype=np.float64)
    j = np.arange(len(s))
    return np.lexsort((j, -s))[: min(k, len(s))]


def _mut_topk_off_by_one(s, k):
    return _TOPK(s, max(k - 1, 0)) if k > 1 else _TOPK(s, k)


def _mut_threshold_strict(s, tau):
    return np.flatnonzero(np.asarray(s, dtype=np.float64) > float(np.float32(tau)))


def _mut_attend_no_scale(q, K, V, scale, return_weights=False):
    return _ATTEND(q, K, V, 1.0, return_weights)


def _mut_attend_no_max(q, K, V, scale, return_weights=False):
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        r = (np.zeros(q.shape[0]), -math.inf)
        return r + (np.zeros(0),) if return_weights else r
    z = (K @ q) * scale
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(z)
        p = e / e.sum()
        r = (p @ V, float(np.log(e.sum())))
    return r + (p,) if return_weights else r


def _mut_attend_lse_no_max(q, K, V, scale, return_weights=False):
    res = _ATTEND(q, K, V, scale, True)
    out, lse, p = res
    z = (np.asarray(K, dtype=np.float64) @ np.asarray(q, dtype=np.float64)) * scale
    wrong = lse - (z.max() if len(z) else 0.0)
    return (out, wrong, p) if return_weights else (out, wrong)


def _mut_attn_padding_as_rows(q, K, V, idx, counts, cap, scale=0.0, rows=None, layers=None):
    # padding entries wrapped around to real rows
    n_cap = K[0].shape[1]
    return _SPARSE(q, K, V, np.mod(idx, n_cap), counts, cap, scale, rows, layers)


def _mut_attn_negative_count_slices(q, K, V, idx, counts, cap, scale=0.0, rows=None,
                                    layers=None):
    # a negative count read as a slice end counted from the back
    c = np.where(np.asarray(counts) < 0, cap + np.asarray(counts), counts)
    return _SPARSE(q, K, V, idx, c, cap, scale, rows, layers)


def _mut_visible_unclamped(n_ctx_b, q_pos0, m, n_cap=None):
    # the context length used as given
    return int(n_ctx_b) if q_pos0 < 0 else int(min(n_ctx_b, q_pos0 + m + 1))


MUTANTS = {
    "scores_drop_last_term": dict(route_scores=_mut_scores_drop_last),
    "scores_off_by_one_visible": dict(route_scores=_mut_scores_off_by_one),
    "scores_transposed": dict(route_scores=_mut_scores_transposed),
    "topk_ties_to_higher_index": dict(topk_select=_mut_topk_high_tie),
    "topk_not_ascending": dict(topk_select=_mut_topk_unsorted),
    "topk_off_by_one": dict(topk_select=_mut_topk_off_by_one),
    "threshold_strict": dict(threshold_select=_mut_threshold_strict),
    "attend_missing_scale": dict(attend_head=_mut_attend_no_scale),
    "attend_no_max_subtraction": dict(attend_head=_mut_attend_no_max),
    "attend_lse_missing_max": dict(attend_head=_mut_attend_lse_no_max),
    "attn_padding_as_rows": dict(sparse_attn=_mut_attn_padding_as_rows),
    "attn_negative_count_slices": dict(sparse_attn=_mut_attn_negative_count_slices),
    "visible_count_unclamped": dict(visible_count=_mut_visible_unclamped),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    over = MUTANTS[name]
    # sparse_attn and route call the module-level helpers, so patch those too
    for fn, impl in over.items():
        monkeypatch.setattr(O, fn, impl)
    with pytest.raises(AssertionError):
        battery(_ns(**over))


def test_mutant_gqa_mapping_is_caught(monkeypatch):
    monkeypatch.setattr(O, "kv_head_of", lambda h, Hq, Hkv: h % Hkv)
    with pytest.raises(AssertionError):
        battery(_ns())


def test_planted_keys_diagnostic():
    """Diagnostic only (not a parity pin): in the tiny workload most planted
    keys (score ~3 above the bulk) should be routed."""
    from long_context_sparse_routing_amd.inputs import WORKLOADS, gen_routing_keys, gen_routing_query
    wl = WORKLOADS["tiny_fp32_4k"]
    K, u, planted = gen_routing_keys(wl, "cpu")
    q = gen_routing_query(wl, u, 0, "cpu")
    idx, counts = O.route(q.double().numpy(), K.double().numpy(), [wl.n_ctx], -1, wl.k, wl.k)
    hit = len(set(idx[0, 0, : counts[0, 0]].tolist()) & set(planted[0].tolist()))
    assert counts[0, 0] == wl.k
    assert hit >= 12, hit
