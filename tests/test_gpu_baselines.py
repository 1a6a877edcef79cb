"""GPU parity of the two baselines the shared-routing path is compared with
(CLSA explainer, sections "計算コストの削減効果" and "推論速度の改善結果"):

  * dense decode attention: every visible key attended, i.e. the sparse
    attention call with the full position list (k = N);
  * unshared per-layer routing: each layer has its own index keys and
    queries, routes on its own and attends over its own list.

Acceptance as in the other GPU tests: attention max abs error <= 2e-2 for
bf16 K/V against the oracle; routed sets equal up to boundary pairs within
1e-5 relative of the c-th largest score.
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


def _full_lists(B, n_ctx, cap):
    idx = torch.full((B, 1, cap), -1, dtype=torch.int32)
    for b, n in enumerate(n_ctx):
        idx[b, 0, :n] = torch.arange(n, dtype=torch.int32)
    return idx, torch.tensor([[n] for n in n_ctx], dtype=torch.int32)


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (8, 8, 64)])
def test_dense_attention_is_full_list_sparse_attention(Hq, Hkv, D):
    g = _gen(300 + Hq + D)
    L, B, n_cap = 2, 2, 6000
    n_ctx = [6000, 4321]
    K = torch.randn((L, B, n_cap, Hkv, D), generator=g).to(torch.bfloat16)
    V = torch.randn((L, B, n_cap, Hkv, D), generator=g).to(torch.bfloat16)
    q = torch.randn((L, B, 1, Hq, D), generator=g).to(torch.bfloat16)
    idx, counts = _full_lists(B, n_ctx, n_cap)
    out, lse = clsa.sparse_attn(q.to(DEV), K.to(DEV), V.to(DEV), idx.to(DEV), counts.to(DEV),
                                want_lse=True)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(D)
    G = Hq // Hkv
    err = 0.0
    for l in range(L):
        for b in range(B):
            n = n_ctx[b]
            Kd, Vd = f64(K[l, b, :n]), f64(V[l, b, :n])
            for h in range(Hq):
                o, o_lse = O.attend_head(f64(q[l, b, 0, h]), Kd[:, h // G], Vd[:, h // G], scale)
                err = max(err, float(np.max(np.abs(f64(out[l, b, 0, h]) - o))))
                assert abs(float(lse[l, b, 0, h]) - o_lse) <= 1e-3
    assert err <= 2e-2, err


def test_per_layer_routing_pipeline():
    # L layers, each with its own routing keys and query: one routing call
    # over L*B key sets, then one attention call per layer on its own lists
    g = _gen(310)
    L, B, n, d, k = 3, 2, 9000, 64, 512
    Hq, Hkv, D = 8, 4, 128
    K_idx = torch.randn((L * B, n, d), generator=g).to(torch.bfloat16)
    q_idx = (torch.randn((L * B, 1, d), generator=g) / 8).to(torch.bfloat16)
    K = torch.randn((L, B, n, Hkv, D), generator=g).to(torch.bfloat16)
    V = torch.randn((L, B, n, Hkv, D), generator=g).to(torch.bfloat16)
    q = torch.randn((L, B, 1, Hq, D), generator=g).to(torch.bfloat16)
    idx, counts = clsa.route(q_idx.to(DEV), K_idx.to(DEV), k)
    Kd, Vd, qd = K.to(DEV), V.to(DEV), q.to(DEV)
    outs = []
    for l in range(L):
        o, _ = clsa.sparse_attn(qd[l:l + 1], Kd[l:l + 1], Vd[l:l + 1],
                                idx[l * B:(l + 1) * B], counts[l * B:(l + 1) * B])
        outs.append(o)
    torch.cuda.synchronize()
    gi, gc = idx.cpu().numpy(), counts.cpu().numpy()
    qn, Kn = f64(q_idx), f64(K_idx)
    scale = 1.0 / math.sqrt(D)
    G = Hq // Hkv
    compared = 0
    for l in range(L):
        for b in range(B):
            r = l * B + b
            s = O.route_scores(qn[r, 0], Kn[r], n)
            sel = O.topk_select(s, k)
            o_idx = np.full(k, -1)
            o_idx[:len(sel)] = sel
            check_topk_row(gi[r, 0], int(gc[r, 0]), o_idx, len(sel), s, k)
            # attention over this layer's own list as the GPU routed it
            gsel = torch.from_numpy(gi[r, 0, : int(gc[r, 0])].astype(np.int64))
            Kl, Vl = f64(K[l, b][gsel]), f64(V[l, b][gsel])
            for h in range(Hq):
                o_ref, _ = O.attend_head(f64(q[l, b, 0, h]), Kl[:, h // G], Vl[:, h // G], scale)
                assert np.max(np.abs(f64(outs[l][0, b, 0, h]) - o_ref)) <= 2e-2
                compared += 1
    assert compared == L * B * Hq
