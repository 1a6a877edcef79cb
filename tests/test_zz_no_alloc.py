"""GPU test of clsa_route_static, the routing entry point that allocates
nothing: its results must equal clsa_route's on the same inputs, bit for
bit (both run the same kernels), on two calls in a row whose second one is
smaller, so that the second runs on a scratch array still holding the
first call's contents.  The shapes cover the three routing paths: decode
rows on bf16 keys (sampled threshold, filtered scan, select), fp32 rows
(exhaustive scan) and a block of 64 causal bf16 rows (matrix cores)."""
from __future__ import annotations

import math

import pytest
import torch

from long_context_sparse_routing_amd import binding as clsa

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _inputs(seed, B, M, n, d, dtype):
    g = torch.Generator()
    g.manual_seed(seed)
    K = torch.randn((B, n, d), generator=g).to(dtype)
    q = (torch.randn((B, M, d), generator=g) / math.sqrt(d)).to(dtype)
    return q.to(DEV), K.to(DEV)


@pytest.mark.parametrize("first,second", [
    # (B, M, n, d, k, dtype, q_pos0): decode rows, the larger call first
    ((32, 1, 131072, 64, 2048, torch.bfloat16, -1), (3, 1, 20000, 64, 1024, torch.bfloat16, -1)),
    ((2, 1, 60000, 128, 2048, torch.bfloat16, -1), (1, 1, 5000, 32, 256, torch.bfloat16, -1)),
    ((1, 1, 40000, 32, 2048, torch.float32, -1), (1, 1, 4096, 32, 256, torch.float32, -1)),
    ((1, 64, 12000, 64, 512, torch.bfloat16, 11936), (1, 64, 6000, 64, 256, torch.bfloat16, 5936)),
])
def test_static_route_matches_route(first, second):
    for i, (B, M, n, d, k, dtype, q_pos0) in enumerate((first, second)):
        q, K = _inputs(900 + 17 * i + n, B, M, n, d, dtype)
        n_ctx = torch.tensor([n - 7 * b for b in range(B)], dtype=torch.int32, device=DEV)
        cap = k + 3
        ref_idx, ref_cnt = clsa.route(q, K, k, n_ctx=n_ctx, q_pos0=q_pos0, cap=cap)
        idx = torch.full((B, M, cap), 123, dtype=torch.int32, device=DEV)
        cnt = torch.full((B, M), 123, dtype=torch.int32, device=DEV)
        st_idx, st_cnt = clsa.route_static(q, K, k, n_ctx=n_ctx, q_pos0=q_pos0, cap=cap,
                                           idx=idx, counts=cnt)
        torch.cuda.synchronize()
        print(f"static route call {i}: B={B} M={M} n={n} d={d} k={k} {dtype}", flush=True)
        assert torch.equal(st_cnt, ref_cnt)
        assert torch.equal(st_idx, ref_idx)
        assert int(st_cnt.min()) == min(k, n - 7 * (B - 1)) or q_pos0 >= 0


def test_static_route_rejects_shapes_past_the_scratch_limit():
    # decode rows at 128K keys, k = 2048: 113 rows fit the array, 114 do not
    q, K = _inputs(5, 1, 1, 131072, 64, torch.bfloat16)
    qq = q.expand(114, 1, 64).contiguous()
    KK = K.expand(114, 131072, 64).contiguous()
    with pytest.raises(clsa.ClsaError) as e:
        clsa.route_static(qq, KK, 2048)
    assert e.value.status == -5
    idx, cnt = clsa.route_static(qq[:113], KK[:113], 2048)
    torch.cuda.synchronize()
    ref_idx, _ = clsa.route(qq[:113], KK[:113], 2048)
    assert torch.equal(idx, ref_idx)
