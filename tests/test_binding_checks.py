"""The Python binding's own argument checks, on the CPU.

The C ABI sees only pointers and sizes, so a tensor of the wrong shape or
dtype would make a kernel read or write outside its buffer.  The binding
compares the tensors it is given with each other and raises before it
marshals anything; these tests pass CPU tensors, which would be refused
later anyway, and check that the shape or dtype error comes first."""
from __future__ import annotations

import os

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "long_context_sparse_routing_amd", "libclsa.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libclsa.so not built")

bf = torch.bfloat16


def _route_args():
    return torch.zeros((2, 1, 64), dtype=bf), torch.zeros((2, 100, 64), dtype=bf)


@pytest.mark.parametrize("fn", ["prepare_route", "prepare_route_static"])
@pytest.mark.parametrize("bad,exc,msg", [
    (dict(K_idx=torch.zeros((3, 100, 64), dtype=bf)), ValueError, "does not match"),
    (dict(K_idx=torch.zeros((2, 100, 32), dtype=bf)), ValueError, "does not match"),
    (dict(K_idx=torch.zeros((2, 100, 64))), TypeError, "K_idx is"),
    (dict(q_idx=torch.zeros((2, 64), dtype=bf)), ValueError, "q_idx must be"),
    (dict(n_ctx=torch.zeros(3, dtype=torch.int32)), ValueError, "n_ctx has shape"),
    (dict(n_ctx=torch.zeros(2, dtype=torch.int64)), TypeError, "n_ctx must be int32"),
    (dict(idx=torch.zeros((2, 1, 8), dtype=torch.int32)), ValueError, "idx has shape"),
    (dict(counts=torch.zeros((2, 1), dtype=torch.int64)), TypeError, "counts must be int32"),
])
def test_route_checks(fn, bad, exc, msg):
    from long_context_sparse_routing_amd import binding
    q, K = _route_args()
    kw = dict(q_idx=q, K_idx=K, k=16)
    kw.update(bad)
    with pytest.raises(exc, match=msg):
        getattr(binding, fn)(**kw)


def test_route_threshold_checks():
    from long_context_sparse_routing_amd import binding
    q, K = _route_args()
    with pytest.raises(ValueError, match="tau has shape"):
        binding.prepare_route_threshold(q, K, torch.zeros((3, 1)), 64)
    with pytest.raises(TypeError, match="tau must be float32"):
        binding.prepare_route_threshold(q, K, torch.zeros((2, 1), dtype=torch.float64), 64)


def _attn_args(L=2, B=2, M=1, Hq=8, Hkv=2, D=64, n=50, cap=16):
    q = torch.zeros((L, B, M, Hq, D), dtype=bf)
    K = torch.zeros((L, B, n, Hkv, D), dtype=bf)
    V = torch.zeros_like(K)
    idx = torch.zeros((B, M, cap), dtype=torch.int32)
    counts = torch.zeros((B, M), dtype=torch.int32)
    return dict(q=q, K=K, V=V, idx=idx, counts=counts)


@pytest.mark.parametrize("bad,exc,msg", [
    (dict(K=torch.zeros((2, 1, 50, 2, 64), dtype=bf)), ValueError, r"K\[0\] has shape"),
    (dict(V=torch.zeros((2, 2, 49, 2, 64), dtype=bf)), ValueError, r"V\[0\] has shape"),
    (dict(K=[torch.zeros((2, 50, 2, 64), dtype=bf), torch.zeros((2, 50, 2, 32), dtype=bf)]),
     ValueError, r"K\[1\] has shape"),
    (dict(V=torch.zeros((2, 2, 50, 2, 64))), TypeError, "share one dtype"),
    (dict(idx=torch.zeros((2, 1, 16), dtype=torch.int64)), TypeError, "idx must be int32"),
    (dict(idx=torch.zeros((1, 1, 16), dtype=torch.int32)), ValueError, "idx has shape"),
    (dict(counts=torch.zeros((2, 2), dtype=torch.int32)), ValueError, "counts has shape"),
    (dict(out=torch.zeros((2, 2, 1, 8, 32), dtype=bf)), ValueError, r"out\[0\] has shape"),
    (dict(out=torch.zeros((2, 2, 1, 8, 64))), TypeError, r"out\[0\] is"),
    (dict(out=torch.zeros((1, 2, 1, 8, 64), dtype=bf)), ValueError, "out has 1 layers"),
])
def test_attn_checks(bad, exc, msg):
    from long_context_sparse_routing_amd import binding
    kw = _attn_args()
    kw.update(bad)
    with pytest.raises(exc, match=msg):
        binding.prepare_sparse_attn(**kw)


def test_kv_append_checks():
    from long_context_sparse_routing_amd import binding
    L, B, n, Hkv, D, d = 2, 3, 40, 2, 64, 32
    K = torch.zeros((L, B, n, Hkv, D), dtype=bf)
    V = torch.zeros_like(K)
    sk = torch.zeros((L, B, Hkv, D), dtype=bf)
    ki = torch.zeros((B, n, d), dtype=bf)
    si = torch.zeros((B, d), dtype=bf)
    pos = torch.zeros(B, dtype=torch.int32)
    with pytest.raises(ValueError, match="has shape"):  # pos sets B
        binding.prepare_kv_append(torch.zeros(B + 1, dtype=torch.int32), si, ki, sk, K, sk, V)
    with pytest.raises(ValueError, match=r"src_k\[0\] has shape"):
        binding.prepare_kv_append(pos, si, ki, torch.zeros((L, B, Hkv, 32), dtype=bf), K, sk, V)
    with pytest.raises(ValueError, match="src_idx has shape"):
        binding.prepare_kv_append(pos, torch.zeros((B, 16), dtype=bf), ki, sk, K, sk, V)
    with pytest.raises(ValueError, match="go together"):
        binding.prepare_kv_append(pos, None, ki, sk, K, sk, V)
    with pytest.raises(TypeError, match="share one dtype"):
        binding.prepare_kv_append(pos, si, ki, sk.float(), K, sk, V)
