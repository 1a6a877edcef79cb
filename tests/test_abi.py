"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/clsa.h, sizes workspaces, and rejects bad arguments on
the host before anything is enqueued (so no device pointer is touched)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "clsa.h")
LIB = os.path.join(ROOT, "long_context_sparse_routing_amd", "libclsa.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libclsa.so not built")

OK, INVALID, WORKSPACE, DTYPE = 0, -1, -2, -3
F32, BF16 = 0, 1
FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails first
NULL = ctypes.c_void_p(None)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(clsa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import torch  # noqa: F401  (bind to the HIP runtime torch loads)
    from long_context_sparse_routing_amd.binding import load_library
    return load_library()


def test_header_declares_the_boundary():
    fns = declared_functions()
    for f in ("clsa_route", "clsa_route_threshold", "clsa_sparse_attn",
              "clsa_route_workspace_size", "clsa_route_threshold_workspace_size",
              "clsa_sparse_attn_workspace_size", "clsa_status_string", "clsa_version"):
        assert f in fns


def test_every_declared_symbol_is_exported(lib):
    for f in declared_functions():
        assert hasattr(lib, f), f
    out = os.popen(f"nm -D --defined-only {LIB}").read()
    for f in declared_functions():
        assert re.search(rf"\bT {f}\b", out), f


def test_version_and_status_strings(lib):
    assert lib.clsa_version() == 1
    for s in (0, -1, -2, -3, -4, 17):
        assert isinstance(lib.clsa_status_string(s), bytes)
    assert lib.clsa_status_string(-2) == b"workspace too small"


def test_route_workspace_sizes(lib):
    small = lib.clsa_route_workspace_size(1, 1, 64, 4096, 256, 256, BF16)
    big = lib.clsa_route_workspace_size(8, 1, 64, 131136, 2048, 2048, BF16)
    assert 0 < small < big
    # bf16 rows with k <= 2048: per row 4096 sampled 2-byte key prefixes, a
    # count and a list of 6144 8-byte candidates, whatever the context length
    assert big >= 8 * (4096 * 2 + 6144 * 8)
    assert big == lib.clsa_route_workspace_size(8, 1, 64, 262144, 2048, 2048, BF16)
    # otherwise (fp32, or k > 2048) keys (4 B) and candidates (8 B) per key
    for dt, k in ((F32, 2048), (BF16, 4096)):
        assert lib.clsa_route_workspace_size(8, 1, 64, 131136, k, k, dt) >= 8 * 131136 * 12
    assert lib.clsa_route_workspace_size(1, 1, 48, 4096, 256, 256, BF16) == 0  # bad d
    assert lib.clsa_route_threshold_workspace_size(16, 1, 128, 131072, 16384, BF16) > 0
    # a block of query rows on bf16 keys: sampled keys and candidate segments
    blk = lib.clsa_route_workspace_size(1, 4096, 128, 131136, 2048, 2048, BF16)
    assert blk >= 4096 * 131136 * 8
    assert lib.clsa_route_workspace_size(1, 4096, 128, 131136, 2048, 2048, F32) > 0


def test_attn_workspace_sizes(lib):
    # one sequence is too few workgroups: its lists are split and need
    # partials; 8 sequences x 8 KV heads x 16 layers fill the chip unsplit
    assert lib.clsa_sparse_attn_workspace_size(16, 1, 1, 32, 8, 128, 2048, BF16) > 0
    assert lib.clsa_sparse_attn_workspace_size(16, 8, 1, 32, 8, 128, 2048, BF16) == 0
    assert lib.clsa_sparse_attn_workspace_size(16, 1, 4096, 32, 8, 128, 2048, BF16) == 0
    assert lib.clsa_sparse_attn_workspace_size(1, 1, 1, 4, 2, 64, 300, F32) > 0  # VALU path
    assert lib.clsa_sparse_attn_workspace_size(16, 8, 1, 30, 8, 128, 2048, BF16) == 0  # Hq%Hkv


def _route(lib, q=FAKE, K=FAKE, B=1, M=1, d=64, n_cap=4096, k=256, dt=BF16, idx=FAKE,
           counts=FAKE, cap=256, ws=FAKE, ws_bytes=1 << 40):
    return lib.clsa_route(q, K, B, M, d, n_cap, NULL, -1, k, dt, idx, counts, cap, ws, ws_bytes,
                          NULL)


@pytest.mark.parametrize("kw,want", [
    (dict(q=NULL), INVALID), (dict(K=NULL), INVALID), (dict(idx=NULL), INVALID),
    (dict(counts=NULL), INVALID), (dict(B=0), INVALID), (dict(M=0), INVALID),
    (dict(d=48), INVALID), (dict(n_cap=0), INVALID), (dict(k=0), INVALID),
    (dict(cap=100), INVALID), (dict(dt=7), DTYPE), (dict(ws=NULL), WORKSPACE),
    (dict(ws_bytes=1024), WORKSPACE), (dict(B=70000), INVALID),
])
def test_route_rejects(lib, kw, want):
    assert _route(lib, **kw) == want


def test_route_threshold_rejects(lib):
    f = lib.clsa_route_threshold
    assert f(FAKE, FAKE, 1, 1, 64, 4096, NULL, -1, NULL, BF16, FAKE, FAKE, 64, FAKE, 1 << 40,
             NULL) == INVALID  # tau
    assert f(FAKE, FAKE, 1, 1, 64, 4096, NULL, -1, FAKE, BF16, FAKE, FAKE, 0, FAKE, 1 << 40,
             NULL) == INVALID  # cap
    assert f(FAKE, FAKE, 1, 1, 64, 4096, NULL, -1, FAKE, BF16, FAKE, FAKE, 64, FAKE, 16,
             NULL) == WORKSPACE


def _attn(lib, L=2, B=1, M=1, Hq=32, Hkv=8, D=128, cap=2048, scale=0.0, dt=BF16, ptrs=None,
          ws=FAKE, ws_bytes=1 << 40, idx=FAKE):
    arr = ctypes.c_void_p * max(L, 1)
    p = ptrs if ptrs is not None else [0x100000] * max(L, 1)
    a = arr(*p)
    return lib.clsa_sparse_attn(L, B, M, Hq, Hkv, D, a, a, a, 131072, idx, FAKE, cap,
                                ctypes.c_float(scale), dt, a, NULL, ws, ws_bytes, NULL)


@pytest.mark.parametrize("kw,want", [
    (dict(L=0), INVALID), (dict(L=65), INVALID), (dict(Hq=30), INVALID),
    (dict(Hq=64, Hkv=2), INVALID), (dict(D=130), INVALID), (dict(D=264), INVALID),
    (dict(cap=0), INVALID), (dict(scale=-1.0), INVALID), (dict(dt=5), DTYPE),
    (dict(ptrs=[0x100000, 0]), INVALID), (dict(idx=NULL), INVALID),
    (dict(ws=NULL), WORKSPACE), (dict(ws_bytes=8), WORKSPACE),
])
def test_attn_rejects(lib, kw, want):
    assert _attn(lib, **kw) == want


def test_kv_append_rejects(lib):
    arr = ctypes.c_void_p * 2
    a = arr(0x100000, 0x100000)
    f = lib.clsa_kv_append
    assert f(2, 8, 8, 128, 64, 4096, NULL, FAKE, FAKE, a, a, a, a, BF16, NULL) == INVALID  # pos
    assert f(2, 8, 8, 128, 64, 4096, FAKE, FAKE, NULL, a, a, a, a, BF16, NULL) == INVALID
    assert f(2, 8, 8, 128, 12, 4096, FAKE, FAKE, FAKE, a, a, a, a, BF16, NULL) == INVALID  # d
    assert f(65, 8, 8, 128, 64, 4096, FAKE, FAKE, FAKE, a, a, a, a, BF16, NULL) == INVALID
    assert f(2, 8, 8, 128, 64, 4096, FAKE, FAKE, FAKE, a, a, a, a, 9, NULL) == DTYPE
    bad = arr(0x100000, 0)
    assert f(2, 8, 8, 128, 64, 4096, FAKE, FAKE, FAKE, a, bad, a, a, BF16, NULL) == INVALID


def test_binding_fails_loudly_without_library(tmp_path):
    from long_context_sparse_routing_amd import binding
    with pytest.raises(RuntimeError, match="not found"):
        binding.load_library(str(tmp_path / "missing.so"))


def test_bench_refuses_more_than_one_gpu():
    # the benchmark measures one GPU; asking for more exits with status 2
    # and says why, before touching any device
    import subprocess
    import sys
    from pathlib import Path
    root = Path(__file__).resolve().parents[1]
    res = subprocess.run([sys.executable, str(root / "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""
