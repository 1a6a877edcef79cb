"""Seeded synthetic inputs for the shared-routing decode workloads.

This module only draws random tensors with the shapes and value
distributions of the workloads; it computes none of the routing, selection
or attention steps.  Both the HIP path and the CPU oracle receive the same
tensors from it.  The one recipe that needs routing scores (threshold
placement for the threshold-mode workload) takes the scoring function as an
argument, so that the scores come from the caller's oracle, not from here.

Workload shapes follow the pages' operating point: 128K-token contexts,
k = 2048 routed tokens and 16 cross-decoder layers sharing one routing
(CLSA explainer, ai-papers.net, sections "CLSAの仕組み" and
"推論速度の改善結果"), and the half-space threshold mode of the Louver
summary (gist.science, section "1. 半空間範囲検索への帰着").  The pages
measure on public datasets and trained models; seeded Gaussian tensors of
the same shapes stand in for them.
"""
from __future__ import annotations

import dataclasses
import math
import zlib
from dataclasses import dataclass

import torch

__all__ = [
    "Workload",
    "WORKLOADS",
    "seed_of",
    "make_generator",
    "gen_routing_keys",
    "gen_routing_query",
    "gen_kv",
    "gen_attn_query",
    "gen_threshold_inputs",
    "threshold_counts",
    "torch_dtype",
    "gen_append_rows",
    "gen_prompt_routing_queries",
]


@dataclass(frozen=True)
class Workload:
    """Shapes of one synthetic workload.

    B sequences, M query rows per sequence (1 in decode), n_ctx visible keys
    (n_cap slots allocated, so decode steps can append), d routing dim,
    L layers, Hq/Hkv query/KV heads, D head dim, k routed tokens (None means
    threshold mode), dtype "f32" or "bf16", planted keys per sequence,
    q_pos0 >= 0 for a prefill chunk, steps decode steps.
    """

    name: str
    B: int
    M: int
    n_ctx: int
    n_cap: int
    d: int
    L: int
    Hq: int
    Hkv: int
    D: int
    k: int | None
    dtype: str
    planted: int
    q_pos0: int = -1
    steps: int = 1
    base_seed: int = 1000

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # Tiny single decode step in fp32.
    "tiny_fp32_4k": Workload("tiny_fp32_4k", B=1, M=1, n_ctx=4096, n_cap=4096, d=32, L=1,
                             Hq=1, Hkv=1, D=64, k=256, dtype="f32", planted=16,
                             base_seed=1001),
    # Decode at 32K context, one sequence.
    "decode_32k": Workload("decode_32k", B=1, M=1, n_ctx=32768, n_cap=32768 + 64, d=64, L=16,
                           Hq=32, Hkv=8, D=128, k=2048, dtype="bf16", planted=256,
                           steps=64, base_seed=1002),
    # Decode at 128K context, 8 sequences, 64 steps each appending one row.
    "decode_128k_b8": Workload("decode_128k_b8", B=8, M=1, n_ctx=131072, n_cap=131072 + 64,
                               d=64, L=16, Hq=32, Hkv=8, D=128, k=2048, dtype="bf16",
                               planted=512, steps=64, base_seed=1003),
    # Prefill chunk of 4096 queries at positions 126976..131071.
    "prefill_128k_c4096": Workload("prefill_128k_c4096", B=1, M=4096, n_ctx=131072,
                                   n_cap=131072, d=64, L=16, Hq=32, Hkv=8, D=128, k=2048,
                                   dtype="bf16", planted=0, q_pos0=131072 - 4096,
                                   base_seed=1004),
    # Threshold (half-space) selection, 16 sequences.
    "threshold_128k_b16": Workload("threshold_128k_b16", B=16, M=1, n_ctx=131072,
                                   n_cap=131072, d=128, L=16, Hq=32, Hkv=8, D=128, k=None,
                                   dtype="bf16", planted=0, base_seed=1005),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def seed_of(base: int, *tags) -> int:
    """Deterministic 63-bit seed for (base, tags...)."""
    h = zlib.crc32(repr((base,) + tuple(tags)).encode())
    return (base * 1_000_003 + h) & 0x7FFF_FFFF_FFFF_FFFF


def make_generator(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, gen, device, dtype=torch.float32):
    return torch.randn(*shape, generator=gen, device=device, dtype=dtype)


def gen_routing_keys(wl: Workload, device, seed: int | None = None):
    """Routing keys K_idx [B, n_cap, d] plus the per-sequence base direction.

    Every row ~ N(0, 1).  The base direction u_b ~ N(0,1)/sqrt(d).  When the
    workload plants keys, `planted` rows per sequence (uniform without
    replacement over the first n_ctx rows) get 3 * u_b / |u_b| added, so
    that they score about 3 above the bulk against queries near u_b.
    Returns (K_idx in the workload dtype, u [B, d] float32, planted [B, P]).
    """
    base = wl.base_seed if seed is None else seed
    g = make_generator(device, seed_of(base, "K_idx"))
    K = _randn((wl.B, wl.n_cap, wl.d), g, device)
    gu = make_generator(device, seed_of(base, "u"))
    u = _randn((wl.B, wl.d), gu, device) / math.sqrt(wl.d)
    planted = torch.zeros((wl.B, 0), dtype=torch.int64, device=device)
    if wl.planted > 0:
        gp = make_generator(device, seed_of(base, "planted"))
        rows = []
        for b in range(wl.B):
            perm = torch.randperm(wl.n_ctx, generator=gp, device=device)[: wl.planted]
            rows.append(perm)
        planted = torch.stack(rows)
        uh = u / u.norm(dim=1, keepdim=True)
        for b in range(wl.B):
            K[b, planted[b]] += 3.0 * uh[b]
    return K.to(torch_dtype(wl.dtype)).contiguous(), u, planted


def gen_routing_query(wl: Workload, u, step: int, device, seed: int | None = None):
    """Routing queries q_idx [B, M, d] for decode step `step`.

    Decode workloads with planted keys: q = u_b + 0.3 * N(0,1)/sqrt(d), so the
    planted keys stay relevant while the rest of the selection changes from
    step to step.  The tiny workload (one step) uses q = u_b itself.  Other
    workloads: q ~ N(0,1)/sqrt(d) per row.
    """
    base = wl.base_seed if seed is None else seed
    g = make_generator(device, seed_of(base, "q_idx", step))
    noise = _randn((wl.B, wl.M, wl.d), g, device) / math.sqrt(wl.d)
    if wl.planted > 0 and wl.M == 1:
        if wl.steps == 1:
            q = u[:, None, :].clone()
        else:
            q = u[:, None, :] + 0.3 * noise
    else:
        q = noise
    return q.to(torch_dtype(wl.dtype)).contiguous()


def gen_kv(wl: Workload, device, seed: int | None = None, layers=None):
    """Per-layer K and V caches, each [L, B, n_cap, Hkv, D] ~ N(0, 1).

    One tensor per cache so that layer l is the contiguous slice [l].
    """
    base = wl.base_seed if seed is None else seed
    dt = torch_dtype(wl.dtype)
    lays = range(wl.L) if layers is None else layers
    Kc = torch.empty((wl.L, wl.B, wl.n_cap, wl.Hkv, wl.D), dtype=dt, device=device)
    Vc = torch.empty_like(Kc)
    for l in lays:
        Kc[l].normal_(generator=make_generator(device, seed_of(base, "K", l)))
        Vc[l].normal_(generator=make_generator(device, seed_of(base, "V", l)))
    return Kc, Vc


def gen_attn_query(wl: Workload, q_idx, step: int, device, seed: int | None = None):
    """Attention queries q [L, B, M, Hq, D].

    q_base[h] = W_h q_idx with a seeded W_h ~ N(0,1) of shape [D, d] (a
    fixed random projection of the routing query), and layer l uses
    q_base + 0.3 * N(0,1) (fresh per layer and step), so one routing list
    is meaningful for every layer.  The tiny single-layer workload uses
    q = W q_idx with no noise.
    """
    base = wl.base_seed if seed is None else seed
    gw = make_generator(device, seed_of(base, "W"))
    W = _randn((wl.Hq, wl.D, wl.d), gw, device)
    qi = q_idx.to(torch.float32)
    q_base = torch.einsum("hed,bmd->bmhe", W, qi)
    out = torch.empty((wl.L, wl.B, wl.M, wl.Hq, wl.D), dtype=torch_dtype(wl.dtype), device=device)
    for l in range(wl.L):
        if wl.L == 1 and wl.steps == 1 and wl.planted > 0:
            out[l] = q_base.to(out.dtype)
        else:
            g = make_generator(device, seed_of(base, "q", l, step))
            out[l] = (q_base + 0.3 * _randn(q_base.shape, g, device)).to(out.dtype)
    return out


def threshold_counts(B: int, lo: int = 256, hi: int = 8192):
    """Target set sizes c_b = round(lo * (hi/lo)^(b/(B-1))), from lo to hi."""
    if B == 1:
        return [lo]
    r = hi / lo
    return [int(round(lo * r ** (b / (B - 1)))) for b in range(B)]


def gen_threshold_inputs(wl: Workload, score_fn, device="cpu", seed: int | None = None,
                         margin: float = 1e-4, counts=None, max_rounds: int = 50,
                         clusters: int = 0, sigma: float = 0.05):
    """Routing keys, queries and per-row thresholds for threshold mode.

    score_fn(q_row_f64, K_rows_f64) -> float64 scores; the caller supplies
    it (the oracle's scoring), so this module does no scoring itself.
    tau_b is the midpoint between the c_b-th and (c_b+1)-th largest scores,
    then any key within `margin` of tau_b is redrawn (seeded) until none is.
    Keys are N(0, 1), or with clusters > 0 a mixture: each sequence draws
    `clusters` centers ~ N(0, 1) and every key is a uniformly chosen center
    plus sigma * N(0, 1) (a redrawn key keeps its center).  Trained models'
    keys cluster (the structure an index over them relies on); Gaussian keys
    do not, and the mixture stands in for the former.
    Returns (K_idx [B, n_cap, d], q_idx [B, 1, d], tau [B, 1] float32).
    Generation runs on the CPU; move the tensors afterwards.
    """
    import numpy as np

    base = wl.base_seed if seed is None else seed
    dt = torch_dtype(wl.dtype)
    g = make_generator("cpu", seed_of(base, "K_idx", clusters, sigma) if clusters else
                       seed_of(base, "K_idx"))
    if clusters > 0:
        cent = torch.randn((wl.B, clusters, wl.d), generator=g)
        assign = torch.randint(0, clusters, (wl.B, wl.n_cap), generator=g)
        K = torch.gather(cent, 1, assign[..., None].expand(-1, -1, wl.d))
        K = (K + sigma * torch.randn((wl.B, wl.n_cap, wl.d), generator=g)).to(dt)
    else:
        K = torch.randn((wl.B, wl.n_cap, wl.d), generator=g).to(dt)
    gq = make_generator("cpu", seed_of(base, "q_idx", 0))
    q = (torch.randn((wl.B, 1, wl.d), generator=gq) / math.sqrt(wl.d)).to(dt)
    cnt = threshold_counts(wl.B) if counts is None else list(counts)
    tau = torch.zeros((wl.B, 1), dtype=torch.float32)
    gr = make_generator("cpu", seed_of(base, "redraw"))
    for b in range(wl.B):
        qb = q[b, 0].to(torch.float64).numpy()
        Kb = K[b, : wl.n_ctx].to(torch.float64).numpy()
        s = score_fn(qb, Kb)
        c = min(max(int(cnt[b]), 1), wl.n_ctx - 1)
        srt = np.sort(s)[::-1]
        t = np.float32(0.5 * (srt[c - 1] + srt[c]))
        tau[b, 0] = float(t)
        t64 = float(t)
        for _ in range(max_rounds):
            near = np.flatnonzero(np.abs(s - t64) < margin)
            if near.size == 0:
                break
            fresh = torch.randn((near.size, wl.d), generator=gr)
            if clusters > 0:
                fresh = cent[b, assign[b, torch.from_numpy(near)]] + sigma * fresh
            fresh = fresh.to(dt)
            K[b, torch.from_numpy(near)] = fresh
            s[near] = score_fn(qb, fresh.to(torch.float64).numpy())
        else:
            raise RuntimeError("threshold margin could not be cleared")
    return K.contiguous(), q.contiguous(), tau


def gen_append_rows(wl: Workload, steps: int, device, seed: int | None = None):
    """Rows appended by decode steps: K_idx rows [steps, B, d] and K/V rows
    [steps, L, B, Hkv, D], all ~ N(0, 1) in the workload dtype."""
    base = wl.base_seed if seed is None else seed
    dt = torch_dtype(wl.dtype)
    g = make_generator(device, seed_of(base, "append"))
    new_kidx = _randn((steps, wl.B, wl.d), g, device).to(dt)
    new_k = _randn((steps, wl.L, wl.B, wl.Hkv, wl.D), g, device, dtype=dt)
    new_v = _randn((steps, wl.L, wl.B, wl.Hkv, wl.D), g, device, dtype=dt)
    return new_kidx, new_k, new_v


def gen_prompt_routing_queries(wl: Workload, u, M: int, device, seed: int | None = None):
    """Routing queries of the prompt that preceded a decode workload:
    [B, M, d], drawn like that workload's decode queries (u_b + 0.3 *
    N(0,1)/sqrt(d)), so a table built from them at prefill describes the
    decode steps' queries."""
    base = wl.base_seed if seed is None else seed
    g = make_generator(device, seed_of(base, "prompt_q_idx", M))
    noise = _randn((wl.B, M, wl.d), g, device) / math.sqrt(wl.d)
    return (u[:, None, :] + 0.3 * noise).to(torch_dtype(wl.dtype)).contiguous()
