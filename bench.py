#!/usr/bin/env python3
"""Decode benchmark: shared-routing sparse attention at 128K context.

Workload (decode_128k_b8): 8 independent sequences at 131072 tokens, one
routing step per sequence per decode step (d_idx = 64, bf16, top-2048)
shared by 16 layers of GQA attention (32 query / 8 KV heads, head dim 128,
bf16).  Each step appends one K_idx/K/V row per sequence (the KV cache the
self-decoder would write), routes, and attends in all 16 layers: one pass of
the whole hot path.  Inputs are seeded synthetic tensors already resident in
HBM when timing starts.

Prints one JSON line: decode tokens/s (8 tokens per step), the step's
fraction of HBM peak, the attention kernel against the HBM roofline, and the
CPU oracle timed on a bounded sample of the same workload.  A second leg
times routing of one 4096-token prefill chunk at 128K context (the score
matrix on the matrix cores) against the bf16 MFMA roofline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.0  # MI355X dense bf16: 256 CUs x 2.4 GHz x 4096 flop/clk
ROOT = os.path.dirname(os.path.abspath(__file__))
ATTN_PROFILE = os.path.join(ROOT, "profiles", "attn_bf16_decode_128k_b8.md")
ATTN_SOURCES = ["long_context_sparse_routing_amd/csrc/clsa_attn.hip",
                "long_context_sparse_routing_amd/csrc/clsa_common.h"]


def profiled_traffic():
    """HBM bytes per attention launch measured with rocprofv3 (FETCH_SIZE and
    WRITE_SIZE, calibrated on a plain copy) as recorded in the committed
    profile summary -- or None when the kernel sources changed since."""
    import hashlib
    try:
        text = open(ATTN_PROFILE).read()
    except OSError:
        return None
    m = hashlib.sha256()
    for p in ATTN_SOURCES:
        m.update(open(os.path.join(ROOT, p), "rb").read())
    digest = m.hexdigest()[:16]
    if f": {digest}" not in text:
        return None
    for line in text.splitlines():
        if line.startswith("traffic_bytes_per_launch:"):
            return float(line.split(":")[1])
    return None


def attn_bytes(L, B, M, Hq, Hkv, D, k, esize=2):
    """Algorithmic bytes of one sparse-attention launch: the gathered K and V
    rows (k per row, all KV heads, every layer), q in, out, index lists."""
    gathered = L * B * M * k * Hkv * D * esize * 2
    q_out = 2 * L * B * M * Hq * D * esize
    lists = B * M * (k + 1) * 4
    return gathered + q_out + lists


def route_bytes(B, M, n, d, k, esize=2):
    """Algorithmic bytes of one routing call: scan every visible routing key
    once, read the queries, write the index lists and counts."""
    return B * n * d * esize + B * M * d * esize + B * M * (k + 1) * 4


def per_layer_launches(wl, clsa, K_idx, Kc, Vc, q_idx_all, q_all, n_ctx_all, pos_all,
                       new_rows, steps, dev):
    """The decode steps with attention launched layer by layer.

    A model has layer l's query only after layer l-1's output, so a real
    step is append + one routing call + L single-layer attention calls with
    the rest of each layer in between.  The steps are the decode run's last
    `steps` ones again (their appends rewrite the same rows), launched
    eagerly with every call marshalled beforehand, as in the headline loop:
    capturing each step as HIP graphs measured slower on the MI355X.  One pass
    is timed by the wall clock; a second one brackets the L attention calls
    of every 4th step with HIP events (each recorded pair adds a few
    microseconds to its step).  A repeat of the last step must reproduce
    its outputs bit for bit."""
    import torch
    new_kidx, new_k, new_v = new_rows
    total = len(q_all)
    T = list(range(total - steps, total))
    s = torch.cuda.Stream()
    idx = torch.empty((wl.B, 1, wl.k), dtype=torch.int32, device=dev)
    counts = torch.empty((wl.B, 1), dtype=torch.int32, device=dev)
    out = torch.empty((wl.L, wl.B, 1, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
    ws_r = torch.empty(clsa.route_workspace_size(wl.B, 1, wl.d, wl.n_cap, wl.k, wl.k,
                                                 torch.bfloat16), dtype=torch.uint8, device=dev)
    ws_l = torch.empty(max(1, clsa.sparse_attn_workspace_size(1, wl.B, 1, wl.Hq, wl.Hkv, wl.D,
                                                              wl.k, torch.bfloat16)),
                       dtype=torch.uint8, device=dev)
    calls = []
    for t in T:
        pre = [clsa.prepare_kv_append(pos_all[t], new_kidx[t], K_idx, new_k[t], Kc, new_v[t], Vc,
                                      stream=s),
               clsa.prepare_route(q_idx_all[t], K_idx, wl.k, n_ctx=n_ctx_all[t], idx=idx,
                                  counts=counts, ws=ws_r, stream=s)]
        layers = [clsa.prepare_sparse_attn([q_all[t][l]], [Kc[l]], [Vc[l]], idx, counts,
                                           out=[out[l]], ws=ws_l, stream=s)
                  for l in range(wl.L)]
        calls.append((pre, layers))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in T]

    ev_every = 4

    def run(events):
        with torch.cuda.stream(s):
            for i, (pre, layers) in enumerate(calls):
                mark = events and i % ev_every == 0
                for c in pre:
                    c()
                if mark:
                    ev[i][0].record(s)
                for c in layers:
                    c()
                if mark:
                    ev[i][1].record(s)

    torch.cuda.synchronize()
    run(False)  # untimed pass; it ends with the last step's outputs
    s.synchronize()
    ref = (idx.clone(), out.clone())
    t0 = time.perf_counter()
    run(False)
    s.synchronize()
    wall = time.perf_counter() - t0
    same = torch.equal(idx, ref[0]) and torch.equal(out, ref[1])
    if not same:
        raise RuntimeError("a repeat of the per-layer steps changed the last step's outputs")
    run(True)
    s.synchronize()
    marked = [ev[i] for i in range(len(T)) if i % ev_every == 0]
    attn_ms = sum(a.elapsed_time(b) for a, b in marked) / len(marked)
    ms = wall * 1e3 / len(T)
    return {"steps": len(T), "ms_per_step": ms, "tokens_per_s": wl.B * len(T) / wall,
            "attn_ms_per_step": attn_ms, "attn_ms_per_layer": attn_ms / wl.L,
            "repeat_matches": same,
            "note": "append + route + one clsa_sparse_attn call per layer, launched eagerly; "
                    "attention time from events on every 4th step of a second pass; the "
                    "headline value launches the 16 layers' attention as one call"}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def oracle_decode_rate(wl, K_idx, Kc, Vc, q_idx, q, n_vis, select, budget_s, order=None,
                       threads=None, max_steps=256):
    """Time the CPU oracle (as written) on decode sequence-steps of one
    workload: fp64 routing scores over the sequence's visible keys, the
    selection select(b, scores), then attention in every layer and head over
    the selected rows.  Sequences are taken in `order`, round after round,
    until the budget is spent (or max_steps sequence-steps); host copies of
    the inputs happen before each clock starts.  threads=1 pins the BLAS
    pool to one thread."""
    import contextlib
    import numpy as np
    import torch
    from oracle import clsa_oracle as O
    limit = contextlib.nullcontext()
    if threads is not None:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=threads)
    with limit:
        used = _blas_threads()
        q_np = q_idx.double().cpu().numpy()
        qa = [q[l].double().cpu().numpy() for l in range(wl.L)]
        sc = 1.0 / math.sqrt(wl.D)
        G = wl.Hq // wl.Hkv
        done, t_tot, seqs = 0, 0.0, []
        order = list(order if order is not None else range(wl.B))
        for i in range(max_steps):
            b = order[i % len(order)]
            n = n_vis(b)
            K_np = K_idx[b, :n].double().cpu().numpy()
            t0 = time.perf_counter()
            sel = select(b, O.route_scores(q_np[b, 0], K_np, n))
            t_route = time.perf_counter() - t0
            selt = torch.from_numpy(np.asarray(sel, dtype=np.int64)).to(Kc.device)
            Kr = [Kc[l, b][selt].double().cpu().numpy() for l in range(wl.L)]
            Vr = [Vc[l, b][selt].double().cpu().numpy() for l in range(wl.L)]
            t0 = time.perf_counter()
            for l in range(wl.L):
                for h in range(wl.Hq):
                    O.attend_head(qa[l][b, 0, h], Kr[l][:, h // G, :], Vr[l][:, h // G, :], sc)
            t_tot += t_route + time.perf_counter() - t0
            done += 1
            if b not in seqs:
                seqs.append(b)
            if t_tot >= budget_s:
                break
    return done, t_tot, used, seqs


def cpu_baseline(wl, K_idx, Kc, Vc, q_idx, q, n, budget_s):
    """Time the CPU oracle (as written) on a bounded sample of decode
    sequence-steps: routing over all n keys plus attention in all layers."""
    from oracle import clsa_oracle as O
    affinity = len(os.sched_getaffinity(0))
    done, t_tot, used, _ = oracle_decode_rate(
        wl, K_idx, Kc, Vc, q_idx, q, lambda b: n, lambda b, s: O.topk_select(s, wl.k), budget_s)
    return {
        "value": done / t_tot,
        "unit": "tokens/s",
        "cores": used,
        "kind": "oracle",
        "sample": (f"{done} sequence-steps of {wl.name} (one decode token each: fp64 routing "
                   f"over {n} keys, exact top-{wl.k}, attention in {wl.L} layers x {wl.Hq} "
                   f"heads); NumPy BLAS threads={used}, affinity cpus={affinity}"),
    }


def prefill_cpu_baseline(wl, K_idx, q_idx, budget_s):
    """Time the CPU oracle (as written) routing rows of the prefill chunk,
    evenly spaced over the chunk, until the budget is spent."""
    from oracle import clsa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    K_np = K_idx[0].double().cpu().numpy()  # host copies: input preparation
    q_np = q_idx[0].double().cpu().numpy()
    done, t_tot = 0, 0.0
    for m in range(0, wl.M, 37):
        nv = O.visible_count(wl.n_ctx, wl.q_pos0, m)
        t0 = time.perf_counter()
        O.topk_select(O.route_scores(q_np[m], K_np, nv), wl.k)
        t_tot += time.perf_counter() - t0
        done += 1
        if t_tot >= budget_s:
            break
    return {"value": done / t_tot, "unit": "query tokens/s", "cores": blas_threads,
            "kind": "oracle",
            "sample": (f"{done} rows of {wl.name} (every 37th row from 0: fp64 scores over "
                       f"~{wl.n_ctx} keys, exact top-{wl.k}); NumPy BLAS threads={blas_threads}")}


def prefill_routing(calls, dev, cpu_budget, with_attention=True):
    """Route one prefill chunk (4096 rows at positions 126976.., 128K keys,
    d_idx 64, k 2048, causal) `calls` times; the score matrix runs on MFMA.
    With `with_attention`, also time the chunk's sparse attention."""
    import torch
    from long_context_sparse_routing_amd import binding as clsa
    from long_context_sparse_routing_amd import inputs as gen
    wl = gen.WORKLOADS["prefill_128k_c4096"]
    K_idx, u, _ = gen.gen_routing_keys(wl, dev)
    q_idx = gen.gen_routing_query(wl, u, 0, dev)
    call = clsa.prepare_route(q_idx, K_idx, wl.k, q_pos0=wl.q_pos0)
    # a longer settle than the decode legs': the matrix-core kernels reach
    # their working clocks later (calls after 25 ms of repeats still measure
    # a few percent slow)
    _settle(call, min_ms=200.0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(calls):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / calls
    # K_idx (16 MiB) stays cache-resident across back-to-back calls: the same
    # calls again, each timed alone after evicting the last-level cache
    cold_us = _mall_cold_ms([call] * calls) * 1e3
    idx, counts = call.result
    assert int(counts.min()) == wl.k and int(counts.max()) == wl.k
    n_scores = wl.B * sum(min(wl.n_ctx, wl.q_pos0 + m + 1) for m in range(wl.M))
    flops = 2.0 * wl.d * n_scores  # the causal score matrix
    tflops = flops / (us * 1e-6) / 1e12
    res = {"workload": wl.name, "rows": wl.B * wl.M, "n_ctx": wl.n_ctx, "q_pos0": wl.q_pos0,
           "k": wl.k, "d_idx": wl.d, "calls": calls, "us_per_call": us,
           "query_tokens_per_s": wl.B * wl.M / (us * 1e-6),
           "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                        "algorithmic_flops_per_call": flops,
                        "what": "whole clsa_route call (threshold, filter, select)"},
           "mall_cold": {"us_per_call": cold_us,
                         "frac": flops / (cold_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                         "how": "each call timed alone after a 512 MiB write"}}
    if not with_attention:
        if cpu_budget > 0:
            res["cpu_baseline"] = prefill_cpu_baseline(wl, K_idx, q_idx, cpu_budget)
        return res
    # sparse attention of the chunk over its routed lists, all 16 layers
    # (query-major: every row gathers its own k rows per layer)
    Kc, Vc = gen.gen_kv(wl, dev)
    q = gen.gen_attn_query(wl, q_idx, 0, dev)
    attn = clsa.prepare_sparse_attn(q, Kc, Vc, idx, counts)
    attn()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(2):
        attn()
    e1.record()
    torch.cuda.synchronize()
    a_ms = e0.elapsed_time(e1) / 2
    row_bytes = wl.Hkv * wl.D * 2 * 2  # K and V of one position, all KV heads
    gathered = wl.L * wl.B * wl.M * wl.k * row_bytes
    unique = wl.L * wl.B * wl.n_ctx * row_bytes
    res["attention"] = {
        "ms_per_call": a_ms, "layers": wl.L,
        "gathered_bytes": gathered, "gathered_GBs": gathered / (a_ms * 1e-3) / 1e9,
        "gathered_rate_over_hbm_peak": gathered / (a_ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "unique_row_bytes": unique,
        "unique_row_bound_ms": unique / (HBM_PEAK_GBS * 1e9) * 1e3,
        "note": ("query-major gather with cached loads: each K/V row is picked by about "
                 f"{wl.M * wl.k / wl.n_ctx:.0f} query rows per layer and repeats are served "
                 "from the caches, so the gathered rate can pass the HBM peak; a key-major "
                 "kernel could approach the unique-row bound")}
    del Kc, Vc, q, attn
    if cpu_budget > 0:
        res["cpu_baseline"] = prefill_cpu_baseline(wl, K_idx, q_idx, cpu_budget)
    return res


def baselines(wl, Kc, Vc, q, n, dev, steps, shared_ms):
    """The two designs the shared-routing path is compared with (CLSA
    explainer, sections on compute cost and inference speed), on the same
    caches and attention queries as the decode leg:
      dense     -- every one of the n visible keys attended in all layers
                   (the sparse attention call with the full position list);
      per-layer -- each layer routes with its own index keys and query (one
                   routing call over L*B key sets), then attends over its own
                   list (one attention launch, layers folded into the batch).
    Neither includes the one-row cache append of the decode step (4.5 us)."""
    import torch
    from long_context_sparse_routing_amd import binding as clsa
    from long_context_sparse_routing_amd import inputs as gen

    def timed(fn):
        _settle(fn)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    B, L = wl.B, wl.L
    idx_d = torch.full((B, 1, wl.n_cap), -1, dtype=torch.int32, device=dev)
    idx_d[:, 0, :n] = torch.arange(n, dtype=torch.int32, device=dev)
    counts_d = torch.full((B, 1), n, dtype=torch.int32, device=dev)
    dense = clsa.prepare_sparse_attn(q, Kc, Vc, idx_d, counts_d)
    dense_ms = timed(dense)
    dense_bytes = L * B * n * wl.Hkv * wl.D * 2 * 2
    del dense, idx_d

    wl_pl = wl.with_(name=wl.name + "_per_layer_keys", B=L * B, base_seed=wl.base_seed + 100)
    K_pl, u_pl, _ = gen.gen_routing_keys(wl_pl, dev)
    q_pl = gen.gen_routing_query(wl_pl, u_pl, 0, dev)
    n_pl = torch.full((L * B,), n, dtype=torch.int32, device=dev)
    route_pl = clsa.prepare_route(q_pl, K_pl, wl.k, n_ctx=n_pl)
    idx_pl, counts_pl = route_pl.result
    # layers folded into the batch: row l*B + b attends over layer l's cache
    # of sequence b with its own list, all in one launch
    fold = lambda t: t.reshape((1, L * B) + tuple(t.shape[2:]))
    attn_pl = clsa.prepare_sparse_attn(fold(q), fold(Kc), fold(Vc), idx_pl, counts_pl)

    def per_layer():
        route_pl()
        attn_pl()
    route_pl_ms = timed(route_pl)
    per_layer_ms = timed(per_layer)
    assert int(counts_pl.min()) == wl.k and int(counts_pl.max()) == wl.k
    del K_pl, attn_pl, route_pl
    return {
        "dense_attention": {"ms_per_step": dense_ms, "tokens_per_s": B / (dense_ms * 1e-3),
                            "bytes_per_step": dense_bytes,
                            "hbm_frac": dense_bytes / (dense_ms * 1e-3) / (HBM_PEAK_GBS * 1e9)},
        "per_layer_routing": {"ms_per_step": per_layer_ms, "tokens_per_s": B / (per_layer_ms * 1e-3),
                              "route_call_ms": route_pl_ms,
                              "attn_call_ms": per_layer_ms - route_pl_ms},
        "shared_step_ms": shared_ms,
        "speedup_vs_dense": dense_ms / shared_ms,
        "speedup_vs_per_layer_routing": per_layer_ms / shared_ms,
        "note": "same-box baselines on the decode leg's caches; context, not the metric",
    }


def _settle(fn, min_ms=25.0):
    """Repeat fn until the GPU has run it for at least min_ms: the clocks
    are at their working level before timing starts (a few calls after the
    host-side input preparation measure several percent slow)."""
    import torch
    torch.cuda.synchronize()
    t0, n = time.perf_counter(), 0
    while True:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= min_ms:
                return


def _event_ms(fn, reps):
    import torch
    _settle(fn)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _mall_cold_ms(calls):
    """Time each call on its own with events, after writing a 512 MiB buffer
    (outside the timed region) so that nothing it reads is still resident
    in the 256 MB last-level cache.  Returns the mean per call in ms."""
    import torch
    scrub = torch.empty(1 << 28, dtype=torch.int16, device="cuda")
    evs = []
    for i, fn in enumerate(calls):
        scrub.fill_(i & 0x7FFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    del scrub
    return sum(a.elapsed_time(b) for a, b in evs) / len(evs)


def threshold_step(dev, reps, cpu_budget=0.0):
    """Half-space selection at 128K: 16 sequences, d_idx 128, per-sequence
    tau set so that 256 .. 8192 keys qualify (Louver summary, section on the
    half-space reduction), then attention over those lists in 16 layers."""
    import torch
    from long_context_sparse_routing_amd import binding as clsa
    from long_context_sparse_routing_amd import inputs as gen
    wl = gen.WORKLOADS["threshold_128k_b16"]
    # input preparation: tau from fp64 scores on the host
    K_cpu, q_cpu, tau = gen.gen_threshold_inputs(wl, lambda qq, KK: KK @ qq)
    K_idx, q_idx, tau_d = K_cpu.to(dev), q_cpu.to(dev), tau.to(dev)
    cap = 8192
    route = clsa.prepare_route_threshold(q_idx, K_idx, tau_d, cap)
    idx, counts = route()
    Kc, Vc = gen.gen_kv(wl, dev)
    q = gen.gen_attn_query(wl, q_idx, 0, dev)
    attn = clsa.prepare_sparse_attn(q, Kc, Vc, idx, counts)
    route_ms = _event_ms(route, reps)
    attn_ms = _event_ms(attn, reps)
    step_ms = _event_ms(lambda: (route(), attn()), reps)
    sel = int(counts.sum())
    scan = wl.B * wl.n_ctx * wl.d * 2
    gather = sel * wl.L * wl.Hkv * wl.D * 2 * 2
    step_bytes = scan + gather + 2 * q.numel() * 2
    cpu = None
    if cpu_budget > 0:
        from oracle import clsa_oracle as O
        order = [int(f"{b:04b}"[::-1], 2) for b in range(wl.B)]  # spread over the count range
        done, tt, used, seqs = oracle_decode_rate(
            wl, K_idx, Kc, Vc, q_idx, q, lambda b: wl.n_ctx,
            lambda b, sc_: O.threshold_select(sc_, float(tau[b])), cpu_budget, order=order)
        cpu = {"value": done / tt, "unit": "tokens/s", "cores": used, "kind": "oracle",
               "sample": (f"{done} sequence-steps over sequences {seqs} of {wl.name} (fp64 "
                          f"scores over {wl.n_ctx} keys, threshold selection, attention in "
                          f"{wl.L} layers x {wl.Hq} heads)")}
    del Kc, Vc, q, attn, route, K_idx
    torch.cuda.empty_cache()
    return {"workload": wl.name, "sequences": wl.B, "selected_total": sel, "cpu_baseline": cpu,
            "route_call_ms": route_ms, "attn_call_ms": attn_ms, "ms_per_step": step_ms,
            "tokens_per_s": wl.B / (step_ms * 1e-3),
            "route_roofline": {"bound": "hbm", "achieved": scan / (route_ms * 1e-3) / 1e9,
                               "unit": "GB/s", "frac": scan / (route_ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
                               "algorithmic_bytes_per_call": scan},
            "step_hbm_frac": step_bytes / (step_ms * 1e-3) / (HBM_PEAK_GBS * 1e9)}


def louver_leg(dev, reps):
    """Threshold selection through the Louver index (Louver summary, sections
    on the index and its query algorithms) against the exhaustive scan of
    clsa_route_threshold, on the threshold workload's shapes (16 x 128K
    keys, d_idx 128, 256 .. 8192 keys per row): once on its Gaussian keys and
    once on clustered keys (64 centers per sequence, sigma 0.05), where an
    index can prune.  Reports the build, each query's time, the share of
    keys scored exactly and the bytes each query reads."""
    import torch
    from long_context_sparse_routing_amd import binding as clsa
    from long_context_sparse_routing_amd import inputs as gen
    wl = gen.WORKLOADS["threshold_128k_b16"]
    cap, r = 8192, 64
    out = {"workload": wl.name, "sequences": wl.B, "n": wl.n_ctx, "d_idx": wl.d, "r": r}
    for name, clusters in (("gaussian_keys", 0), ("clustered_keys", 64)):
        K_cpu, q_cpu, tau = gen.gen_threshold_inputs(wl, lambda qq, KK: KK @ qq,
                                                     clusters=clusters)
        K, q, tau_d = K_cpu.to(dev), q_cpu.to(dev), tau.to(dev)
        ref = clsa.prepare_route_threshold(q, K, tau_d, cap)
        ref_idx, ref_cnt = [t.clone() for t in ref()]
        scan_bytes = wl.B * wl.n_ctx * wl.d * 2
        exh_ms = _event_ms(ref, reps)
        leg = {"exhaustive": {"ms_per_call": exh_ms, "bytes": scan_bytes,
                              "GBs": scan_bytes / (exh_ms * 1e-3) / 1e9}}
        for S, mode in ((1, 1), (4, 1), (4, 2)):
            ix = clsa.LouverIndex(wl.B, wl.d, wl.n_ctx, S=S, r=r, device=dev)
            ix.build(K, wl.n_ctx)  # first build: kernels load
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ix2 = clsa.LouverIndex(wl.B, wl.d, wl.n_ctx, S=S, r=r, device=dev)
            e0.record()
            ix2.build(K, wl.n_ctx)
            e1.record()
            torch.cuda.synchronize()
            build_ms = e0.elapsed_time(e1)
            chk = torch.zeros(wl.B, dtype=torch.int32, device=dev)
            qc = ix.prepare_query(q, K, tau_d, cap, mode=mode, checked=chk)
            idx, cnt, _ = qc()
            torch.cuda.synchronize()
            same = torch.equal(idx, ref_idx) and torch.equal(cnt, ref_cnt)
            if not same:
                raise RuntimeError(f"Louver query (S={S}, mode={mode}) differs from the scan")
            ms = _event_ms(qc, reps)
            checked = int(chk.sum())
            C = 1 << max(0, math.ceil(math.log2(wl.n_ctx / r)))
            q_bytes = (wl.B * S * C * (wl.d // S * 2 + 4)  # centers and radii
                       + checked * (wl.d * 2 + 4)            # keys scored and their slots
                       + (wl.B * S * wl.n_ctx * 2 if S > 1 and mode == 1 else 0))  # cluster ids
            leg[f"S{S}_query{mode}"] = {
                "build_ms": build_ms, "ms_per_call": ms, "speedup_vs_exhaustive": exh_ms / ms,
                "keys_checked_frac": checked / (wl.B * wl.n_ctx), "bytes": q_bytes,
                "bytes_vs_scan": q_bytes / scan_bytes, "GBs": q_bytes / (ms * 1e-3) / 1e9,
                "matches_exhaustive": same}
            del ix, ix2, qc
        out[name] = leg
        del K, ref
        torch.cuda.empty_cache()
    return out


def alt_routers_leg(dev, reps):
    """The two alternative ways to produce the shared list, on the headline
    decode shapes (8 sequences x 128K keys, d_idx 64, k 2048), against the
    shared routing call:
      centroid table (CSAttention summary): k-means of 4096 prompt routing
        queries per sequence into 64 centroids, each with its top-2048 keys
        (built once, at prefill); a decode query scores its 3 best
        centroids' rows (6144 keys) instead of all 128K;
      cross-layer aggregation (CLAA abstract): the top-k of 16 layers' index
        head scores summed, i.e. 16 index heads scanned per token.
    Reports times, bytes read, and the overlap of each list with the exact
    shared top-k (a diagnostic of what the cheaper lookup gives up)."""
    import torch
    from long_context_sparse_routing_amd import binding as clsa
    from long_context_sparse_routing_amd import inputs as gen
    wl = gen.WORKLOADS["decode_128k_b8"]
    n = wl.n_ctx
    K_idx, u, _ = gen.gen_routing_keys(wl, dev)
    nc = torch.full((wl.B,), n, dtype=torch.int32, device=dev)
    q_idx = gen.gen_routing_query(wl, u, 0, dev)
    shared = clsa.prepare_route(q_idx, K_idx, wl.k, n_ctx=nc)
    ex_idx = shared()[0].clone()
    shared_ms = _event_ms(shared, reps)
    qp = gen.gen_prompt_routing_queries(wl, u, 4096, dev)
    C, T, P, rounds = 64, 2048, 3, 8
    clsa.csa_build(qp, K_idx, C, T, rounds=rounds, n_ctx=nc)  # kernels load
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    cent, table = clsa.csa_build(qp, K_idx, C, T, rounds=rounds, n_ctx=nc)
    e1.record()
    torch.cuda.synchronize()
    build_ms = e0.elapsed_time(e1)
    look = clsa.prepare_csa_route(q_idx, K_idx, cent, table, n, P, wl.k, n_ctx=nc)
    c_idx = look()[0]
    csa_ms = _event_ms(look, reps)
    overlap = lambda a: [len(set(a[b, 0].tolist()) & set(ex_idx[b, 0].tolist())) / wl.k  # noqa: E731
                         for b in range(wl.B)]
    csa_bytes = wl.B * (C * wl.d * 2 + P * T * (4 + wl.d * 2))
    out = {"workload": wl.name, "shared_route_ms": shared_ms,
           "centroid_table": {"C": C, "T": T, "P": P, "kmeans_rounds": rounds,
                              "prompt_queries": 4096, "build_ms": build_ms, "route_ms": csa_ms,
                              "speedup_vs_shared": shared_ms / csa_ms, "bytes": csa_bytes,
                              "recall_of_exact_topk": overlap(c_idx.cpu())}}
    del cent, table, look, qp
    # cross-layer aggregation: one index head per layer
    H = wl.L
    wl_h = wl.with_(name=wl.name + "_layer_heads", B=H * wl.B, base_seed=wl.base_seed + 100)
    Kh, uh, _ = gen.gen_routing_keys(wl_h, dev)
    qh = gen.gen_routing_query(wl_h, uh, 0, dev)
    Kh = Kh.view(H, wl.B, wl.n_cap, wl.d)
    qh = qh.view(H, wl.B, 1, wl.d)
    agg = clsa.prepare_route_aggregated(qh, Kh, wl.k, n_ctx=nc)
    agg()
    agg_ms = _event_ms(agg, max(1, reps // 2))
    per = [clsa.prepare_route(qh[h], Kh[h], wl.k, n_ctx=nc) for h in range(H)]
    per_ms = _event_ms(lambda: [c() for c in per], max(1, reps // 2))
    agg_bytes = H * wl.B * n * wl.d * 2
    out["cross_layer_aggregation"] = {
        "heads": H, "route_ms": agg_ms, "bytes": agg_bytes,
        "GBs": agg_bytes / (agg_ms * 1e-3) / 1e9, "per_layer_routing_ms": per_ms,
        "vs_shared": agg_ms / shared_ms,
        "note": "one shared list from 16 heads' summed scores; per-layer routing makes 16 lists"}
    del Kh, qh, agg, per, K_idx
    torch.cuda.empty_cache()
    return out


def tiny_fp32_step(dev, reps, cpu_budget=0.0):
    """The smallest configuration: one fp32 sequence at 4K context, d_idx 32,
    one layer with one head of dim 64, k = 256 -- a routing call plus an
    attention call, bound by launch latency rather than bytes."""
    import torch
    from long_context_sparse_routing_amd import binding as clsa
    from long_context_sparse_routing_amd import inputs as gen
    wl = gen.WORKLOADS["tiny_fp32_4k"]
    K_idx, u, _ = gen.gen_routing_keys(wl, dev)
    Kc, Vc = gen.gen_kv(wl, dev)
    q_idx = gen.gen_routing_query(wl, u, 0, dev)
    q = gen.gen_attn_query(wl, q_idx, 0, dev)
    route = clsa.prepare_route(q_idx, K_idx, wl.k)
    idx, counts = route()
    attn = clsa.prepare_sparse_attn(q, Kc, Vc, idx, counts)
    ms = _event_ms(lambda: (route(), attn()), reps)
    cpu = None
    if cpu_budget > 0:
        from oracle import clsa_oracle as O
        cpu = {}
        for name, threads in (("all_cores", None), ("single_thread", 1)):
            done, tt, used, _ = oracle_decode_rate(
                wl, K_idx, Kc, Vc, q_idx, q, lambda b: wl.n_ctx,
                lambda b, sc_: O.topk_select(sc_, wl.k), cpu_budget, threads=threads)
            cpu[name] = {"value": done / tt, "unit": "tokens/s", "cores": used, "kind": "oracle",
                         "sample": f"{done} decode steps at n = {wl.n_ctx}"}
    return {"workload": wl.name, "ms_per_step": ms, "tokens_per_s": 1.0 / (ms * 1e-3),
            "what": "routing call + attention call, back to back", "cpu_baseline": cpu}


def decode_32k_step(dev, steps, cpu_budget=0.0):
    """One sequence at 32K context: append + route + attention in 16 layers,
    the single-sequence case where attention lists are split across
    workgroups and merged."""
    import torch
    from long_context_sparse_routing_amd import binding as clsa
    from long_context_sparse_routing_amd import inputs as gen
    base = gen.WORKLOADS["decode_32k"]
    wl = base.with_(n_cap=base.n_ctx + steps + 2)
    N0 = wl.n_ctx
    K_idx, u, _ = gen.gen_routing_keys(wl, dev)
    Kc, Vc = gen.gen_kv(wl, dev)
    T = steps + 2
    new_kidx, new_k, new_v = gen.gen_append_rows(wl, T, dev)
    qi = [gen.gen_routing_query(wl, u, t, dev) for t in range(T)]
    qa = [gen.gen_attn_query(wl, qi[t], t, dev) for t in range(T)]
    nctx = torch.tensor([[N0 + t + 1] for t in range(T)], dtype=torch.int32, device=dev)
    idx = torch.empty((1, 1, wl.k), dtype=torch.int32, device=dev)
    counts = torch.empty((1, 1), dtype=torch.int32, device=dev)
    out = torch.empty((wl.L, 1, 1, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
    calls = [(clsa.prepare_kv_append(nctx[t] - 1, new_kidx[t], K_idx, new_k[t], Kc, new_v[t], Vc),
              clsa.prepare_route(qi[t], K_idx, wl.k, n_ctx=nctx[t], idx=idx, counts=counts),
              clsa.prepare_sparse_attn(qa[t], Kc, Vc, idx, counts, out=out)) for t in range(T)]
    for t in range(2):
        for c in calls[t]:
            c()
    _settle(lambda: [c() for c in calls[1]])  # step 1 again: its append rewrites one row
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(2, T):
        for c in calls[t]:
            c()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # the 32K working set (~139 MB) fits the last-level cache: the same
    # steps again, each timed alone after evicting it
    cold_ms = _mall_cold_ms([lambda c=c: [f() for f in c] for c in calls[2:]])
    n_mid = N0 + 2 + steps // 2
    step_bytes = (n_mid * wl.d * 2 + wl.L * wl.k * wl.Hkv * wl.D * 2 * 2
                  + 2 * wl.L * wl.Hq * wl.D * 2)
    cpu = None
    if cpu_budget > 0:
        from oracle import clsa_oracle as O
        t, cpu = T - 1, {}
        for name, threads in (("all_cores", None), ("single_thread", 1)):
            done, tt, used, _ = oracle_decode_rate(
                wl, K_idx, Kc, Vc, qi[t], qa[t], lambda b: N0 + t + 1,
                lambda b, sc_: O.topk_select(sc_, wl.k), cpu_budget, threads=threads)
            cpu[name] = {"value": done / tt, "unit": "tokens/s", "cores": used, "kind": "oracle",
                         "sample": f"{done} decode steps at n = {N0 + t + 1}"}
    del Kc, Vc, K_idx, calls
    torch.cuda.empty_cache()
    return {"workload": wl.name, "steps": steps, "ms_per_step": ms,
            "tokens_per_s": 1.0 / (ms * 1e-3), "bytes_per_step": step_bytes, "cpu_baseline": cpu,
            "step_hbm_frac": step_bytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
            "mall_cold": {"ms_per_step": cold_ms,
                          "step_hbm_frac": step_bytes / (cold_ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
                          "how": "each step timed alone after a 512 MiB write"}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="decode_128k_b8")
    ap.add_argument("--settle-ms", type=float, default=400.0,
                    help="untimed GPU run of routing + attention before the warm-up steps")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of CPU oracle work in the baseline sample (0 = skip)")
    ap.add_argument("--baseline-steps", type=int, default=5,
                    help="timed steps of the dense and per-layer-routing baselines (0: skip)")
    ap.add_argument("--other-configs", type=int, default=1,
                    help="also time the threshold (16 x 128K) and 32K decode configurations")
    ap.add_argument("--prefill-calls", type=int, default=10,
                    help="timed calls of the prefill-chunk routing leg (0: skip)")
    ap.add_argument("--prefill-attention", type=int, default=1,
                    help="also time the prefill chunk's sparse attention (0: skip)")
    ap.add_argument("--repeats", type=int, default=5,
                    help="runs of --steps fresh decode steps in 'repeats' (value is the first)")
    ap.add_argument("--per-layer-steps", type=int, default=16,
                    help="decode steps timed again with one attention call per layer (0: skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (scale for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported "
              "(decode sequences would shard across GPUs with no exchange, each GPU "
              "running this path on its share)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_sparse_routing_amd import binding as clsa
    from long_context_sparse_routing_amd import inputs as gen

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": src.numel() * 2,
                          "copy_calibration_bytes_written": dst.numel() * 2, "launches": 5}))
        return
    clsa.load_library()
    base = gen.WORKLOADS[args.workload]
    # warmup, the timed run, then args.repeats - 1 more runs of fresh steps
    # (the decode simply continues), each args.steps long
    n_runs = max(1, args.repeats)
    total_steps = args.warmup + args.steps * n_runs
    wl = base.with_(n_cap=base.n_ctx + total_steps)
    N0 = wl.n_ctx

    # ---- inputs, resident in HBM before timing ----
    K_idx, u, _ = gen.gen_routing_keys(wl, dev)
    Kc, Vc = gen.gen_kv(wl, dev)
    new_kidx, new_k, new_v = gen.gen_append_rows(wl, total_steps, dev)
    q_idx_all, q_all = [], []
    for t in range(total_steps):
        qi = gen.gen_routing_query(wl, u, t, dev)
        q_idx_all.append(qi)
        q_all.append(gen.gen_attn_query(wl, qi, t, dev))
    n_ctx_all = torch.tensor([[N0 + t + 1] * wl.B for t in range(total_steps)],
                             dtype=torch.int32, device=dev)
    pos_all = n_ctx_all - 1  # slot each step appends into
    idx = torch.empty((wl.B, 1, wl.k), dtype=torch.int32, device=dev)
    counts = torch.empty((wl.B, 1), dtype=torch.int32, device=dev)
    out = torch.empty((wl.L, wl.B, 1, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
    ws_r = torch.empty(clsa.route_workspace_size(wl.B, 1, wl.d, wl.n_cap, wl.k, wl.k,
                                                 torch.bfloat16), dtype=torch.uint8, device=dev)
    ws_a = torch.empty(max(1, clsa.sparse_attn_workspace_size(wl.L, wl.B, 1, wl.Hq, wl.Hkv, wl.D,
                                                              wl.k, torch.bfloat16)),
                       dtype=torch.uint8, device=dev)
    # every call of every step marshalled up front: the loop only launches
    appends = [clsa.prepare_kv_append(pos_all[t], new_kidx[t], K_idx, new_k[t], Kc, new_v[t], Vc)
               for t in range(total_steps)]
    routes = [clsa.prepare_route(q_idx_all[t], K_idx, wl.k, n_ctx=n_ctx_all[t], idx=idx,
                                 counts=counts, ws=ws_r) for t in range(total_steps)]
    attns = [clsa.prepare_sparse_attn(q_all[t], Kc, Vc, idx, counts, out=out, ws=ws_a)
             for t in range(total_steps)]
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev_attn = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(total_steps)]

    # HIP events bracket the attention call on every 8th step of the timed
    # run: each recorded pair adds a few microseconds to its step
    ev_every = 8

    def step(t, timed):
        mark = timed and (t - args.warmup) % ev_every == 0
        appends[t]()                 # append (the self-decoder's KV write)
        routes[t]()                  # one routing step shared by all layers
        if mark:
            ev_attn[t][0].record(stream)
        attns[t]()                   # sparse attention in all layers
        if mark:
            ev_attn[t][1].record(stream)

    # Clock settle, outside any timed region and before the warm-up steps:
    # routing and attention over the context as generated (no append, so the
    # caches and context lengths the warm-up steps find are unchanged; idx,
    # counts and out are rewritten by every later step), repeated until the
    # GPU has run them for --settle-ms.  A few warm-up steps alone leave the
    # clocks below their working level for the first timed steps.
    if args.settle_ms > 0:
        n0 = torch.full((wl.B,), N0, dtype=torch.int32, device=dev)
        r0 = clsa.prepare_route(q_idx_all[0], K_idx, wl.k, n_ctx=n0, idx=idx, counts=counts,
                                ws=ws_r)
        _settle(lambda: (r0(), attns[0]()), args.settle_ms)
    for t in range(args.warmup):
        step(t, False)
    torch.cuda.synchronize()
    t_end = args.warmup + args.steps  # the timed run: `value`
    t0 = time.perf_counter()
    for t in range(args.warmup, t_end):
        step(t, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert int(counts.min()) == wl.k and int(counts.max()) == wl.k
    # further runs over the next steps, no events: the spread of the rate
    walls = [wall]
    for r in range(1, n_runs):
        t1 = time.perf_counter()
        for t in range(t_end + (r - 1) * args.steps, t_end + r * args.steps):
            step(t, False)
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t1)
    marked = [ev_attn[t] for t in range(args.warmup, t_end)
              if (t - args.warmup) % ev_every == 0]
    attn_ms = sum(a.elapsed_time(b) for a, b in marked) / len(marked)

    # routing call duration, from a separate pass over the last steps' inputs
    # (kept out of the timed loop so its events do not add gaps there); one
    # untimed pass first, since the first launch after the GPU idles starts
    # some XCDs' workgroups microseconds late
    n_rt, n_pass = min(8, args.steps), 3
    for i in range(n_rt):
        routes[t_end - n_rt + i]()
    ev_r = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    ev_r[0].record(stream)
    for _ in range(n_pass):
        for i in range(n_rt):
            routes[t_end - n_rt + i]()
    ev_r[1].record(stream)
    torch.cuda.synchronize()
    route_ms = ev_r[0].elapsed_time(ev_r[1]) / (n_rt * n_pass)

    ms_step = wall * 1e3 / args.steps
    tokens = wl.B * args.steps
    n_mid = N0 + args.warmup + args.steps // 2 + 1
    a_bytes = attn_bytes(wl.L, wl.B, 1, wl.Hq, wl.Hkv, wl.D, wl.k)
    r_bytes = route_bytes(wl.B, 1, n_mid, wl.d, wl.k)
    app_bytes = wl.B * (wl.d * 2 + wl.L * 2 * wl.Hkv * wl.D * 2) * 2  # read staged + write
    step_bytes = a_bytes + r_bytes + app_bytes
    achieved = a_bytes / (attn_ms * 1e-3) / 1e9

    res = {
        "metric": "decode tokens/s at 128K ctx, k=2048, 16 shared-routing layers; % HBM peak",
        "value": tokens / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "n_ctx": N0, "k": wl.k,
                   "layers": wl.L, "d_idx": wl.d, "Hq": wl.Hq, "Hkv": wl.Hkv,
                   "head_dim": wl.D, "append_per_step": 1},
        "step_hbm_frac": step_bytes / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "repeats": {"runs": len(walls),
                    "tokens_per_s_median": tokens / sorted(walls)[len(walls) // 2],
                    "tokens_per_s_min": tokens / max(walls),
                    "tokens_per_s_max": tokens / min(walls),
                    "tokens_per_s_runs": [tokens / w for w in walls],
                    "how": (f"{n_runs} runs of {args.steps} consecutive decode steps (the "
                            "decode continues from run to run); value is the first run")},
        "step_breakdown_ms": {"route_call": route_ms, "attn_call": attn_ms,
                              "append_and_gaps": ms_step - route_ms - attn_ms,
                              "route_call_source": ("separate pass after the timed loop: "
                                                    "the run's last 8 routing calls, back to back, "
                                                    "3 times after one untimed pass"),
                              "attn_call_source": f"HIP events on every {ev_every}th timed step",
                              "note": ("the parts come from separate instruments; an event pair "
                                       "keeps the attention dispatch from overlapping the "
                                       "routing call's tail, so the parts can sum above the "
                                       "step")},
        "roofline": {"kernel": "attn_bf16<4,128,streaming> (one clsa_sparse_attn launch, 16 layers)",
                     "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": profiled_traffic(),
                     "algorithmic_bytes_per_launch": a_bytes},
        "route_roofline": {"achieved": r_bytes / (route_ms * 1e-3) / 1e9, "unit": "GB/s",
                           "frac": r_bytes / (route_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           "algorithmic_bytes_per_call": r_bytes},
    }
    if args.per_layer_steps > 0:
        res["per_layer_launches"] = per_layer_launches(
            wl, clsa, K_idx, Kc, Vc, q_idx_all, q_all, n_ctx_all, pos_all,
            (new_kidx, new_k, new_v), min(args.per_layer_steps, total_steps), dev)
    if args.baseline_steps > 0:
        res["baselines"] = baselines(wl, Kc, Vc, q_all[total_steps - 1], N0 + total_steps, dev,
                                     args.baseline_steps, ms_step)
    if args.cpu_budget > 0:
        t = total_steps - 1
        res["cpu_baseline"] = cpu_baseline(wl, K_idx, Kc, Vc, q_idx_all[t], q_all[t],
                                           N0 + t + 1, args.cpu_budget)
    # the decode caches are released before the other configurations
    del Kc, Vc, appends, routes, attns, q_all, q_idx_all, new_kidx, new_k, new_v, K_idx
    torch.cuda.empty_cache()
    if args.other_configs:
        cb = min(3.0, args.cpu_budget)
        res["threshold_128k_b16"] = threshold_step(dev, 5, cb)
        res["decode_32k"] = decode_32k_step(dev, 64, cb)
        res["tiny_fp32_4k"] = tiny_fp32_step(dev, 200, min(1.0, cb))
        res["louver"] = louver_leg(dev, 5)
        res["alt_routers"] = alt_routers_leg(dev, 10)
    if args.prefill_calls > 0:
        res["prefill_routing"] = prefill_routing(args.prefill_calls, dev, min(5.0, args.cpu_budget),
                                                 bool(args.prefill_attention))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
