#!/usr/bin/env python3
"""Benchmark: split-KV paged decode attention on one MI355X.

One step = the whole decode hot path for one batch: steady bind (seq_lens and
position_ids +1, kv_indptr scan, kv_indices fill) followed by 24 layers of
(split-KV attention, log-sum-exp merge), captured once into a hipGraph and
replayed.  Workload: 24 layers in [24, slots, 8, 128] bf16 stores, B=32,
seq_lens ~ U[1, 2048] (+1 per step), 32 query heads, page size 16.

Prints ONE JSON line on stdout.  ``value`` is KV bytes read per second (K and
V rows actually attended, summed over layers and steps) over the timed graph
replays.  ``roofline`` is for the dominant kernel (the split attention),
timed live with HIP events on its stream over a replayed graph of the 24
attention launches.  ``batch_sweep`` times one layer (attention and merge,
caches flushed) at B = 1, 2, 4, 8, 16, 32 requests of 4096 tokens.
``cpu_baseline`` times the CPU oracle on a bounded sample of the same
workload.  Diagnostics go to stderr.

    python bench.py [--gpus 1] [--steps 100] [--warmup 10] [--no-cpu-baseline] [--sweep 1,2,4,8,16,32]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attn: KV HBM GB/s (% of peak) and µs/layer at B=1..32"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic.json")
ATTN_SOURCES = ("paged_kv_decode_10_amd/csrc/attn_split.hip", "paged_kv_decode_10_amd/csrc/pd_internal.h",
                "paged_kv_decode_10_amd/csrc/paged_decode.cpp")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attn_kernel_digest() -> str:
    """Digest of the attention sources' code: comments and whitespace are
    dropped, so only a change to the code itself invalidates the committed
    counter figures."""
    import re

    h = hashlib.sha256()
    for rel in ATTN_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def plan_args(n_kv_heads):
    """The launch's split-plan parameters: bundle size T = gcd(n_kv_heads,
    PD_PLAN_TEAM_MAX) and chunk count C = PD_PLAN_WAVES / T."""
    import math

    from paged_kv_decode_10_amd._abi import PD_PLAN_TEAM_MAX, PD_PLAN_WAVES

    team = math.gcd(int(n_kv_heads), PD_PLAN_TEAM_MAX)
    return {"n_chunks": PD_PLAN_WAVES // team, "team": team}


def row_splits(seq_lens, page_size, n_kv_heads, num_splits):
    """Splits of every (request, kv head) row under the launch's plan.  Kv
    heads form bundles of T heads; a bundle row of P pages starting at global
    page G meets the chunks floor(G/Qp) .. floor((G+P-1)/Qp) of the C chunks
    (one split per non-empty row when S = 1)."""
    import numpy as np

    pa = plan_args(n_kv_heads)
    team, nch = pa["team"], pa["n_chunks"]
    hs = n_kv_heads // team
    P = (np.asarray(seq_lens, dtype=np.int64) + page_size - 1) // page_size
    Pr = np.repeat(P[:, None], hs, axis=1)
    if num_splits == 1:
        n = (Pr > 0).astype(np.int64)
    else:
        tp = int(P.sum()) * hs
        qp = max(-(-tp // nch), -(-int(P.max()) // (num_splits - 1)), 1)
        G = np.concatenate([[0], np.cumsum(P)[:-1]])[:, None] * hs + np.arange(hs)[None, :] * P[:, None]
        n = np.where(Pr > 0, (G + Pr - 1) // qp - G // qp + 1, 0)
    return np.repeat(n, team, axis=1)


def split_segments(seq_lens, page_size, n_kv_heads, num_splits):
    """Number of non-empty (request, kv head, split) partials the plan writes."""
    return int(row_splits(seq_lens, page_size, n_kv_heads, num_splits).sum())


def attn_bytes(seq_lens, n_kv_heads, head_dim, batch, n_heads, num_splits, page_size):
    """Algorithmic bytes of one attention launch: the K and V rows of every
    cached token, the kv_indices list, q, and the partials of the non-empty
    splits (o row fp32 + (m, ln l) per query head)."""
    tok = int(seq_lens.sum())
    kv = tok * n_kv_heads * head_dim * 2 * 2
    idx = tok * 4
    q = batch * n_heads * head_dim * 2
    group = n_heads // n_kv_heads
    parts = split_segments(seq_lens, page_size, n_kv_heads, num_splits) * group * (head_dim * 4 + 8)
    return kv, kv + idx + q + parts


def cpu_baseline(w, budget_s: float, num_splits: int):
    """Time the oracle on the same step, layer after layer, until ~budget_s.

    Per layer it computes what the GPU path produces, the way the GPU path
    does: the bind (kv_indptr, kv_indices), the per-split partials (one pass
    over the layer's K and V) and their log-sum-exp merge into the output.
    """
    import numpy as np
    import torch

    import oracle

    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        blas = 1
    L = w.seq_lens.numpy()
    layers, kv = 0, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        layer = layers % w.n_layers
        ip, ix = oracle.bind_full(L, w.req_to_page.numpy(), w.page_size)
        o, _, lse = oracle.split_partials(w.q[layer], w.k_store[layer], w.v_store[layer], L, ip, ix, w.scale,
                                          w.n_kv_heads, w.page_size, num_splits, **plan_args(w.n_kv_heads))
        oracle.merge_splits(o, lse)
        layers += 1
        kv += int(L.sum()) * w.n_kv_heads * w.head_dim * 2 * 2
    dt = time.perf_counter() - t0
    cores = max(torch.get_num_threads(), blas)
    return {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"float64 numpy oracle on the same decode step: {layers} layer passes (bind, "
                      f"per-split partials with S={num_splits}, log-sum-exp merge; all 32 requests x 8 kv "
                      f"heads; K and V read once per pass), {kv / 1e6:.0f} MB of KV in {dt:.1f} s; host affinity "
                      f"{len(os.sched_getaffinity(0))} cpus, torch threads {torch.get_num_threads()}, "
                      f"BLAS threads {blas}; numpy {np.__version__}"}


def config_sweep(names, reps: int, oracle_budget: float, splits: int = 0, in_step: bool = False):
    """Per-config attention and merge timings with the caches flushed.

    For each workload: one bind, then ``reps`` iterations of [1 GiB
    flush-write, attn, merge] with HIP events around the attention and the
    merge separately (on the launch stream).  Reports median / p10 / p90 and
    the KV-only and all-algorithmic rates at the median.  With ``in_step``
    the workload has two layers and each iteration is [flush, attn + merge
    of layer 0 (untimed), attn + merge of layer 1 (timed)]: the timed layer
    reads KV that no launch has touched since the flush, with the step's
    index lists already read once, as every layer after the first of a
    decode step does.  With ``oracle_budget`` > 0 the oracle is timed on the
    same inputs, one (request, kv head) pair at a time, for at most about
    that many seconds per config.
    """
    import numpy as np
    import torch

    import workloads
    from paged_kv_decode_10_amd import PD_BIND_FULL, Config, PagedDecode

    flush = torch.empty(1 << 28, dtype=torch.int32, device="cuda")
    rows = []
    for name in names:
        t0 = time.perf_counter()
        base_name, _, layout = name.partition("@")  # "b16@contiguous": the contiguous-cache layout
        w = workloads.make(base_name, layout=layout or "paged", **({"n_layers": 2} if in_step else {}))
        B, H, Hkv, D = w.batch, w.n_heads, w.n_kv_heads, w.head_dim
        cfg = Config(n_layers=w.n_layers, n_heads=H, n_kv_heads=Hkv, head_dim=D, page_size=w.page_size,
                     max_batch=B, max_splits=256, max_pages_per_req=w.max_pages_per_req, num_slots=w.num_slots,
                     max_total_tokens=int(w.seq_lens.sum()))
        ws = PagedDecode(cfg)
        seq, pos, tab = w.seq_lens.cuda(), w.position_ids.cuda(), w.req_to_page.cuda()
        q, kst, vst = w.q.cuda(), w.k_store.cuda(), w.v_store.cuda()
        out = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
        S = ws.num_splits(B, splits)
        if layout == "contiguous":
            ws.bind_contiguous(B, PD_BIND_FULL, seq, pos, w.meta["req_base"].cuda())
        else:
            ws.bind(B, PD_BIND_FULL, seq, pos, tab)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ta, tm = [], []
        lt = 1 if in_step else 0  # the timed layer
        for r in range(reps + 2):
            flush.fill_(r)
            if in_step:
                ws.attn(B, 0, S, q[0], kst, vst, w.scale)
                ws.merge(B, S, out)
            ev[0].record()
            ws.attn(B, lt, S, q[lt], kst, vst, w.scale)
            ev[1].record()
            ws.merge(B, S, out)
            ev[2].record()
            torch.cuda.synchronize()
            if r >= 2:
                ta.append(ev[0].elapsed_time(ev[1]) * 1e3)
                tm.append(ev[1].elapsed_time(ev[2]) * 1e3)
        assert ws.read_error() == 0 and torch.isfinite(out.float()).all()
        L = w.seq_lens.to(torch.int64)
        kv, alg = attn_bytes(L, Hkv, D, B, H, S, w.page_size)
        pa = np.percentile(ta, [50, 10, 90])
        pm = np.percentile(tm, [50, 10, 90])
        row = {"workload": name, "timing": "in-step (second layer after a flush)" if in_step else "cold (after a flush)",
               "batch": B, "n_heads": H, "n_kv_heads": Hkv, "head_dim": D,
               "sum_seq_len": int(L.sum()), "num_splits": S,
               "attn_us": {"median": round(pa[0], 2), "p10": round(pa[1], 2), "p90": round(pa[2], 2)},
               "merge_us": {"median": round(pm[0], 2), "p10": round(pm[1], 2), "p90": round(pm[2], 2)},
               "kv_bytes": kv, "algorithmic_bytes": alg,
               "kv_gbs": round(kv / pa[0] / 1e3, 1), "kv_pct_of_peak": round(100 * kv / pa[0] / 1e3 / HBM_PEAK_GBS, 1),
               "alg_gbs": round(alg / pa[0] / 1e3, 1),
               "kv_gbs_attn_plus_merge": round(kv / (pa[0] + pm[0]) / 1e3, 1),
               "us_per_layer_attn_plus_merge": round(pa[0] + pm[0], 2)}
        if oracle_budget > 0:
            row["oracle"] = oracle_time(w, oracle_budget)
        rows.append(row)
        log(f"[configs] {name}: B={B} sum(L)={int(L.sum())} S={S} attn {pa[0]:.2f} us (p10 {pa[1]:.2f}, "
            f"p90 {pa[2]:.2f}) -> {row['kv_gbs']:.0f} GB/s KV ({row['kv_pct_of_peak']}%), merge {pm[0]:.2f} us; "
            f"{time.perf_counter() - t0:.1f} s")
        del ws, q, kst, vst
        torch.cuda.empty_cache()
    return rows


def graph_sweep(names, reps: int, rounds: int, splits: int = 0):
    """Per-batch attention and merge time, each launch after a cache flush,
    measured the way a captured step runs them: three graphs of ``reps``
    repetitions each -- [flush], [flush, attn], [flush, attn, merge] (flush =
    a 1 GiB fill kernel, four times the 256 MB Infinity Cache) -- are replayed
    one after another ``rounds`` times with HIP events around each replay;
    per round attn = (T[flush, attn] - T[flush]) / reps and merge =
    (T[flush, attn, merge] - T[flush, attn]) / reps, medians over the rounds.
    Each kernel's time includes the boundary before it, as in the step's
    kernel trace; no per-launch event sits between the kernels."""
    import numpy as np
    import torch

    import workloads
    from paged_kv_decode_10_amd import PD_BIND_FULL, Config, PagedDecode

    flush = torch.empty(1 << 28, dtype=torch.int32, device="cuda")
    rows = []
    for name in names:
        w = workloads.make(name)
        B, H, Hkv, D = w.batch, w.n_heads, w.n_kv_heads, w.head_dim
        cfg = Config(n_layers=1, n_heads=H, n_kv_heads=Hkv, head_dim=D, page_size=w.page_size, max_batch=B,
                     max_splits=256, max_pages_per_req=w.max_pages_per_req, num_slots=w.num_slots,
                     max_total_tokens=int(w.seq_lens.sum()))
        ws = PagedDecode(cfg)
        seq, pos, tab = w.seq_lens.cuda(), w.position_ids.cuda(), w.req_to_page.cuda()
        q, kst, vst = w.q.cuda(), w.k_store.cuda(), w.v_store.cuda()
        out = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
        S = ws.num_splits(B, splits)
        ws.bind(B, PD_BIND_FULL, seq, pos, tab)
        torch.cuda.synchronize()

        def capture(parts):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for r in range(reps):
                    flush.fill_(r + 1)
                    if "attn" in parts:
                        ws.attn(B, 0, S, q[0], kst, vst, w.scale)
                    if "merge" in parts:
                        ws.merge(B, S, out)
            return g

        graphs = [capture(()), capture(("attn",)), capture(("attn", "merge"))]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = [[], [], []]
        for rnd in range(rounds + 1):
            for i, g in enumerate(graphs):
                e0.record()
                g.replay()
                e1.record()
                torch.cuda.synchronize()
                if rnd:  # the first round warms up
                    times[i].append(e0.elapsed_time(e1) * 1e3 / reps)
        assert ws.read_error() == 0 and torch.isfinite(out.float()).all()
        tf = float(np.median(times[0]))
        attn_us = float(np.median([b - a for a, b in zip(times[0], times[1])]))
        merge_us = float(np.median([c - b for b, c in zip(times[1], times[2])]))
        L = w.seq_lens.to(torch.int64)
        kv, alg = attn_bytes(L, Hkv, D, B, H, S, w.page_size)
        rows.append({"batch": B, "num_splits": S, "attn_us": round(attn_us, 2), "merge_us": round(merge_us, 2),
                     "us_per_layer": round(attn_us + merge_us, 2), "kv_bytes": kv,
                     "kv_gbs_attn": round(kv / attn_us / 1e3, 1),
                     "kv_pct_of_peak_attn": round(100 * kv / attn_us / 1e3 / HBM_PEAK_GBS, 1),
                     "kv_gbs_layer": round(kv / (attn_us + merge_us) / 1e3, 1)})
        log(f"[sweep] {name}: B={B} S={S} attn {attn_us:.2f} us -> {kv / attn_us / 1e3:.0f} GB/s KV "
            f"({100 * kv / attn_us / 1e3 / HBM_PEAK_GBS:.1f}%), merge {merge_us:.2f} us (flush {tf:.1f} us)")
        del graphs, ws, q, kst, vst
        torch.cuda.empty_cache()
    return rows


def pool_sweep(batches, steps: int, warmup: int):
    """Graph pool on the 24-layer step workload: per batch size, the step time
    replaying the pool's captured graph vs the same pool run eagerly (every
    kernel launched from the host), both HIP-event timed over `steps` steps."""
    import torch

    import workloads
    from paged_kv_decode_10_amd import PD_BIND_FULL, Config, GraphPool, PagedDecode

    growth = 2 * (steps + warmup) * len(batches) + 8
    w = workloads.make("step", growth=growth)
    B, H, Hkv, D, NL = w.batch, w.n_heads, w.n_kv_heads, w.head_dim, w.n_layers
    cfg = Config(n_layers=NL, n_heads=H, n_kv_heads=Hkv, head_dim=D, page_size=w.page_size, max_batch=B,
                 max_splits=256, max_pages_per_req=w.max_pages_per_req, num_slots=w.num_slots,
                 max_total_tokens=int(w.seq_lens.sum()) + growth * B)
    ws = PagedDecode(cfg)
    seq, pos, tab = w.seq_lens.cuda(), w.position_ids.cuda(), w.req_to_page.cuda()
    q, kst, vst = w.q.cuda(), w.k_store.cuda(), w.v_store.cuda()
    out = torch.empty((NL, B, H, D), dtype=torch.bfloat16, device="cuda")
    ws.bind(B, PD_BIND_FULL, seq, pos, tab)
    pools = {}
    for eager in (False, True):
        pools[eager] = GraphPool(ws, seq_lens=seq, position_ids=pos, q=q, k_store=kst, v_store=vst, out=out,
                                 scale=w.scale, req_to_page=tab, eager=eager)
        pools[eager].warmup()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rows = []
    for b in batches:
        res = {}
        for eager in (False, True):
            p = pools[eager]
            for _ in range(warmup):
                p.step(b)
            torch.cuda.synchronize()
            L0 = seq[:b].to(torch.int64).clone()
            e0.record()
            for _ in range(steps):
                p.step(b)
            e1.record()
            torch.cuda.synchronize()
            kv = sum(int((L0 + i + 1).sum()) for i in range(steps)) * Hkv * D * 4 * NL
            us = e0.elapsed_time(e1) * 1e3 / steps
            res[eager] = (us, kv / (us * 1e-6 * steps) / 1e9)
        rows.append({"batch": b, "graph_us_per_step": round(res[False][0], 1),
                     "eager_us_per_step": round(res[True][0], 1),
                     "speedup": round(res[True][0] / res[False][0], 3),
                     "graph_kv_gbs": round(res[False][1], 1)})
        log(f"[pool] B={b}: graph {res[False][0]:.1f} us/step ({res[False][1]:.0f} GB/s KV), "
            f"eager {res[True][0]:.1f} us/step -> x{res[True][0] / res[False][0]:.2f}")
    keys = pools[False].keys()
    for p in pools.values():
        p.close()
    return rows, keys


def prefill_bench(name: str, reps: int):
    """Prefill / extend attention on a prefill workload, one launch at a time
    with the caches flushed: HIP-event median, algorithmic flops (QK^T and PV
    over each query's causal range) and the K/V bytes the kernel streams
    (every work item of 128 query rows reads its causal range once)."""
    import numpy as np
    import torch

    import workloads
    from paged_kv_decode_10_amd import Config, PagedDecode

    w = workloads.make(name)
    B, H, Hkv, D = w.batch, w.n_heads, w.n_kv_heads, w.head_dim
    G = H // Hkv
    cfg = Config(n_layers=w.n_layers, n_heads=H, n_kv_heads=Hkv, head_dim=D, page_size=w.page_size, max_batch=B,
                 max_splits=8, max_pages_per_req=w.max_pages_per_req, num_slots=w.num_slots,
                 max_total_tokens=int(w.seq_lens.sum()))
    ws = PagedDecode(cfg)
    seq, tab = w.seq_lens.cuda(), w.req_to_page.cuda()
    ext = w.meta["extend_lens"].cuda()
    q, kst, vst = w.q.cuda(), w.k_store.cuda(), w.v_store.cuda()
    out = torch.empty_like(q[0])
    ws.bind_extend(B, seq, ext, req_to_page=tab)
    flush = torch.empty(1 << 28, dtype=torch.int32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for r in range(reps + 2):
        flush.fill_(r)
        e0.record()
        ws.prefill_attn(B, 0, q[0], kst, vst, w.scale, out)
        e1.record()
        torch.cuda.synchronize()
        if r >= 2:
            ts.append(e0.elapsed_time(e1) * 1e3)
    assert ws.read_error() == 0 and torch.isfinite(out.float()).all()
    L = w.seq_lens.numpy().astype(np.int64)
    n = w.meta["extend_lens"].numpy().astype(np.int64)
    keys = sum(int(((L[b] - n[b]) + np.arange(n[b]) + 1).sum()) for b in range(B))  # causal key count per query
    flops = 4 * D * H * keys  # 2 flops per MAC, QK^T and PV
    rows = 128  # query rows per work item of the library's prefill kernel (4 waves x 32)
    streamed = 0
    for b in range(B):
        for t in range(-(-int(n[b]) * G // rows)):
            last = min(int(n[b]) - 1, (rows * t + rows - 1) // G)
            streamed += (int(L[b] - n[b]) + last + 1) * D * 2 * 2 * Hkv
    kv_unique = int(L.sum()) * Hkv * D * 4
    us = float(np.median(ts))
    rec = {"workload": name, "batch": B, "new_tokens": int(n.sum()), "cached_tokens": int(L.sum()),
           "us": round(us, 2), "p10_us": round(float(np.percentile(ts, 10)), 2),
           "p90_us": round(float(np.percentile(ts, 90)), 2),
           "tflops": round(flops / us / 1e6, 1), "mfma_bf16_peak_tflops": 2500.0,
           "frac_of_mfma_peak": round(flops / us / 1e6 / 2500.0, 4),
           "kv_bytes_streamed": streamed, "kv_streamed_gbs": round(streamed / us / 1e3, 1),
           "kv_bytes_unique": kv_unique}
    log(f"[prefill] {name}: {us:.1f} us, {rec['tflops']} TFLOP/s ({100 * rec['frac_of_mfma_peak']:.1f}% of bf16 "
        f"MFMA), K/V streamed {streamed / 1e6:.0f} MB -> {rec['kv_streamed_gbs']} GB/s (unique {kv_unique / 1e6:.0f} MB)")
    return rec


def oracle_time(w, budget_s: float):
    """The oracle's decode attention on (request, kv head) pairs of the same
    inputs until about budget_s, scaled to KV bytes per second."""
    import oracle

    L = w.seq_lens.numpy()
    ip, ix = oracle.bind_full(L, w.req_to_page.numpy(), w.page_size)
    pairs = [(b, g) for b in range(w.batch) for g in range(w.n_kv_heads)]
    done, kv = 0, 0
    t0 = time.perf_counter()
    for pr in pairs:
        oracle.decode_attention(w.q[0], w.k_store[0], w.v_store[0], L, ip, ix, w.scale, w.n_kv_heads, pairs=[pr])
        done += 1
        kv += int(L[pr[0]]) * w.head_dim * 4
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"pairs": done, "of": len(pairs), "seconds": round(dt, 2), "kv_gbs": round(kv / dt / 1e9, 4)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--roofline-reps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--splits", type=int, default=0, help="0 = library heuristic")
    ap.add_argument("--append", choices=("none", "separate", "fused"), default="none",
                    help="also write each layer's new-token K/V into the cache: its own kernel, or inside the "
                         "attention launch")
    ap.add_argument("--configs", default="",
                    help="instead of the step: comma-separated workloads (e.g. tiny,b1,b16,long,sweep1,...,sweep32; "
                         "NAME@contiguous for the contiguous-cache layout) timed one launch at a time with the "
                         "caches flushed; prints one JSON line")
    ap.add_argument("--config-reps", type=int, default=20)
    ap.add_argument("--in-step", action="store_true",
                    help="--configs: time the second of two layers after each flush (index lists warm, KV cold)")
    ap.add_argument("--prefill", default="",
                    help="instead of the step: comma-separated prefill workloads (e.g. prefill) timed one launch at "
                         "a time with the caches flushed; prints one JSON line")
    ap.add_argument("--pool", default="",
                    help="instead of the step: comma-separated batch sizes run through the graph pool (replayed "
                         "and eager) on the 24-layer step workload; prints one JSON line")
    ap.add_argument("--oracle-budget", type=float, default=0.0,
                    help="with --configs: seconds of oracle timing per config (0 = none)")
    ap.add_argument("--sweep", default="1,2,4,8,16,32",
                    help="default mode: also time one layer at these batch sizes (4096 tokens each, caches "
                         "flushed) and report them in the JSON line; empty = skip")
    ap.add_argument("--calib-copy-gib", type=float, default=0.0,
                    help="also run a plain device copy of this many GiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the split-KV path has no multi-GPU mode; requests, "
              "kv heads or pages would shard with at most one all-gather of the split partials.",
              file=sys.stderr)
        return 2

    import torch

    import workloads
    from paged_kv_decode_10_amd import PD_BIND_FULL, PD_BIND_STEADY, Config, PagedDecode

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        return 2
    if args.prefill:
        rows = [prefill_bench(x, args.config_reps) for x in args.prefill.split(",") if x]
        print(json.dumps({"metric": "paged prefill attention", "unit": "TFLOP/s", "n_gpus": 1, "data": "synthetic",
                          "dtype": "bf16", "workloads": rows}), flush=True)
        return 0
    if args.pool:
        rows, keys = pool_sweep([int(x) for x in args.pool.split(",") if x], args.steps, args.warmup)
        print(json.dumps({"metric": "graph pool: decode step time, replay vs eager", "unit": "us/step",
                          "n_gpus": 1, "data": "synthetic", "dtype": "bf16", "keys": keys, "batches": rows}),
              flush=True)
        return 0
    if args.configs:
        rows = config_sweep([x for x in args.configs.split(",") if x], args.config_reps, args.oracle_budget,
                            args.splits, args.in_step)
        if args.calib_copy_gib > 0:  # a plain copy of known size, for counter calibration
            n = int(args.calib_copy_gib * (1 << 30))
            src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst
        print(json.dumps({"metric": METRIC, "unit": "GB/s", "n_gpus": 1, "data": "synthetic", "dtype": "bf16",
                          "timing": "HIP events per launch, 1 GiB flush-write before each iteration",
                          "configs": rows}), flush=True)
        return 0
    K, W = args.steps, args.warmup
    growth = max(256, K + W + 8)
    t0 = time.perf_counter()
    w = workloads.make("step", growth=growth)
    log(f"[bench] workload generated in {time.perf_counter() - t0:.1f}s: B={w.batch} layers={w.n_layers} "
        f"sum(L)={int(w.seq_lens.sum())} pages={w.num_pages}")
    B, H, Hkv, D, NL = w.batch, w.n_heads, w.n_kv_heads, w.head_dim, w.n_layers
    cfg = Config(n_layers=NL, n_heads=H, n_kv_heads=Hkv, head_dim=D, page_size=w.page_size, max_batch=B,
                 max_splits=64, max_pages_per_req=w.max_pages_per_req, num_slots=w.num_slots,
                 max_total_tokens=int(w.seq_lens.sum()) + growth * B)
    ws = PagedDecode(cfg)
    seq = w.seq_lens.cuda()
    pos = w.position_ids.cuda()
    table = w.req_to_page.cuda()
    q = w.q.cuda()
    kst = w.k_store.cuda()
    vst = w.v_store.cuda()
    out = torch.empty((NL, B, H, D), dtype=torch.bfloat16, device="cuda")
    S = ws.num_splits(B, args.splits)
    log(f"[bench] splits S={S}")

    if args.append != "none":
        gen = torch.Generator().manual_seed(123)
        k_new = torch.randn((NL, B, Hkv, D), generator=gen).to(torch.bfloat16).cuda()
        v_new = torch.randn((NL, B, Hkv, D), generator=gen).to(torch.bfloat16).cuda()

    def attention(layer):
        if args.append == "fused":
            ws.append_attn(B, layer, S, q[layer], k_new[layer], v_new[layer], kst, vst, w.scale)
        else:
            if args.append == "separate":
                ws.append_kv(B, layer, k_new[layer], v_new[layer], kst, vst)
            ws.attn(B, layer, S, q[layer], kst, vst, w.scale)

    def step():
        ws.bind(B, PD_BIND_STEADY, seq, pos, table)
        for layer in range(NL):
            attention(layer)
            ws.merge(B, S, out[layer])

    L0 = w.seq_lens.to(torch.int64)
    ws.bind(B, PD_BIND_FULL, seq, pos, table)
    step()  # live run before capture
    torch.cuda.synchronize()
    done = 1
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for _ in range(W):
        graph.replay()
    torch.cuda.synchronize()
    done += W
    assert ws.read_error() == 0, "device error word set"

    kv_bytes = 0
    for i in range(K):
        kv_bytes += int((L0 + done + i + 1).sum()) * Hkv * D * 4 * NL
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(K):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    done += K
    assert torch.equal(seq.cpu().to(torch.int64), L0 + done), "steady bind did not advance once per step"
    gbs = kv_bytes / (ms / 1e3) / 1e9
    ms_step = ms / K
    log(f"[bench] {K} steps in {ms:.2f} ms: {ms_step * 1e3:.1f} us/step, {ms_step * 1e3 / NL:.2f} us/layer, "
        f"{gbs:.0f} GB/s KV ({100 * gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s)")

    # Roofline of the dominant kernel: a graph of the 24 attention launches at
    # the current lengths, replayed; HIP events on the launch stream.
    ag = torch.cuda.CUDAGraph()
    with torch.cuda.graph(ag):
        for layer in range(NL):
            if args.append == "fused":
                ws.append_attn(B, layer, S, q[layer], k_new[layer], v_new[layer], kst, vst, w.scale)
            else:
                ws.attn(B, layer, S, q[layer], kst, vst, w.scale)
    for _ in range(3):
        ag.replay()
    torch.cuda.synchronize()
    R = args.roofline_reps
    e0.record()
    for _ in range(R):
        ag.replay()
    e1.record()
    torch.cuda.synchronize()
    attn_us = e0.elapsed_time(e1) * 1e3 / (R * NL)
    Lnow = seq.cpu().to(torch.int64)
    kv_l, alg_l = attn_bytes(Lnow, Hkv, D, B, H, S, w.page_size)
    if args.append == "fused":
        alg_l += 2 * 2 * B * Hkv * D * 2  # new K and V rows read and written
    achieved = alg_l / (attn_us * 1e-6) / 1e9
    log(f"[bench] attention kernel: {attn_us:.2f} us/launch, {alg_l / 1e6:.1f} MB algorithmic "
        f"({kv_l / 1e6:.1f} MB KV) -> {achieved:.0f} GB/s")
    # HBM traffic per launch from the committed counter summary, valid only
    # for the same kernel sources and the same launch (split count, KV bytes).
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if (tr.get("kernel_digest") == attn_kernel_digest() and tr.get("splits") == S
                and tr.get("kv_bytes_per_launch") == kv_l and tr.get("kv_append", "none") == args.append):
            traffic = tr.get("hbm_bytes_per_launch")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": ("split_attn_kernel<128,4,true> (paged_decode_append_attn)" if args.append == "fused"
                           else "split_attn_kernel<128,4,false> (paged_decode_attn)"), "us_per_launch": round(attn_us, 3),
                "algorithmic_bytes_per_launch": alg_l, "kv_bytes_per_launch": kv_l}

    if args.calib_copy_gib > 0:
        n = int(args.calib_copy_gib * (1 << 30))
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: 3 x {n} bytes")
        del src, dst

    # The metric's batch sweep: one layer per batch size, B requests of 4096
    # tokens, each launch after a cache flush, timed from graph replays.
    sweep = None
    if args.sweep:
        rows = graph_sweep([f"sweep{int(b)}" for b in args.sweep.split(",") if b], 20, 7, args.splits)
        sweep = {"timing": "graph replays of 20 x [1 GiB flush, attn(, merge)] minus 20 x [flush], HIP events "
                           "around each replay; median over 7 rounds of the per-round differences",
                 "seq_len": 4096, "n_heads": 32, "n_kv_heads": 8, "head_dim": 128, "page_size": 16, "rows": rows}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_budget, S)
        log(f"[bench] cpu oracle: {cpu['value']} GB/s on {cpu['cores']} threads")

    rec = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode step: 24 layers, B=32, seq_lens~U[1,2048] +1/step, 32 q heads, "
                               "8 kv heads, head_dim 128, page 16; steady bind + 24 x ("
                               + {"none": "", "separate": "kv append, ", "fused": "kv append fused into "}[args.append]
                               + "split attn, merge), hipGraph replay",
                   "batch": B, "n_layers": NL, "n_heads": H, "n_kv_heads": Hkv, "head_dim": D,
                   "page_size": w.page_size, "num_splits": S, "kv_append": args.append,
                   "parallelism": "single GPU",
                   "accumulate": "fp32"},
        "us_per_layer": round(ms_step * 1e3 / NL, 3),
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if sweep is not None:
        rec["batch_sweep"] = sweep
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
