"""Seeded synthetic inputs for split-KV paged decode attention.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It only *draws* inputs: sequence lengths, a shuffled page
assignment, queries and the paged K/V stores.  It holds none of the method's
arithmetic (no prefix sums, no index lists, no softmax); those are computed
independently by the oracle and by the HIP kernels.

Layouts (all CPU torch tensors):
  seq_lens      int32 [B]
  position_ids  int32 [B]            (= seq_lens - 1: the position of the
                                      newest token, whose K/V is already stored)
  req_to_page   int32 [B, max_pages_per_req]   page ids, -1 where unused
  q             bf16  [n_layers, B, n_heads, head_dim]  (prefill workloads:
                                      [n_layers, sum(extend_lens), n_heads, head_dim])
  k_store       bf16  [n_layers, num_slots, n_kv_heads, head_dim]
  v_store       bf16  [n_layers, num_slots, n_kv_heads, head_dim]
Page p owns slots [p*page_size, (p+1)*page_size).  Pages that no request owns
are filled with NaN so that any stray read poisons the result.

Draw order from one CPU ``torch.Generator`` seeded per workload:
seq_lens -> page permutation -> q -> K store -> V store.  bf16 values are
float32 N(0,1) draws rounded to bf16 (round-to-nearest-even).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

__all__ = ["Workload", "make", "make_custom", "CONFIGS", "PREFILL_CONFIGS"]


@dataclass
class Workload:
    name: str
    n_layers: int
    batch: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    max_pages_per_req: int
    scale: float
    seq_lens: torch.Tensor
    position_ids: torch.Tensor
    req_to_page: torch.Tensor
    q: torch.Tensor
    k_store: torch.Tensor
    v_store: torch.Tensor
    meta: dict = field(default_factory=dict)

    @property
    def num_slots(self) -> int:
        return self.num_pages * self.page_size

    @property
    def group(self) -> int:
        return self.n_heads // self.n_kv_heads

    def kv_bytes_per_layer(self, seq_lens=None) -> int:
        """Bytes of K plus V one layer must read: sum(L_b) * Hkv * D * 2 B * 2."""
        L = self.seq_lens if seq_lens is None else seq_lens
        return int(L.to(torch.int64).sum()) * self.n_kv_heads * self.head_dim * 4


def _pages_needed(lengths, page_size):
    return [-(-int(x) // page_size) for x in lengths]


def _fill_store(gen, n_layers, num_slots, hkv, d, chunk_rows=1 << 16):
    """N(0,1) float32 draws rounded to bf16, generated in row chunks to bound
    host memory; the chunk order is fixed so the result is deterministic."""
    out = torch.empty((n_layers, num_slots, hkv, d), dtype=torch.bfloat16)
    flat = out.view(n_layers * num_slots, hkv * d)
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(r0 + chunk_rows, flat.shape[0])
        flat[r0:r1] = torch.randn((r1 - r0, hkv * d), generator=gen).to(torch.bfloat16)
    return out


def make_custom(name, *, seed, n_layers, seq_lens, n_heads, n_kv_heads, head_dim,
                page_size=16, num_pages=None, pool_factor=1.25, growth=0,
                max_pages_per_req=None, q_scale=1.0, scale=None,
                nan_unassigned=True, shuffle=True, layout="paged", extend_lens=None, nan_growth=False):
    """Build a workload.

    ``seq_lens`` is either a list of ints or a callable ``gen -> list`` that
    draws them (so that the draw happens first, from the seeded generator).
    ``growth`` reserves pages for that many future tokens per request (decode
    steps that add one token each), so steady-state steps need no new pages.
    ``shuffle=False`` assigns pages in order instead of by the seeded
    permutation (a locality experiment; the named workloads shuffle).
    ``layout="contiguous"`` gives every request one contiguous region of
    max_pages_per_req pages instead (regions in a seeded random order, plus
    one spare region of NaN); ``meta["req_base"]`` holds each request's first
    slot, and ``req_to_page`` lists the region's pages in order.
    ``extend_lens`` (a list or a callable ``(gen, lens) -> list``, drawn right
    after the lengths) makes a prefill / extend workload: request b's last
    extend_lens[b] tokens are new, and q holds one row per new token,
    [n_layers, sum(extend_lens), n_heads, head_dim], request after request.
    ``nan_growth=True`` also fills the slots a request owns past its current
    length (its reserved growth, and the rest of its last page) with NaN, as a
    cache whose new pages hold stale data would: only a KV append may make
    them valid.
    """
    gen = torch.Generator().manual_seed(seed)
    lens = list(seq_lens(gen)) if callable(seq_lens) else list(seq_lens)
    B = len(lens)
    ext = None
    if extend_lens is not None:
        ext = list(extend_lens(gen, lens)) if callable(extend_lens) else list(extend_lens)
        if len(ext) != B or any(e < 0 or e > x for e, x in zip(ext, lens)):
            raise ValueError("extend_lens must have one entry per request, 0 <= extend_lens[b] <= seq_lens[b]")
    pages_b = _pages_needed([x + growth for x in lens], page_size)
    if layout == "contiguous":
        mppr = max_pages_per_req if max_pages_per_req is not None else max(1, max(pages_b))
        if mppr < max(pages_b):
            raise ValueError("max_pages_per_req smaller than a request's page count")
        pages_b = [mppr] * B
        num_pages = (B + 1) * mppr
        regions = torch.randperm(B + 1, generator=gen).to(torch.int32)
        perm = (regions[:, None] * mppr + torch.arange(mppr, dtype=torch.int32)[None, :]).flatten()
        max_pages_per_req = mppr
    elif layout != "paged":
        raise ValueError(f"unknown layout {layout}")
    total_pages = sum(pages_b)
    if num_pages is None:
        num_pages = max(total_pages, math.ceil(pool_factor * (sum(lens) + growth * B) / page_size))
    if num_pages < total_pages:
        raise ValueError("pool too small for the requested lengths")
    if layout == "paged":
        perm = torch.randperm(num_pages, generator=gen).to(torch.int32)
        if not shuffle:  # pages in order (same draw order, permutation unused)
            perm = torch.arange(num_pages, dtype=torch.int32)
    mppr = max_pages_per_req if max_pages_per_req is not None else max(1, max(pages_b))
    if mppr < max(pages_b):
        raise ValueError("max_pages_per_req smaller than a request's page count")
    req_to_page = torch.full((B, mppr), -1, dtype=torch.int32)
    off = 0
    for b, pb in enumerate(pages_b):
        req_to_page[b, :pb] = perm[off:off + pb]
        off += pb
    q_rows = B if ext is None else sum(ext)
    q = torch.randn((n_layers, q_rows, n_heads, head_dim), generator=gen)
    if q_scale != 1.0:
        q = q * q_scale
    q = q.to(torch.bfloat16)
    num_slots = num_pages * page_size
    k_store = _fill_store(gen, n_layers, num_slots, n_kv_heads, head_dim)
    v_store = _fill_store(gen, n_layers, num_slots, n_kv_heads, head_dim)
    if nan_unassigned:
        owned = torch.zeros(num_pages, dtype=torch.bool)
        owned[perm[:total_pages].long()] = True
        free_pages = (~owned).nonzero().flatten()
        if free_pages.numel():
            slot_idx = (free_pages[:, None] * page_size + torch.arange(page_size)[None, :]).flatten()
            k_store[:, slot_idx] = float("nan")
            v_store[:, slot_idx] = float("nan")
    if nan_growth:
        for b, pb in enumerate(pages_b):
            pos = torch.arange(lens[b], pb * page_size)
            if pos.numel():
                slots = req_to_page[b, pos // page_size].long() * page_size + pos % page_size
                k_store[:, slots] = float("nan")
                v_store[:, slots] = float("nan")
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    seq = torch.tensor(lens, dtype=torch.int32)
    return Workload(name=name, n_layers=n_layers, batch=B, n_heads=n_heads,
                    n_kv_heads=n_kv_heads, head_dim=head_dim, page_size=page_size,
                    num_pages=num_pages, max_pages_per_req=mppr, scale=float(torch.tensor(scale, dtype=torch.float32)),
                    seq_lens=seq, position_ids=(seq - 1).clamp(min=0), req_to_page=req_to_page,
                    q=q, k_store=k_store, v_store=v_store,
                    meta={"seed": seed, "growth": growth, "q_scale": q_scale, "layout": layout,
                          "extend_lens": None if ext is None else torch.tensor(ext, dtype=torch.int32),
                          "req_base": (req_to_page[:, 0].to(torch.int32) * page_size if layout == "contiguous"
                                       else None)})


def _uniform_lens(B, lo, hi):
    # integers, inclusive at both ends
    return lambda gen: torch.randint(lo, hi + 1, (B,), generator=gen).tolist()


# Named workloads: the shapes of the decode configurations this kernel is
# measured on.  ``tiny`` is small enough for pure-Python checks.
CONFIGS = {
    "tiny": dict(seed=0, n_layers=1, seq_lens=[37, 100], n_heads=4, n_kv_heads=2,
                 head_dim=64, page_size=16, num_pages=64, scale=1.0 / 8.0),
    "b1": dict(seed=1, n_layers=1, seq_lens=[4096], n_heads=32, n_kv_heads=8,
               head_dim=128, page_size=16, num_pages=8192),
    "b16": dict(seed=2, n_layers=1, seq_lens=_uniform_lens(16, 512, 8192), n_heads=32,
                n_kv_heads=8, head_dim=128, page_size=16),
    "step": dict(seed=3, n_layers=24, seq_lens=_uniform_lens(32, 1, 2048), n_heads=32,
                 n_kv_heads=8, head_dim=128, page_size=16, growth=256),
    "long": dict(seed=4, n_layers=1, seq_lens=[131072] * 4, n_heads=64, n_kv_heads=8,
                 head_dim=128, page_size=16, q_scale=3.0),
}


def _extend_uniform(lo, hi):
    """New tokens per request ~ U{lo..hi}, at most the request's length."""
    def draw(gen, lens):
        return [min(int(x), int(torch.randint(lo, hi + 1, (1,), generator=gen))) for x in lens]
    return draw


PREFILL_CONFIGS = {
    # 2 requests: a fresh prompt (no prefix) and an extend over a 9-token prefix
    "prefill_tiny": dict(seed=20, n_layers=1, seq_lens=[21, 40], extend_lens=[21, 31], n_heads=4,
                         n_kv_heads=2, head_dim=64, page_size=16),
    # extends: prefix ~U[0, 2048] plus U[64, 1024] new tokens, 4 requests
    "prefill": dict(seed=21, n_layers=1, seq_lens=_uniform_lens(4, 64, 3072), extend_lens=_extend_uniform(64, 1024),
                    n_heads=32, n_kv_heads=8, head_dim=128, page_size=16),
}


def make(name: str, **overrides) -> Workload:
    """Build a named workload; ``sweepN`` gives B=N requests of 4096 tokens."""
    if name.startswith("sweep"):
        B = int(name[5:])
        cfg = dict(seed=5, n_layers=1, seq_lens=[4096] * B, n_heads=32, n_kv_heads=8,
                   head_dim=128, page_size=16)
    elif name in PREFILL_CONFIGS:
        cfg = dict(PREFILL_CONFIGS[name])
    else:
        cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    return make_custom(name, **cfg)
