"""Split-KV paged decode attention for MI355X (gfx950).

A thin Python binding over the C ABI of ``libpaged_decode.so``
(``include/paged_decode.h``): it only checks and marshals arguments (torch
tensors -> device pointers, torch streams -> hipStream_t).  Every step of the
decode path runs in the library's HIP kernels; nothing here computes.

    ws = PagedDecode(Config(...), device="cuda")
    S = ws.num_splits(batch)
    ws.bind(batch, PD_BIND_FULL, seq_lens, position_ids, req_to_page)
    for layer in range(n_layers):
        ws.attn(batch, layer, S, q[layer], k_store, v_store, scale)
        ws.merge(batch, S, out[layer])
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _abi
from ._abi import (  # noqa: F401
    PD_BIND_FULL,
    PD_BIND_STEADY,
    PD_E_CAPACITY,
    PD_E_HIP,
    PD_E_INVALID,
    PD_E_SCRATCH,
    PD_E_UNSUPPORTED,
    PD_ERR_BAD_PAGE,
    PD_ERR_EXTEND_OVER_LEN,
    PD_ERR_NEG_SEQ_LEN,
    PD_ERR_SEQ_OVER_TABLE,
    PD_ERR_TOTAL_OVER_CAP,
    PD_OK,
    PagedDecodeError,
)

__all__ = ["Config", "PagedDecode", "GraphPool", "PagedDecodeError", "PD_BIND_FULL", "PD_BIND_STEADY",
           "workspace_bytes", "library_path"]


def library_path() -> str:
    return _abi.LIB_PATH


@dataclass
class Config:
    n_layers: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    page_size: int
    max_batch: int
    max_splits: int
    max_pages_per_req: int
    num_slots: int
    max_total_tokens: int

    def to_c(self) -> _abi.PdConfig:
        return _abi.PdConfig(self.n_layers, self.n_heads, self.n_kv_heads, self.head_dim,
                             self.page_size, self.max_batch, self.max_splits,
                             self.max_pages_per_req, self.num_slots, self.max_total_tokens)


def workspace_bytes(cfg: Config) -> int:
    n = ctypes.c_size_t(0)
    c = cfg.to_c()
    _abi.check("paged_decode_workspace_bytes",
               _abi.lib().paged_decode_workspace_bytes(ctypes.byref(c), ctypes.byref(n)))
    return int(n.value)


def _stream_ptr(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _dev_ptr(t: torch.Tensor, dtype, name: str, numel: int | None = None) -> int:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return t.data_ptr()


class PagedDecode:
    """One workspace: a device arena carved by the library, plus its handle."""

    def __init__(self, cfg: Config, device="cuda"):
        self.cfg = cfg
        self.device = torch.device(device)
        L = _abi.lib()
        nbytes = workspace_bytes(cfg)
        self.arena = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        h = ctypes.c_void_p()
        c = cfg.to_c()
        with torch.cuda.device(self.device):
            _abi.check("paged_decode_init_workspace",
                       L.paged_decode_init_workspace(ctypes.byref(c), ctypes.c_void_p(self.arena.data_ptr()),
                                                     nbytes, ctypes.byref(h)))
        self._h = h
        lay = _abi.PdLayout()
        _abi.check("paged_decode_layout", L.paged_decode_layout(self._h, ctypes.byref(lay)))
        self.layout = {f: getattr(lay, f) for f, _ in _abi.PdLayout._fields_}

    # ---------------------------------------------------------- views -----
    def _view(self, off: int, dtype, shape):
        n = 1
        for s in shape:
            n *= s
        itemsize = torch.empty((), dtype=dtype).element_size()
        return self.arena[off: off + n * itemsize].view(dtype).view(*shape)

    @property
    def kv_indptr(self):
        return self._view(self.layout["kv_indptr"], torch.int32, (self.cfg.max_batch + 1,))

    @property
    def kv_indices(self):
        return self._view(self.layout["kv_indices"], torch.int32, (self.cfg.max_total_tokens,))

    @property
    def o_part(self):
        c = self.cfg
        return self._view(self.layout["o_part"], torch.float32,
                          (c.max_batch, c.n_heads, c.max_splits, c.head_dim))

    @property
    def ml_part(self):
        c = self.cfg
        return self._view(self.layout["ml_part"], torch.float32, (c.max_batch, c.n_heads, c.max_splits, 2))

    @property
    def meta(self):
        return self._view(self.layout["meta"], torch.int32, (16,))

    # ---------------------------------------------------------- calls -----
    def num_splits(self, batch: int, requested: int = 0) -> int:
        s = ctypes.c_int32(0)
        _abi.check("paged_decode_num_splits",
                   _abi.lib().paged_decode_num_splits(self._h, batch, requested, ctypes.byref(s)))
        return int(s.value)

    def bind(self, batch: int, mode: int, seq_lens: torch.Tensor, position_ids, req_to_page: torch.Tensor,
             stream=None) -> None:
        c = self.cfg
        p_sl = _dev_ptr(seq_lens, torch.int32, "seq_lens", batch)
        p_pos = None if position_ids is None else _dev_ptr(position_ids, torch.int32, "position_ids", batch)
        p_tab = _dev_ptr(req_to_page, torch.int32, "req_to_page", batch * c.max_pages_per_req)
        if req_to_page.dim() == 2 and req_to_page.shape[1] != c.max_pages_per_req:
            raise ValueError("req_to_page rows must have max_pages_per_req entries")
        _abi.check("paged_decode_bind",
                   _abi.lib().paged_decode_bind(self._h, batch, mode, p_sl, p_pos, p_tab, _stream_ptr(stream)))

    def bind_contiguous(self, batch: int, mode: int, seq_lens: torch.Tensor, position_ids,
                        req_base: torch.Tensor, stream=None) -> None:
        """Bind for a contiguous cache: request b's tokens sit at slots req_base[b] + t."""
        p_sl = _dev_ptr(seq_lens, torch.int32, "seq_lens", batch)
        p_pos = None if position_ids is None else _dev_ptr(position_ids, torch.int32, "position_ids", batch)
        p_base = _dev_ptr(req_base, torch.int32, "req_base", batch)
        _abi.check("paged_decode_bind_contiguous",
                   _abi.lib().paged_decode_bind_contiguous(self._h, batch, mode, p_sl, p_pos, p_base,
                                                           _stream_ptr(stream)))

    def attn(self, batch: int, layer: int, num_splits: int, q: torch.Tensor, k_store: torch.Tensor,
             v_store: torch.Tensor, scale: float, stream=None) -> None:
        c = self.cfg
        store_numel = c.n_layers * c.num_slots * c.n_kv_heads * c.head_dim
        p_q = _dev_ptr(q, torch.bfloat16, "q", batch * c.n_heads * c.head_dim)
        p_k = _dev_ptr(k_store, torch.bfloat16, "k_store", store_numel)
        p_v = _dev_ptr(v_store, torch.bfloat16, "v_store", store_numel)
        _abi.check("paged_decode_attn",
                   _abi.lib().paged_decode_attn(self._h, batch, layer, num_splits, p_q, p_k, p_v,
                                                float(scale), _stream_ptr(stream)))

    def append_kv(self, batch: int, layer: int, k_new: torch.Tensor, v_new: torch.Tensor, k_store: torch.Tensor,
                  v_store: torch.Tensor, stream=None) -> None:
        """Write each request's new-token K/V rows ([batch, n_kv_heads, D]) at its slot."""
        c = self.cfg
        store_numel = c.n_layers * c.num_slots * c.n_kv_heads * c.head_dim
        row = batch * c.n_kv_heads * c.head_dim
        p_kn = _dev_ptr(k_new, torch.bfloat16, "k_new", row)
        p_vn = _dev_ptr(v_new, torch.bfloat16, "v_new", row)
        p_k = _dev_ptr(k_store, torch.bfloat16, "k_store", store_numel)
        p_v = _dev_ptr(v_store, torch.bfloat16, "v_store", store_numel)
        _abi.check("paged_decode_append_kv",
                   _abi.lib().paged_decode_append_kv(self._h, batch, layer, p_kn, p_vn, p_k, p_v,
                                                     _stream_ptr(stream)))

    def append_attn(self, batch: int, layer: int, num_splits: int, q: torch.Tensor, k_new: torch.Tensor,
                    v_new: torch.Tensor, k_store: torch.Tensor, v_store: torch.Tensor, scale: float,
                    stream=None) -> None:
        """append_kv() and attn() in one launch (bit-identical results)."""
        c = self.cfg
        store_numel = c.n_layers * c.num_slots * c.n_kv_heads * c.head_dim
        row = batch * c.n_kv_heads * c.head_dim
        p_q = _dev_ptr(q, torch.bfloat16, "q", batch * c.n_heads * c.head_dim)
        p_kn = _dev_ptr(k_new, torch.bfloat16, "k_new", row)
        p_vn = _dev_ptr(v_new, torch.bfloat16, "v_new", row)
        p_k = _dev_ptr(k_store, torch.bfloat16, "k_store", store_numel)
        p_v = _dev_ptr(v_store, torch.bfloat16, "v_store", store_numel)
        _abi.check("paged_decode_append_attn",
                   _abi.lib().paged_decode_append_attn(self._h, batch, layer, num_splits, p_q, p_kn, p_vn, p_k,
                                                       p_v, float(scale), _stream_ptr(stream)))

    def bind_extend(self, batch: int, seq_lens: torch.Tensor, extend_lens: torch.Tensor, req_to_page=None,
                    req_base=None, stream=None) -> None:
        """Extend / prefill bind: the last extend_lens[b] of seq_lens[b] tokens are new (query rows)."""
        c = self.cfg
        p_sl = _dev_ptr(seq_lens, torch.int32, "seq_lens", batch)
        p_ext = _dev_ptr(extend_lens, torch.int32, "extend_lens", batch)
        p_tab = None if req_to_page is None else _dev_ptr(req_to_page, torch.int32, "req_to_page",
                                                           batch * c.max_pages_per_req)
        p_base = None if req_base is None else _dev_ptr(req_base, torch.int32, "req_base", batch)
        _abi.check("paged_decode_bind_extend",
                   _abi.lib().paged_decode_bind_extend(self._h, batch, p_sl, p_ext, p_tab, p_base,
                                                       _stream_ptr(stream)))

    def prefill_attn(self, batch: int, layer: int, q: torch.Tensor, k_store: torch.Tensor, v_store: torch.Tensor,
                     scale: float, out: torch.Tensor, stream=None) -> None:
        """Causal attention of the new tokens of the last extend bind (q, out: [rows, n_heads, head_dim])."""
        c = self.cfg
        store_numel = c.n_layers * c.num_slots * c.n_kv_heads * c.head_dim
        if q.dim() != 3 or q.shape[1:] != (c.n_heads, c.head_dim) or out.shape != q.shape:
            raise ValueError("q and out must be [rows, n_heads, head_dim] with the same shape")
        p_q = _dev_ptr(q, torch.bfloat16, "q")
        p_o = _dev_ptr(out, torch.bfloat16, "out")
        p_k = _dev_ptr(k_store, torch.bfloat16, "k_store", store_numel)
        p_v = _dev_ptr(v_store, torch.bfloat16, "v_store", store_numel)
        _abi.check("paged_decode_prefill_attn",
                   _abi.lib().paged_decode_prefill_attn(self._h, batch, layer, p_q, int(q.shape[0]), p_k, p_v,
                                                        float(scale), p_o, _stream_ptr(stream)))

    @property
    def qo_indptr(self):
        return self._view(self.layout["qo_indptr"], torch.int32, (self.cfg.max_batch + 1,))

    @property
    def item_indptr(self):
        """Extend bind: prefix sum of the prefill work items, in schedule order."""
        return self._view(self.layout["item_indptr"], torch.int32, (self.cfg.max_batch + 1,))

    @property
    def req_order(self):
        """Extend bind: the requests in schedule order (decreasing length)."""
        return self._view(self.layout["req_order"], torch.int32, (self.cfg.max_batch,))

    def merge(self, batch: int, num_splits: int, out: torch.Tensor, stream=None) -> None:
        c = self.cfg
        p_o = _dev_ptr(out, torch.bfloat16, "out", batch * c.n_heads * c.head_dim)
        _abi.check("paged_decode_merge",
                   _abi.lib().paged_decode_merge(self._h, batch, num_splits, p_o, _stream_ptr(stream)))

    def attn_merge_noalloc(self, batch: int, layer: int, num_splits: int, q: torch.Tensor, k_store: torch.Tensor,
                           v_store: torch.Tensor, scale: float, out: torch.Tensor, stream=None) -> None:
        """attn() + merge() with the split partials in the library's static scratch array (no allocation)."""
        c = self.cfg
        store_numel = c.n_layers * c.num_slots * c.n_kv_heads * c.head_dim
        p_q = _dev_ptr(q, torch.bfloat16, "q", batch * c.n_heads * c.head_dim)
        p_k = _dev_ptr(k_store, torch.bfloat16, "k_store", store_numel)
        p_v = _dev_ptr(v_store, torch.bfloat16, "v_store", store_numel)
        p_o = _dev_ptr(out, torch.bfloat16, "out", batch * c.n_heads * c.head_dim)
        _abi.check("paged_decode_attn_merge_noalloc",
                   _abi.lib().paged_decode_attn_merge_noalloc(self._h, batch, layer, num_splits, p_q, p_k, p_v,
                                                              float(scale), p_o, _stream_ptr(stream)))

    def read_error(self, stream=None) -> int:
        v = ctypes.c_uint32(0)
        _abi.check("paged_decode_read_error",
                   _abi.lib().paged_decode_read_error(self._h, ctypes.byref(v), _stream_ptr(stream)))
        return int(v.value)

    def close(self) -> None:
        if getattr(self, "_h", None):
            _abi.lib().paged_decode_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class GraphPool:
    """Batch-size graph pool over a workspace (``paged_decode_graph_pool_*``).

    The tensors are the caller's fixed step buffers, each sized for the
    workspace's max_batch (see ``pd_step_buffers``); the pool keeps references
    to them.  ``step(batch)`` runs one steady decode step of requests
    0 .. batch-1 through the smallest captured key >= batch.
    """

    def __init__(self, ws: PagedDecode, *, seq_lens, position_ids, q, k_store, v_store, out, scale,
                 req_to_page=None, req_base=None, k_new=None, v_new=None, eager=False):
        c = ws.cfg
        nb = c.max_batch
        store_numel = c.n_layers * c.num_slots * c.n_kv_heads * c.head_dim
        per_layer = c.n_layers * nb * c.n_heads * c.head_dim
        new_numel = c.n_layers * nb * c.n_kv_heads * c.head_dim
        b = _abi.PdStepBuffers()
        b.seq_lens = _dev_ptr(seq_lens, torch.int32, "seq_lens", nb)
        b.position_ids = _dev_ptr(position_ids, torch.int32, "position_ids", nb)
        b.req_to_page = None if req_to_page is None else _dev_ptr(req_to_page, torch.int32, "req_to_page",
                                                                   nb * c.max_pages_per_req)
        b.req_base = None if req_base is None else _dev_ptr(req_base, torch.int32, "req_base", nb)
        b.q = _dev_ptr(q, torch.bfloat16, "q", per_layer)
        b.k_store = _dev_ptr(k_store, torch.bfloat16, "k_store", store_numel)
        b.v_store = _dev_ptr(v_store, torch.bfloat16, "v_store", store_numel)
        b.k_new = None if k_new is None else _dev_ptr(k_new, torch.bfloat16, "k_new", new_numel)
        b.v_new = None if v_new is None else _dev_ptr(v_new, torch.bfloat16, "v_new", new_numel)
        b.out = _dev_ptr(out, torch.bfloat16, "out", per_layer)
        b.scale = float(scale)
        self.ws = ws
        self._keep = (seq_lens, position_ids, req_to_page, req_base, q, k_store, v_store, k_new, v_new, out)
        self._buf = b
        h = ctypes.c_void_p()
        _abi.check("paged_decode_graph_pool_create",
                   _abi.lib().paged_decode_graph_pool_create(ws._h, ctypes.byref(b),
                                                             _abi.PD_POOL_EAGER if eager else 0, ctypes.byref(h)))
        self._p = h

    def warmup(self) -> None:
        _abi.check("paged_decode_graph_pool_warmup", _abi.lib().paged_decode_graph_pool_warmup(self._p))

    def step(self, batch: int, stream=None) -> None:
        _abi.check("paged_decode_graph_pool_step",
                   _abi.lib().paged_decode_graph_pool_step(self._p, batch, _stream_ptr(stream)))

    def keys(self):
        """[(key, num_splits, replays_a_graph)] for every key."""
        L = _abi.lib()
        n = ctypes.c_int32(0)
        _abi.check("paged_decode_graph_pool_num_keys", L.paged_decode_graph_pool_num_keys(self._p, ctypes.byref(n)))
        out = []
        for i in range(n.value):
            k, s, g = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
            _abi.check("paged_decode_graph_pool_key",
                       L.paged_decode_graph_pool_key(self._p, i, ctypes.byref(k), ctypes.byref(s), ctypes.byref(g)))
            out.append((k.value, s.value, bool(g.value)))
        return out

    def close(self) -> None:
        if getattr(self, "_p", None):
            _abi.lib().paged_decode_graph_pool_destroy(self._p)
            self._p = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
