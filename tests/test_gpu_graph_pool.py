"""GPU: the batch-size graph pool (paged_decode_graph_pool_*).

Every step of the pool must equal, bit for bit, the eager calls at the same
batch with the key's split count, and leave the padding requests (batch ..
key-1) untouched.  A pool forced to run eagerly must give the same bits.  The
pool's own outputs (and, with the fused append, its stores) are compared with
the oracle after every step, at the lengths the step advanced to.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from paged_kv_decode_10_amd import PD_BIND_FULL, PD_BIND_STEADY, GraphPool
from tests.gpu_harness import assert_close_out, make_ws, say, to_device

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")


def _bits(t):
    return t.contiguous().view(torch.int16)


def _workload(layout="paged", append=False):
    # With the fused append the slots past each length start as NaN: only the
    # append may make them valid.
    return workloads.make_custom("pool", seed=80, n_layers=2,
                                 seq_lens=lambda g: torch.randint(1, 700, (6,), generator=g).tolist(),
                                 n_heads=16, n_kv_heads=4, head_dim=128, page_size=16, growth=12, layout=layout,
                                 nan_growth=append)


def _new_rows_host(w, seed=9):
    g = torch.Generator().manual_seed(seed)
    shape = (w.n_layers, w.batch, w.n_kv_heads, w.head_dim)
    return (torch.randn(shape, generator=g).to(torch.bfloat16),
            torch.randn(shape, generator=g).to(torch.bfloat16))


def _new_rows(w, seed=9):
    k, v = _new_rows_host(w, seed)
    return k.cuda(), v.cuda()


class _OracleState:
    """Host copies of the lengths and stores, advanced by the oracle."""

    def __init__(self, w, append, layout):
        self.w = w
        self.L = w.seq_lens.numpy().astype(np.int64).copy()
        self.k = w.k_store.clone()
        self.v = w.v_store.clone()
        self.kn, self.vn = _new_rows_host(w) if append else (None, None)
        self.layout = layout

    def step(self, B):
        """A steady step of requests 0 .. B-1: their lengths +1, the new rows
        appended (fused-append pools), then attention per layer: [layers, B, H, D]."""
        w = self.w
        self.L[:B] += 1
        L = self.L[:B]
        table = w.req_to_page.numpy()[:B]
        ip = oracle.kv_indptr(L)
        ix = (oracle.kv_indices_contiguous(L, w.meta["req_base"].numpy()[:B]) if self.layout == "contiguous"
              else oracle.kv_indices(L, table, w.page_size))
        outs = []
        for l in range(w.n_layers):
            if self.kn is not None:
                slots = oracle.append_slots(L, table, w.page_size)
                self.k[l] = oracle.append_kv(self.k[l], self.kn[l][:B], slots)
                self.v[l] = oracle.append_kv(self.v[l], self.vn[l][:B], slots)
            o, _ = oracle.decode_attention(w.q[l][:B], self.k[l], self.v[l], L, ip, ix, w.scale, w.n_kv_heads)
            outs.append(o)
        return np.stack(outs)


class _State:
    def __init__(self, w, append, layout):
        self.w = w
        self.dev = to_device(w)
        self.ws = make_ws(w)
        self.out = torch.full((w.n_layers, w.batch, w.n_heads, w.head_dim), SENTINEL, dtype=torch.bfloat16,
                              device="cuda")
        self.kn, self.vn = _new_rows(w) if append else (None, None)
        self.base = w.meta["req_base"].cuda() if layout == "contiguous" else None
        self.bind(w.batch, PD_BIND_FULL)

    def bind(self, B, mode):
        d = self.dev
        if self.base is not None:
            self.ws.bind_contiguous(B, mode, d.seq_lens, d.position_ids, self.base)
        else:
            self.ws.bind(B, mode, d.seq_lens, d.position_ids, d.req_to_page)

    def eager_step(self, B, S):
        w, d = self.w, self.dev
        self.bind(B, PD_BIND_STEADY)
        for l in range(w.n_layers):
            if self.kn is not None:
                self.ws.append_attn(B, l, S, d.q[l][:B], self.kn[l][:B], self.vn[l][:B], d.k, d.v, w.scale)
            else:
                self.ws.attn(B, l, S, d.q[l][:B], d.k, d.v, w.scale)
            self.ws.merge(B, S, self.out[l][:B])

    def pool(self, eager=False):
        d = self.dev
        return GraphPool(self.ws, seq_lens=d.seq_lens, position_ids=d.position_ids, q=d.q, k_store=d.k,
                         v_store=d.v, out=self.out, scale=self.w.scale,
                         req_to_page=None if self.base is not None else d.req_to_page, req_base=self.base,
                         k_new=self.kn, v_new=self.vn, eager=eager)


@pytest.mark.parametrize("append,layout", [(False, "paged"), (False, "contiguous"), (True, "paged"), (True, "contiguous")])
def test_pool_steps_match_eager(append, layout):
    say(f"[pool] append={append} layout={layout}")
    w = _workload(layout, append)
    ref, got, eag = _State(w, append, layout), _State(w, append, layout), _State(w, append, layout)
    orc = _OracleState(w, append, layout)
    pool = got.pool()
    pool.warmup()
    keys = pool.keys()
    assert [k for k, _, _ in keys] == [1, 2, 4, 6]
    assert all(g for _, _, g in keys), keys
    eager_pool = eag.pool(eager=True)
    eager_pool.warmup()
    assert not any(g for _, _, g in eager_pool.keys())
    split_of = {k: s for k, s, _ in keys}
    for B in (6, 3, 3, 1, 4, 2, 5):
        key = min(k for k in split_of if k >= B)
        seq_before = got.dev.seq_lens.clone()
        out_before = got.out.clone()
        ref.eager_step(B, split_of[key])
        a0 = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
        pool.step(B)
        eager_pool.step(B)
        torch.cuda.synchronize()
        assert torch.cuda.memory_stats().get("allocation.all.allocated", 0) == a0, "the pool step allocated"
        for s in (got, eag):
            assert torch.equal(_bits(s.out[:, :B]), _bits(ref.out[:, :B])), f"B={B} key={key}"
            assert torch.equal(_bits(s.out[:, B:]), _bits(out_before[:, B:])), "padding outputs were written"
            assert torch.equal(s.dev.seq_lens, ref.dev.seq_lens), "lengths differ"
            assert torch.equal(_bits(s.dev.k), _bits(ref.dev.k)) and torch.equal(_bits(s.dev.v), _bits(ref.dev.v))
        assert torch.equal(got.dev.seq_lens[B:], seq_before[B:]), "padding lengths were advanced"
        assert torch.equal(got.dev.seq_lens[:B], seq_before[:B] + 1)
        # the pool's replayed (or eager) step against the oracle
        want = orc.step(B)
        assert got.dev.seq_lens.cpu().numpy().tolist() == orc.L.tolist()
        assert_close_out(got.out[:, :B].double().cpu().numpy(), want, f"pool step B={B} key={key}")
        if append:
            assert torch.equal(_bits(got.dev.k.cpu()), _bits(orc.k)) and torch.equal(_bits(got.dev.v.cpu()),
                                                                                     _bits(orc.v)), "stores"
    assert got.ws.read_error() == 0
    pool.close()
    eager_pool.close()


def test_per_layer_calls_after_pool_steps():
    """The pool keeps the handle's record of the bound batch in step with what
    the device holds: warmup (capture only) leaves the bind it found, and a
    step of `batch` requests binds exactly those, so per-layer calls made
    after it take that batch (and reproduce the step's own outputs bit for
    bit) and any other batch is rejected on the host."""
    from paged_kv_decode_10_amd import PD_E_INVALID, PagedDecodeError

    say("[pool] per-layer calls after pool steps")
    w = _workload()
    st = _State(w, append=False, layout="paged")  # bound: a full bind of all 6 requests
    pool = st.pool()
    pool.warmup()
    keys = {k: s for k, s, _ in pool.keys()}
    d = st.dev

    def rejected(fn):
        with pytest.raises(PagedDecodeError) as e:
            fn()
        assert e.value.status == PD_E_INVALID

    out = torch.full((w.batch, w.n_heads, w.head_dim), SENTINEL, dtype=torch.bfloat16, device="cuda")
    rejected(lambda: st.ws.attn(4, 0, keys[4], d.q[0][:4], d.k, d.v, w.scale))  # still the full bind of 6
    st.ws.attn(w.batch, 0, keys[6], d.q[0], d.k, d.v, w.scale)
    st.ws.merge(w.batch, keys[6], out)
    for B in (3, 5, 1):
        key = min(k for k in keys if k >= B)
        pool.step(B)
        torch.cuda.synchronize()
        rejected(lambda: st.ws.attn(key, 0, keys[key], d.q[0][:key], d.k, d.v, w.scale) if key != B else
                 st.ws.merge(B + 1, keys[key], out[:B + 1]))
        for layer in range(w.n_layers):
            out.fill_(SENTINEL)
            st.ws.attn(B, layer, keys[key], d.q[layer][:B], d.k, d.v, w.scale)
            st.ws.merge(B, keys[key], out[:B])
            torch.cuda.synchronize()
            assert torch.equal(_bits(out[:B]), _bits(st.out[layer, :B])), f"B={B} layer={layer}"
    assert st.ws.read_error() == 0
    pool.close()
