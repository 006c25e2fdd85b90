"""GPU: paged prefill / extend attention (causal over the request's cache,
ragged query rows) through the C ABI, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from paged_kv_decode_10_amd import PD_ERR_EXTEND_OVER_LEN, PD_ERR_TOTAL_OVER_CAP
from tests.gpu_harness import assert_close_out, make_ws, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")


def _run(w, layer=0, contiguous=False):
    dev = to_device(w)
    ext = w.meta["extend_lens"].cuda()
    ws = make_ws(w)
    if contiguous:
        ws.bind_extend(w.batch, dev.seq_lens, ext, req_base=w.meta["req_base"].cuda())
    else:
        ws.bind_extend(w.batch, dev.seq_lens, ext, req_to_page=dev.req_to_page)
    out = torch.full(dev.q[layer].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    ws.prefill_attn(w.batch, layer, dev.q[layer], dev.k, dev.v, w.scale, out)
    torch.cuda.synchronize()
    return ws, out.float().cpu().numpy()


def _oracle(w, layer=0):
    L = w.seq_lens.numpy()
    n = w.meta["extend_lens"].numpy()
    if w.meta.get("layout") == "contiguous":
        ix = oracle.kv_indices_contiguous(L, w.meta["req_base"].numpy())
        ip = oracle.kv_indptr(L)
    else:
        ip, ix = oracle.bind_full(L, w.req_to_page.numpy(), w.page_size)
    return oracle.prefill_attention(w.q[layer], w.k_store[layer], w.v_store[layer], L, n, ip, ix, w.scale,
                                    w.n_kv_heads)


def test_prefill_tiny():
    say("[prefill] tiny")
    w = workloads.make("prefill_tiny")
    ws, got = _run(w)
    assert ws.read_error() == 0
    assert ws.qo_indptr[:3].cpu().tolist() == oracle.qo_indptr(w.meta["extend_lens"].numpy()).tolist()
    ref, _ = _oracle(w)
    assert np.isfinite(got).all()
    assert_close_out(got, ref, "prefill tiny")


@pytest.mark.parametrize("G,hkv,D,ps", [(1, 4, 128, 16), (2, 2, 64, 16), (4, 8, 128, 16), (8, 1, 128, 32),
                                        (16, 2, 64, 16), (3, 2, 128, 7), (4, 2, 128, 1)])
def test_prefill_shapes(G, hkv, D, ps):
    say(f"[prefill] G={G} hkv={hkv} D={D} ps={ps}")
    w = workloads.make_custom("pshape", seed=200 + G * 3 + D + ps, n_layers=2,
                              seq_lens=[1, 37, 300, 64, 17, 90], extend_lens=[1, 37, 45, 1, 0, 33],
                              n_heads=G * hkv, n_kv_heads=hkv, head_dim=D, page_size=ps)
    ws, got = _run(w, layer=1)
    assert ws.read_error() == 0
    ref, _ = _oracle(w, layer=1)
    assert_close_out(got, ref, "prefill shapes")


def test_prefill_one_new_token_equals_decode():
    """n_b = 1: each request's single query is the decode query over all L_b tokens."""
    say("[prefill] n=1 vs decode")
    w = workloads.make_custom("pdec", seed=210, n_layers=1, seq_lens=[100, 1, 2000, 513], extend_lens=[1, 1, 1, 1],
                              n_heads=32, n_kv_heads=8, head_dim=128, page_size=16)
    ws, got = _run(w)
    L = w.seq_lens.numpy()
    ip, ix = oracle.bind_full(L, w.req_to_page.numpy(), w.page_size)
    ref, _ = oracle.decode_attention(w.q[0], w.k_store[0], w.v_store[0], L, ip, ix, w.scale, w.n_kv_heads)
    assert_close_out(got, ref, "prefill n=1")


def test_prefill_fresh_prompt_first_token_bit_exact():
    """No prefix: token 0 of a fresh prompt sees only itself -> its V row exactly."""
    w = workloads.make("prefill_tiny")
    _, got = _run(w)
    slot0 = int(w.req_to_page[0, 0]) * w.page_size
    for h in range(w.n_heads):
        assert np.array_equal(got[0, h], w.v_store[0, slot0, h // w.group].float().numpy()), h


def test_prefill_contiguous_layout():
    say("[prefill] contiguous")
    w = workloads.make_custom("pcont", seed=220, n_layers=1, seq_lens=[500, 64, 1200], extend_lens=[200, 64, 7],
                              n_heads=16, n_kv_heads=4, head_dim=128, page_size=16, layout="contiguous")
    ws, got = _run(w, contiguous=True)
    assert ws.read_error() == 0
    ref, _ = _oracle(w)
    assert_close_out(got, ref, "prefill contiguous")


def test_prefill_config():
    say("[prefill] 4 requests, extends of 64..1024 new tokens over prefixes")
    w = workloads.make("prefill")
    ws, got = _run(w)
    assert ws.read_error() == 0
    ref, _ = _oracle(w)
    assert_close_out(got, ref, "prefill config")


def test_rows_past_the_q_capacity_are_not_computed():
    """q / out hold fewer rows than the extend bind's total: the rows past them
    are skipped (nothing is read or written out of bounds) and flagged."""
    w = workloads.make("prefill_tiny")
    dev = to_device(w)
    ws = make_ws(w)
    ws.bind_extend(w.batch, dev.seq_lens, w.meta["extend_lens"].cuda(), req_to_page=dev.req_to_page)
    rows = 30  # of 52
    q = dev.q[0][:rows].contiguous()
    out = torch.full((rows + 8, w.n_heads, w.head_dim), 3.0, dtype=torch.bfloat16, device="cuda")
    ws.prefill_attn(w.batch, 0, q, dev.k, dev.v, w.scale, out[:rows])
    torch.cuda.synchronize()
    assert ws.read_error() & PD_ERR_TOTAL_OVER_CAP
    ref, _ = _oracle(w)
    assert_close_out(out[:rows].float().cpu().numpy(), ref[:rows], "prefill rows within the capacity")
    assert torch.all(out[rows:].float() == 3.0)


def test_extend_over_length_is_flagged():
    w = workloads.make_custom("pbad", seed=230, n_layers=1, seq_lens=[20, 30], extend_lens=[5, 10], n_heads=4,
                              n_kv_heads=2, head_dim=64, page_size=16)
    dev = to_device(w)
    ws = make_ws(w)
    ext = torch.tensor([25, 10], dtype=torch.int32, device="cuda")
    ws.bind_extend(w.batch, dev.seq_lens, ext, req_to_page=dev.req_to_page)
    torch.cuda.synchronize()
    assert ws.read_error() & PD_ERR_EXTEND_OVER_LEN
    assert ws.qo_indptr[:3].cpu().tolist() == [0, 20, 30]


def test_prefill_repeated_launches_bit_identical():
    """Items are handed out dynamically; the result must not depend on the
    schedule, and the work counter must be back at zero after every launch
    (else a later launch would skip items and leave NaN rows)."""
    w = workloads.make("prefill")
    dev = to_device(w)
    ws = make_ws(w)
    ws.bind_extend(w.batch, dev.seq_lens, w.meta["extend_lens"].cuda(), req_to_page=dev.req_to_page)
    outs = []
    for _ in range(4):
        out = torch.full(dev.q[0].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        ws.prefill_attn(w.batch, 0, dev.q[0], dev.k, dev.v, w.scale, out)
        torch.cuda.synchronize()
        outs.append(out.view(torch.int16).cpu())
    assert torch.isfinite(outs[0].view(torch.bfloat16).float()).all()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    # a second bind with a different mix reuses the counter
    ext2 = (w.meta["extend_lens"] // 2).cuda()
    ws.bind_extend(w.batch, dev.seq_lens, ext2, req_to_page=dev.req_to_page)
    rows = int(ext2.sum())
    out = torch.full((rows, w.n_heads, w.head_dim), float("nan"), dtype=torch.bfloat16, device="cuda")
    # the new tokens are the last n_b/2 of each request: their query rows
    qrows = torch.cat([dev.q[0][int(s) - int(e):int(s)] for s, e in
                       zip(torch.cumsum(w.meta["extend_lens"], 0), ext2.cpu())]).contiguous()
    ws.prefill_attn(w.batch, 0, qrows, dev.k, dev.v, w.scale, out)
    torch.cuda.synchronize()
    assert ws.read_error() == 0
    L = w.seq_lens.numpy()
    ip, ix = oracle.bind_full(L, w.req_to_page.numpy(), w.page_size)
    ref, _ = oracle.prefill_attention(qrows.cpu(), w.k_store[0], w.v_store[0], L, ext2.cpu().numpy(), ip, ix,
                                      w.scale, w.n_kv_heads)
    assert_close_out(out.float().cpu().numpy(), ref, "prefill after a rebind")


@pytest.mark.parametrize("B", [1, 2, 5, 16, 33, 1000])
def test_extend_bind_schedule(B):
    """The extend bind's work list: qo_indptr is the prefix sum of the clamped
    new-token counts; req_order lists the requests with work by decreasing
    length (ties by index), then the rest by index; item_indptr is the prefix
    sum, in that order, of n_kv_heads * ceil(n_b * G / 128) items."""
    from paged_kv_decode_10_amd import Config, PagedDecode

    say(f"[extend bind] B={B}")
    rng = np.random.default_rng(500 + B)
    H, Hkv, D, ps, cap = 32, 8, 128, 16, 64 * 16
    L = rng.integers(0, cap + 1, size=B)
    L[rng.random(B) < 0.2] = int(rng.integers(0, cap + 1))  # ties
    n = np.minimum(rng.integers(0, 300, size=B), L)
    n[rng.random(B) < 0.1] = 0  # requests without new tokens
    cfg = Config(n_layers=1, n_heads=H, n_kv_heads=Hkv, head_dim=D, page_size=ps, max_batch=B, max_splits=4,
                 max_pages_per_req=cap // ps, num_slots=B * cap, max_total_tokens=int(L.sum()) + 1)
    ws = PagedDecode(cfg)
    seq = torch.from_numpy(L.astype(np.int32)).cuda()
    ext = torch.from_numpy(n.astype(np.int32)).cuda()
    base = torch.arange(B, dtype=torch.int32, device="cuda") * cap
    ws.bind_extend(B, seq, ext, req_base=base)
    torch.cuda.synchronize()
    assert ws.read_error() == 0
    items = Hkv * -(-(n * (H // Hkv)) // 128)
    want_qo = np.concatenate([[0], np.cumsum(n)])
    order = sorted(range(B), key=lambda b: (0, -int(L[b]), b) if items[b] > 0 else (1, 0, b))
    want_items = np.concatenate([[0], np.cumsum(items[order])])
    assert np.array_equal(ws.qo_indptr[: B + 1].cpu().numpy(), want_qo)
    assert ws.req_order[:B].cpu().numpy().tolist() == order
    assert np.array_equal(ws.item_indptr[: B + 1].cpu().numpy(), want_items)


def test_prefill_store_past_4gib():
    """A layer store larger than 4 GiB takes the 64-bit addressing path: the
    same K/V rows placed past the 4 GiB mark (slot + offset, page table moved
    by the same number of pages) give the oracle's result on the compact
    store.  (Smaller stores use 32-bit byte offsets from a uniform base.)"""
    from paged_kv_decode_10_amd import Config, PagedDecode

    say("[prefill] store past 4 GiB")
    w = workloads.make_custom("pbig", seed=230, n_layers=1, seq_lens=[300, 45, 700], extend_lens=[60, 45, 33],
                              n_heads=8, n_kv_heads=2, head_dim=64, page_size=16)
    row_bytes = w.n_kv_heads * w.head_dim * 2
    off_pages = -(-(1 << 32) // (row_bytes * w.page_size))  # pages whose rows span 4 GiB
    off = off_pages * w.page_size
    slots = off + w.num_slots
    k_big = torch.empty((1, slots, w.n_kv_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    v_big = torch.empty_like(k_big)
    k_big[:, off:] = w.k_store.cuda()
    v_big[:, off:] = w.v_store.cuda()
    cfg = Config(n_layers=1, n_heads=w.n_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                 page_size=w.page_size, max_batch=w.batch, max_splits=8, max_pages_per_req=w.max_pages_per_req,
                 num_slots=slots, max_total_tokens=int(w.seq_lens.sum()))
    ws = PagedDecode(cfg)
    table = (w.req_to_page + off_pages).cuda().contiguous()
    ws.bind_extend(w.batch, w.seq_lens.cuda(), w.meta["extend_lens"].cuda(), req_to_page=table)
    q = w.q[0].cuda()
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    ws.prefill_attn(w.batch, 0, q, k_big, v_big, w.scale, out)
    torch.cuda.synchronize()
    assert ws.read_error() == 0
    ref, _ = _oracle(w)
    assert_close_out(out.float().cpu().numpy(), ref, "prefill past 4 GiB")
    del k_big, v_big
    torch.cuda.empty_cache()
