"""GPU: paged_decode_attn_merge_noalloc, the variant of attn + merge whose
split partials live in the library's static scratch array, through the C ABI.

Its decode_out must equal that of paged_decode_attn + paged_decode_merge bit
for bit (same kernels, same partials), on two calls in a row where the second
has a smaller input (the array keeps the first call's contents), with no
device allocation during the calls; both also match the oracle.  A request
whose partials do not fit the array is rejected on the host.  Captured in a
graph (the callers it is for), every replay equals attn + merge on the same
inputs, bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from paged_kv_decode_10_amd import PD_BIND_FULL, PD_E_SCRATCH, Config, PagedDecode, PagedDecodeError
from tests.gpu_harness import assert_close_out, make_ws, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")


def _bits(t):
    return t.contiguous().view(torch.int16)


def _one(w, layer, S_req):
    dev = to_device(w)
    ws = make_ws(w, max_splits=256)
    B = w.batch
    S = ws.num_splits(B, S_req)
    ws.bind(B, PD_BIND_FULL, dev.seq_lens, dev.position_ids, dev.req_to_page)
    ref = torch.full((B, w.n_heads, w.head_dim), 3.0, dtype=torch.bfloat16, device="cuda")
    got = torch.full_like(ref, -5.0)
    ws.attn(B, layer, S, dev.q[layer], dev.k, dev.v, w.scale)
    ws.merge(B, S, ref)
    torch.cuda.synchronize()
    arena_ml = ws.ml_part.clone()
    a0 = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    ws.attn_merge_noalloc(B, layer, S, dev.q[layer], dev.k, dev.v, w.scale, got)
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats().get("allocation.all.allocated", 0) == a0, "the call allocated"
    assert torch.equal(ws.ml_part.view(torch.int32), arena_ml.view(torch.int32)), "arena partials touched"
    return ws, dev, S, ref, got


@pytest.mark.parametrize("order", ["large_then_small", "small_then_large_then_small"])
def test_noalloc_matches_attn_merge(order):
    big = ("b16", 0, 0)
    small = ("tiny", 0, 4)
    seq = [big, small] if order == "large_then_small" else [small, big, ("tiny", 0, 65)]
    for name, layer, S_req in seq:
        w = workloads.make(name)
        ws, dev, S, ref, got = _one(w, layer, S_req)
        say(f"[noalloc] {name} B={w.batch} S={S}")
        assert torch.equal(_bits(got), _bits(ref)), f"{name}: noalloc output differs from attn + merge"
        L = w.seq_lens.numpy()
        ip, ix = oracle.bind_full(L, w.req_to_page.numpy(), w.page_size)
        want, _ = oracle.decode_attention(w.q[layer], w.k_store[layer], w.v_store[layer], L, ip, ix, w.scale,
                                          w.n_kv_heads)
        assert_close_out(got.double().cpu().numpy(), want, f"{name} noalloc decode_out")
        assert ws.read_error() == 0


def test_noalloc_rejects_oversize_on_host():
    """4 requests x 64 heads x 256 splits x 130 fp32 = 34 MB > 32 MiB: rejected before any launch."""
    cfg = Config(n_layers=1, n_heads=64, n_kv_heads=8, head_dim=128, page_size=16, max_batch=4, max_splits=256,
                 max_pages_per_req=4, num_slots=64, max_total_tokens=64)
    ws = PagedDecode(cfg)
    q = torch.zeros((4, 64, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 64, 8, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros_like(q)
    with pytest.raises(PagedDecodeError) as e:
        ws.attn_merge_noalloc(4, 0, 256, q, kv, kv, 0.1, out)
    assert e.value.status == PD_E_SCRATCH
    assert torch.all(out == 0)
    # 3 requests fit (25.6 MB)
    assert np.ceil(3 * 64 * 256 * 128 * 4 / 256) * 256 + 3 * 64 * 256 * 8 <= 32 << 20


def test_noalloc_under_graph_capture():
    w = workloads.make_custom("nag", seed=91, n_layers=2,
                              seq_lens=lambda g: torch.randint(1, 900, (7,), generator=g).tolist(),
                              n_heads=32, n_kv_heads=8, head_dim=128, page_size=16)
    dev = to_device(w)
    ws = make_ws(w, max_splits=64)
    B = w.batch
    S = ws.num_splits(B)
    say(f"[noalloc graph] B={B} S={S}")
    ws.bind(B, PD_BIND_FULL, dev.seq_lens, dev.position_ids, dev.req_to_page)
    q = dev.q[1].clone()
    out = torch.empty((B, w.n_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    ref = torch.empty_like(out)
    ws.attn_merge_noalloc(B, 1, S, q, dev.k, dev.v, w.scale, out)  # live run before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ws.attn_merge_noalloc(B, 1, S, q, dev.k, dev.v, w.scale, out)
    gen = torch.Generator().manual_seed(5)
    for i in range(4):
        q.copy_(torch.randn(q.shape, generator=gen).to(torch.bfloat16).cuda())  # next step's queries
        a0 = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.cuda.memory_stats().get("allocation.all.allocated", 0) == a0
        ws.attn(B, 1, S, q, dev.k, dev.v, w.scale)
        ws.merge(B, S, ref)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref)), f"replay {i}"
        _ = float(out.float().abs().sum())  # eager work between replays
    assert ws.read_error() == 0
