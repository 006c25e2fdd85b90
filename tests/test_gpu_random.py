"""GPU: seeded random shapes through the whole decode path (bind, split
attention, merge) and through prefill, against the oracle.  Each case draws
its batch, length mix (zeros included), group size, head dim, page size and
split count from a fixed seed."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from paged_kv_decode_10_amd import PD_BIND_FULL
from tests.gpu_harness import assert_close_out, check_bind, check_layer, make_ws, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")


def _draw(seed):
    rng = np.random.default_rng(1000 + seed)
    hkv = int(rng.choice([1, 2, 3, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    D = int(rng.choice([64, 128]))
    ps = int(rng.choice([1, 3, 8, 16, 32, 64]))
    B = int(rng.integers(1, 40))
    kind = rng.integers(0, 3)
    if kind == 0:
        lens = rng.integers(0, 600, size=B)
    elif kind == 1:
        lens = np.where(rng.random(B) < 0.3, 0, rng.integers(1, 3000, size=B))
    else:
        lens = rng.integers(1, 40, size=B)
    lens = [int(x) for x in lens]
    S = int(rng.choice([0, 1, 2, 5, 17, 64, 100]))
    return hkv, G, D, ps, lens, S


@pytest.mark.parametrize("seed", range(12))
def test_random_decode(seed):
    hkv, G, D, ps, lens, S = _draw(seed)
    say(f"[random {seed}] hkv={hkv} G={G} D={D} ps={ps} B={len(lens)} sumL={sum(lens)} S={S}")
    w = workloads.make_custom("rnd", seed=2000 + seed, n_layers=1, seq_lens=lens, n_heads=G * hkv,
                              n_kv_heads=hkv, head_dim=D, page_size=ps)
    dev = to_device(w)
    ws = make_ws(w, max_splits=128)
    ws.bind(w.batch, PD_BIND_FULL, dev.seq_lens, dev.position_ids, dev.req_to_page)
    torch.cuda.synchronize()
    check_bind(ws, w, w.seq_lens.numpy())
    S_ = ws.num_splits(w.batch, S)
    check_layer(ws, w, dev, 0, S_)
    assert ws.read_error() == 0


@pytest.mark.parametrize("seed", range(6))
def test_random_prefill(seed):
    hkv, G, D, ps, lens, _ = _draw(100 + seed)
    lens = [max(1, x) for x in lens][:12]
    rng = np.random.default_rng(3000 + seed)
    ext = [int(rng.integers(0, x + 1)) for x in lens]
    say(f"[random prefill {seed}] hkv={hkv} G={G} D={D} ps={ps} B={len(lens)} new={sum(ext)}")
    w = workloads.make_custom("rndp", seed=4000 + seed, n_layers=1, seq_lens=lens, extend_lens=ext,
                              n_heads=G * hkv, n_kv_heads=hkv, head_dim=D, page_size=ps)
    if sum(ext) == 0:
        pytest.skip("no new tokens drawn")
    dev = to_device(w)
    ws = make_ws(w)
    ws.bind_extend(w.batch, dev.seq_lens, w.meta["extend_lens"].cuda(), req_to_page=dev.req_to_page)
    out = torch.full(dev.q[0].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    ws.prefill_attn(w.batch, 0, dev.q[0], dev.k, dev.v, w.scale, out)
    torch.cuda.synchronize()
    assert ws.read_error() == 0
    L = w.seq_lens.numpy()
    ip, ix = oracle.bind_full(L, w.req_to_page.numpy(), w.page_size)
    ref, _ = oracle.prefill_attention(w.q[0], w.k_store[0], w.v_store[0], L, np.array(ext), ip, ix, w.scale,
                                      w.n_kv_heads)
    assert_close_out(out.float().cpu().numpy(), ref, f"random prefill {seed}")


@pytest.mark.parametrize("B,S", [(100, 0), (100, 7), (1024, 0), (1024, 1), (1024, 3)])
def test_many_requests(B, S):
    """Batches past the 64 requests one wave holds in registers (the plan then
    reads page_indptr / kv_indptr from memory), up to the largest batch the
    bind supports; the oracle is checked on a sample of (request, kv head)
    pairs, the bind in full."""
    rng = np.random.default_rng(B * 10 + S)
    lens = [int(x) for x in np.where(rng.random(B) < 0.1, 0, rng.integers(1, 200 if B > 200 else 900, size=B))]
    say(f"[many] B={B} sumL={sum(lens)} S={S}")
    w = workloads.make_custom("many", seed=3000 + B + S, n_layers=1, seq_lens=lens, n_heads=8, n_kv_heads=2,
                              head_dim=64, page_size=16)
    dev = to_device(w)
    ws = make_ws(w, max_splits=64)
    ws.bind(w.batch, PD_BIND_FULL, dev.seq_lens, dev.position_ids, dev.req_to_page)
    torch.cuda.synchronize()
    check_bind(ws, w, w.seq_lens.numpy())
    S_ = ws.num_splits(w.batch, S)
    picks = sorted({int(x) for x in rng.choice(B, size=min(B, 48), replace=False)} | {0, B - 1})
    pairs = [(b, g) for b in picks for g in range(2)]
    check_layer(ws, w, dev, 0, S_, pairs=pairs)
    assert ws.read_error() == 0
