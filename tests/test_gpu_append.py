"""GPU: per-layer KV append (the new token's K/V rows written at its slot),
through the C ABI, against the oracle; bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from paged_kv_decode_10_amd import PD_BIND_FULL, PD_BIND_STEADY
from tests.gpu_harness import assert_close_out, make_ws, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")


def _new_rows(w, seed):
    g = torch.Generator().manual_seed(seed)
    shape = (w.n_layers, w.batch, w.n_kv_heads, w.head_dim)
    return (torch.randn(shape, generator=g).to(torch.bfloat16),
            torch.randn(shape, generator=g).to(torch.bfloat16))


def _bits(t):
    return t.contiguous().view(torch.int16)


@pytest.mark.parametrize("hkv,D,ps", [(4, 128, 16), (2, 64, 7), (8, 128, 1)])
def test_append_matches_oracle(hkv, D, ps):
    say(f"[append] hkv={hkv} D={D} ps={ps}")
    w = workloads.make_custom("app", seed=40 + hkv + ps, n_layers=2, seq_lens=[5, 0, 130, 17, 1, 64],
                              n_heads=2 * hkv, n_kv_heads=hkv, head_dim=D, page_size=ps)
    dev = to_device(w)
    ws = make_ws(w)
    kn, vn = _new_rows(w, 1)
    ws.bind(w.batch, PD_BIND_FULL, dev.seq_lens, dev.position_ids, dev.req_to_page)
    ws.append_kv(w.batch, 1, kn[1].cuda(), vn[1].cuda(), dev.k, dev.v)
    torch.cuda.synchronize()
    slots = oracle.append_slots(w.seq_lens.numpy(), w.req_to_page.numpy(), w.page_size)
    assert slots[1] == -1
    k_ref = oracle.append_kv(w.k_store[1], kn[1], slots)
    v_ref = oracle.append_kv(w.v_store[1], vn[1], slots)
    got_k, got_v = dev.k.cpu(), dev.v.cpu()
    assert torch.equal(_bits(got_k[1]), _bits(k_ref)), "K layer 1"
    assert torch.equal(_bits(got_v[1]), _bits(v_ref)), "V layer 1"
    assert torch.equal(_bits(got_k[0]), _bits(w.k_store[0])), "layer 0 must not change"
    assert torch.equal(_bits(got_v[0]), _bits(w.v_store[0]))


def _oracle_step(w, k_store, v_store, L, kn, vn, layer):
    """Stores after the append of layer `layer` at lengths L, and the attention."""
    table = w.req_to_page.numpy()
    slots = oracle.append_slots(L, table, w.page_size)
    k_l = oracle.append_kv(k_store[layer], kn[layer], slots)
    v_l = oracle.append_kv(v_store[layer], vn[layer], slots)
    ip, ix = oracle.bind_full(L, table, w.page_size)
    out, _ = oracle.decode_attention(w.q[layer], k_l, v_l, L, ip, ix, w.scale, w.n_kv_heads)
    return k_l, v_l, out


def test_steady_step_with_append():
    """bind steady (+1), then per layer: append the new token, attend, merge."""
    say("[append] steady step")
    w = workloads.make_custom("appstep", seed=44, n_layers=3, seq_lens=[300, 1, 0, 47, 1029],
                              n_heads=16, n_kv_heads=4, head_dim=128, page_size=16, growth=8)
    dev = to_device(w)
    ws = make_ws(w)
    B = w.batch
    S = ws.num_splits(B)
    kn, vn = _new_rows(w, 2)
    kn_d, vn_d = kn.cuda(), vn.cuda()
    out = torch.empty((w.n_layers, B, w.n_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    ws.bind(B, PD_BIND_FULL, dev.seq_lens, dev.position_ids, dev.req_to_page)
    ws.bind(B, PD_BIND_STEADY, dev.seq_lens, dev.position_ids, dev.req_to_page)
    for layer in range(w.n_layers):
        ws.append_kv(B, layer, kn_d[layer], vn_d[layer], dev.k, dev.v)
        ws.attn(B, layer, S, dev.q[layer], dev.k, dev.v, w.scale)
        ws.merge(B, S, out[layer])
    torch.cuda.synchronize()
    L = w.seq_lens.numpy() + 1
    assert dev.seq_lens.cpu().numpy().tolist() == L.tolist()
    got = out.float().cpu().numpy()
    got_k, got_v = dev.k.cpu(), dev.v.cpu()
    for layer in range(w.n_layers):
        k_l, v_l, ref = _oracle_step(w, w.k_store, w.v_store, L, kn, vn, layer)
        assert torch.equal(_bits(got_k[layer]), _bits(k_l)) and torch.equal(_bits(got_v[layer]), _bits(v_l))
        assert_close_out(got[layer], ref, f"decode_out layer {layer}")
    # the request that was empty now holds exactly its new token: out = its V row
    G = w.group
    for h in range(w.n_heads):
        assert torch.equal(_bits(out[0, 2, h].cpu()), _bits(vn[0, 2, h // G])), h


def test_graph_step_with_append_matches_eager():
    say("[append] graph")
    w = workloads.make_custom("appgraph", seed=45, n_layers=2,
                              seq_lens=lambda g: torch.randint(1, 400, (6,), generator=g).tolist(),
                              n_heads=32, n_kv_heads=8, head_dim=128, page_size=16, growth=8)
    B = w.batch
    kn, vn = _new_rows(w, 3)

    def run(graph):
        dev = to_device(w)
        ws = make_ws(w)
        S = ws.num_splits(B)
        kn_d, vn_d = kn.cuda(), vn.cuda()
        out = torch.empty((w.n_layers, B, w.n_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
        ws.bind(B, PD_BIND_FULL, dev.seq_lens, dev.position_ids, dev.req_to_page)

        def step():
            ws.bind(B, PD_BIND_STEADY, dev.seq_lens, dev.position_ids, dev.req_to_page)
            for layer in range(w.n_layers):
                ws.append_kv(B, layer, kn_d[layer], vn_d[layer], dev.k, dev.v)
                ws.attn(B, layer, S, dev.q[layer], dev.k, dev.v, w.scale)
                ws.merge(B, S, out[layer])

        outs = []
        if graph:
            step()  # live run
            torch.cuda.synchronize()
            outs.append(out.clone())
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step()
            for i in range(3):
                kn_d.add_(1.0 / 64)  # next token's rows, written into the captured buffers
                vn_d.sub_(1.0 / 64)
                g.replay()
                torch.cuda.synchronize()
                outs.append(out.clone())
        else:
            for i in range(4):
                if i:
                    kn_d.add_(1.0 / 64)
                    vn_d.sub_(1.0 / 64)
                step()
                torch.cuda.synchronize()
                outs.append(out.clone())
        return outs, dev.k.cpu(), dev.v.cpu()

    eager, ke, ve = run(False)
    graph, kg, vg = run(True)
    for i, (a, b) in enumerate(zip(eager, graph)):
        assert torch.equal(_bits(a), _bits(b)), f"step {i}"
    assert torch.equal(_bits(ke), _bits(kg)) and torch.equal(_bits(ve), _bits(vg))


@pytest.mark.parametrize("hkv,D,ps,S", [(4, 128, 16, 0), (2, 64, 7, 5), (8, 128, 1, 17), (4, 128, 32, 3),
                                        (1, 64, 32, 1), (8, 128, 16, 64)])
def test_fused_append_attn_bit_identical(hkv, D, ps, S):
    """append_attn == append_kv + attn: stores, partial statistics and decode_out, bit for bit."""
    say(f"[append fused] hkv={hkv} D={D} ps={ps} S={S}")
    w = workloads.make_custom("appf", seed=50 + hkv + ps + S, n_layers=2,
                              seq_lens=[5, 0, 130, 17, 1, 64, 47, 33, 16, 32],
                              n_heads=4 * hkv, n_kv_heads=hkv, head_dim=D, page_size=ps, growth=2,
                              nan_growth=True)
    B = w.batch
    kn, vn = _new_rows(w, 5)
    results = []
    for fused in (False, True):
        dev = to_device(w)
        ws = make_ws(w)
        S_ = ws.num_splits(B, S)
        out = torch.empty((B, w.n_heads, D), dtype=torch.bfloat16, device="cuda")
        ws.bind(B, PD_BIND_FULL, dev.seq_lens, dev.position_ids, dev.req_to_page)
        ws.bind(B, PD_BIND_STEADY, dev.seq_lens, dev.position_ids, dev.req_to_page)
        layer = 1
        if fused:
            ws.append_attn(B, layer, S_, dev.q[layer], kn[layer].cuda(), vn[layer].cuda(), dev.k, dev.v, w.scale)
        else:
            ws.append_kv(B, layer, kn[layer].cuda(), vn[layer].cuda(), dev.k, dev.v)
            ws.attn(B, layer, S_, dev.q[layer], dev.k, dev.v, w.scale)
        ws.merge(B, S_, out)
        torch.cuda.synchronize()
        results.append((out.cpu(), ws.ml_part[:B, :, :S_].cpu(), dev.k.cpu(), dev.v.cpu()))
    (o0, m0, k0, v0), (o1, m1, k1, v1) = results
    assert torch.equal(_bits(k0), _bits(k1)) and torch.equal(_bits(v0), _bits(v1)), "stores differ"
    assert torch.equal(m0.view(torch.int32), m1.view(torch.int32)), "partial statistics differ"
    assert torch.equal(_bits(o0), _bits(o1)), "decode_out differs"
    assert torch.isfinite(o1.float()).all(), "stale NaN slot leaked into decode_out"
    L = w.seq_lens.numpy() + 1
    _, _, ref = _oracle_step(w, w.k_store, w.v_store, L, kn, vn, 1)
    assert_close_out(o1.float().numpy(), ref, "fused decode_out")


def test_fused_graph_step_matches_eager():
    say("[append fused] graph")
    w = workloads.make_custom("appfg", seed=46, n_layers=3,
                              seq_lens=lambda g: torch.randint(0, 500, (9,), generator=g).tolist(),
                              n_heads=32, n_kv_heads=8, head_dim=128, page_size=16, growth=8, nan_growth=True)
    B = w.batch
    kn, vn = _new_rows(w, 6)

    def run(fused, graph):
        dev = to_device(w)
        ws = make_ws(w)
        S = ws.num_splits(B)
        kn_d, vn_d = kn.cuda(), vn.cuda()
        out = torch.empty((w.n_layers, B, w.n_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
        ws.bind(B, PD_BIND_FULL, dev.seq_lens, dev.position_ids, dev.req_to_page)

        def step():
            ws.bind(B, PD_BIND_STEADY, dev.seq_lens, dev.position_ids, dev.req_to_page)
            for layer in range(w.n_layers):
                if fused:
                    ws.append_attn(B, layer, S, dev.q[layer], kn_d[layer], vn_d[layer], dev.k, dev.v, w.scale)
                else:
                    ws.append_kv(B, layer, kn_d[layer], vn_d[layer], dev.k, dev.v)
                    ws.attn(B, layer, S, dev.q[layer], dev.k, dev.v, w.scale)
                ws.merge(B, S, out[layer])

        outs = []
        step()
        torch.cuda.synchronize()
        outs.append(out.clone())
        if graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step()
        for i in range(3):
            kn_d.add_(1.0 / 64)
            vn_d.sub_(1.0 / 64)
            if graph:
                g.replay()
            else:
                step()
            torch.cuda.synchronize()
            outs.append(out.clone())
        return outs, dev.k.cpu(), dev.v.cpu()

    ref, kr, vr = run(False, False)
    assert all(torch.isfinite(o.float()).all() for o in ref)
    for fused, graph in ((True, False), (True, True)):
        got, kg, vg = run(fused, graph)
        for i, (a, b) in enumerate(zip(ref, got)):
            assert torch.equal(_bits(a), _bits(b)), f"fused={fused} graph={graph} step {i}"
        assert torch.equal(_bits(kr), _bits(kg)) and torch.equal(_bits(vr), _bits(vg))


@pytest.mark.parametrize("ps", [1, 7, 16, 32])
def test_fused_append_over_stale_nan_slots(ps):
    """The slots past every request's length hold NaN (a freshly handed-out
    page): the fused append must read the newest token only from the new-row
    buffer, in every lane that resolves to it, and match the oracle."""
    say(f"[append fused] stale NaN slots ps={ps}")
    w = workloads.make_custom("appnan", seed=60 + ps, n_layers=1,
                              seq_lens=[0, 1, ps - 1 if ps > 1 else 2, ps, ps + 1, 2 * ps - 1, 31, 33, 100],
                              n_heads=16, n_kv_heads=4, head_dim=128, page_size=ps, growth=3, nan_growth=True)
    B = w.batch
    kn, vn = _new_rows(w, 7)
    dev = to_device(w)
    ws = make_ws(w)
    out = torch.empty((B, w.n_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    L = w.seq_lens.numpy().astype(np.int64)
    k_host, v_host = w.k_store[0].clone(), w.v_store[0].clone()
    ws.bind(B, PD_BIND_FULL, dev.seq_lens, dev.position_ids, dev.req_to_page)
    for step in range(3):
        ws.bind(B, PD_BIND_STEADY, dev.seq_lens, dev.position_ids, dev.req_to_page)
        L = L + 1
        for S in (1, 3, ws.num_splits(B)):
            ws.append_attn(B, 0, S, dev.q[0], kn[0].cuda(), vn[0].cuda(), dev.k, dev.v, w.scale)
            ws.merge(B, S, out)
            torch.cuda.synchronize()
            got = out.float().cpu().numpy()
            assert np.isfinite(got).all(), f"step {step} S={S}: NaN from a stale slot"
        slots = oracle.append_slots(L, w.req_to_page.numpy(), w.page_size)
        k_host = oracle.append_kv(k_host, kn[0], slots)
        v_host = oracle.append_kv(v_host, vn[0], slots)
        assert torch.equal(_bits(dev.k[0].cpu()), _bits(k_host)) and torch.equal(_bits(dev.v[0].cpu()), _bits(v_host))
        ip, ix = oracle.bind_full(L, w.req_to_page.numpy(), w.page_size)
        ref, _ = oracle.decode_attention(w.q[0], k_host, v_host, L, ip, ix, w.scale, w.n_kv_heads)
        assert_close_out(got, ref, f"fused decode_out over NaN slots, step {step}")
    assert ws.read_error() == 0
