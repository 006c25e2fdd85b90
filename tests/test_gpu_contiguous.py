"""GPU: the contiguous cache (request b's tokens at slots base_b + t), bound
through paged_decode_bind_contiguous, against the oracle; and bit-identical to
the paged bind of the same layout (consecutive page lists)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from paged_kv_decode_10_amd import PD_BIND_FULL, PD_BIND_STEADY, PD_ERR_BAD_PAGE
from tests.gpu_harness import assert_close_out, make_ws, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")


def _bits(t):
    return t.contiguous().view(torch.int16)


@pytest.mark.parametrize("hkv,D,ps,S", [(8, 128, 16, 0), (2, 64, 16, 5), (4, 128, 7, 1), (1, 64, 32, 9)])
def test_contiguous_matches_oracle_and_paged(hkv, D, ps, S):
    say(f"[contig] hkv={hkv} D={D} ps={ps} S={S}")
    w = workloads.make_custom("contig", seed=60 + hkv + ps, n_layers=1, seq_lens=[700, 0, 1, 2049, 33, 96],
                              n_heads=4 * hkv, n_kv_heads=hkv, head_dim=D, page_size=ps, layout="contiguous",
                              growth=4)
    dev = to_device(w)
    base = w.meta["req_base"].cuda()
    B = w.batch
    outs, idx = [], []
    for contiguous in (True, False):
        ws = make_ws(w)
        S_ = ws.num_splits(B, S)
        if contiguous:
            ws.bind_contiguous(B, PD_BIND_FULL, dev.seq_lens, dev.position_ids, base)
        else:
            ws.bind(B, PD_BIND_FULL, dev.seq_lens, dev.position_ids, dev.req_to_page)
        out = torch.empty((B, w.n_heads, D), dtype=torch.bfloat16, device="cuda")
        ws.attn(B, 0, S_, dev.q[0], dev.k, dev.v, w.scale)
        ws.merge(B, S_, out)
        torch.cuda.synchronize()
        assert ws.read_error() == 0
        n = int(w.seq_lens.sum())
        idx.append(ws.kv_indices[:n].cpu().numpy())
        outs.append(out.cpu())
    L = w.seq_lens.numpy()
    ref_idx = oracle.kv_indices_contiguous(L, w.meta["req_base"].numpy())
    assert np.array_equal(idx[0], ref_idx), "kv_indices (contiguous)"
    assert np.array_equal(idx[1], ref_idx), "kv_indices (paged, consecutive pages)"
    assert torch.equal(_bits(outs[0]), _bits(outs[1])), "contiguous and paged binds must agree bit for bit"
    ip = oracle.kv_indptr(L)
    ref, _ = oracle.decode_attention(w.q[0], w.k_store[0], w.v_store[0], L, ip, ref_idx, w.scale, w.n_kv_heads)
    assert_close_out(outs[0].float().numpy(), ref, "contiguous decode_out")


def test_contiguous_steady_and_bad_base():
    say("[contig] steady + bad base")
    w = workloads.make_custom("contig2", seed=70, n_layers=1, seq_lens=[10, 200, 3], n_heads=8, n_kv_heads=2,
                              head_dim=128, page_size=16, layout="contiguous", growth=8)
    dev = to_device(w)
    base = w.meta["req_base"].cuda()
    B = w.batch
    ws = make_ws(w)
    ws.bind_contiguous(B, PD_BIND_FULL, dev.seq_lens, dev.position_ids, base)
    ws.bind_contiguous(B, PD_BIND_STEADY, dev.seq_lens, dev.position_ids, base)
    torch.cuda.synchronize()
    L = w.seq_lens.numpy() + 1
    assert dev.seq_lens.cpu().numpy().tolist() == L.tolist()
    n = int(L.sum())
    assert np.array_equal(ws.kv_indices[:n].cpu().numpy(),
                          oracle.kv_indices_contiguous(L, w.meta["req_base"].numpy()))
    assert ws.read_error() == 0
    # a base past the store: flagged, and every index stays inside the store
    bad = base.clone()
    bad[1] = w.num_slots - 5
    ws.bind_contiguous(B, PD_BIND_FULL, dev.seq_lens, dev.position_ids, bad)
    torch.cuda.synchronize()
    assert ws.read_error() & PD_ERR_BAD_PAGE
    got = ws.kv_indices[:n].cpu().numpy()
    assert got.min() >= 0 and got.max() < w.num_slots
