"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: brute-force
enumeration, hand-derived examples, closed forms, torch's float64 scaled dot
product attention over a dense layout built without the oracle's gather, and
invariances the definition implies.  They are chosen so that a plausible slip
(wrong kv-head map, dropped max shift, transposed operand, off-by-one page
index, wrong merge weight) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.plan_params import PLAN_TEAM_MAX, PLAN_WAVES, plan_args

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- bind ----

def _brute_indptr(seq_lens):
    out = []
    for b in range(len(seq_lens) + 1):
        n = 0
        for bb in range(b):
            for _t in range(int(seq_lens[bb])):
                n += 1
        out.append(n)
    return out


def _brute_indices(seq_lens, req_to_page, ps, num_slots):
    """Scan every pool slot; keep the ones a request owns, ordered by token."""
    res = []
    for b, L in enumerate(seq_lens):
        owned = {}
        row = list(req_to_page[b])
        for s in range(num_slots):
            page, off = divmod(s, ps)
            if page in row:
                t = row.index(page) * ps + off
                if t < L:
                    owned[t] = s
        res.extend(owned[t] for t in range(int(L)))
    return res


def test_bind_golden():
    g = _load("bind_example.json")
    ip, ix = oracle.bind_full(g["seq_lens"], np.array(g["req_to_page"]), g["page_size"])
    assert ip.tolist() == g["kv_indptr"]
    assert ix.tolist() == g["kv_indices"]
    sl, pos = oracle.bind_steady(g["seq_lens"], g["position_ids"])
    assert sl.tolist() == g["steady"]["seq_lens"]
    assert pos.tolist() == g["steady"]["position_ids"]
    ip2, ix2 = oracle.bind_full(sl, np.array(g["req_to_page"]), g["page_size"])
    assert ip2.tolist() == g["steady"]["kv_indptr"]
    assert ix2.tolist() == g["steady"]["kv_indices"]
    assert oracle.append_slots(g["seq_lens"], np.array(g["req_to_page"]), g["page_size"]).tolist() == \
        g["append_slots"]
    assert oracle.append_slots(sl, np.array(g["req_to_page"]), g["page_size"]).tolist() == \
        g["steady"]["append_slots"]


def test_contiguous_bind_golden():
    g = _load("contiguous_example.json")
    assert oracle.kv_indptr(g["seq_lens"]).tolist() == g["kv_indptr"]
    assert oracle.kv_indices_contiguous(g["seq_lens"], g["req_base"]).tolist() == g["kv_indices"]


@pytest.mark.parametrize("ps", [1, 4, 16])
def test_contiguous_equals_paged_with_consecutive_pages(ps):
    """A contiguous buffer that starts on a page boundary is the paged cache
    whose page list is consecutive pages."""
    rng = np.random.default_rng(ps)
    lens = [int(x) for x in rng.integers(0, 60, size=5)]
    width = max(-(-x // ps) for x in lens) + 1
    first_page = rng.permutation(5) * width
    base = first_page * ps
    table = first_page[:, None] + np.arange(width)[None, :]
    assert oracle.kv_indices_contiguous(lens, base).tolist() == oracle.kv_indices(lens, table, ps).tolist()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_append_slots_brute_force(seed):
    """The newest token's slot, found another way: walk the request's pages in
    order, listing their slots, and take entry L_b - 1."""
    rng = np.random.default_rng(100 + seed)
    ps = int(rng.choice([1, 3, 16]))
    lens = [int(x) for x in rng.integers(0, 50, size=int(rng.integers(1, 7)))]
    lens[0] = 0
    pages = [-(-x // ps) for x in lens]
    perm = rng.permutation(sum(pages) + 3)
    width = max(pages + [1])
    table = np.full((len(lens), width), -1, dtype=np.int64)
    off = 0
    for b, p in enumerate(pages):
        table[b, :p] = perm[off:off + p]
        off += p
    got = oracle.append_slots(lens, table, ps)
    for b, lb in enumerate(lens):
        listed = [int(pg) * ps + o for pg in table[b, :pages[b]] for o in range(ps)]
        assert got[b] == (listed[lb - 1] if lb else -1)


def test_append_kv_writes_only_the_new_rows():
    g = torch.Generator().manual_seed(7)
    store = torch.randn((40, 3, 8), generator=g).to(torch.bfloat16)
    new = torch.randn((4, 3, 8), generator=g).to(torch.bfloat16)
    slots = np.array([5, -1, 39, 0])
    out = oracle.append_kv(store, new, slots)
    assert store.shape == out.shape and out.data_ptr() != store.data_ptr()
    for b, s in enumerate(slots):
        if s >= 0:
            assert torch.equal(out[s].view(torch.int16), new[b].view(torch.int16))
    keep = [i for i in range(40) if i not in (5, 39, 0)]
    assert torch.equal(out[keep].view(torch.int16), store[keep].view(torch.int16))


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_bind_brute_force(seed):
    rng = np.random.default_rng(seed)
    ps = int(rng.choice([1, 4, 16]))
    B = int(rng.integers(1, 6))
    lens = rng.integers(0, 40, size=B)
    pages = [-(-int(x) // ps) for x in lens]
    num_pages = sum(pages) + 5
    perm = rng.permutation(num_pages)
    table = -np.ones((B, max(pages + [1])), dtype=np.int64)
    off = 0
    for b, p in enumerate(pages):
        table[b, :p] = perm[off:off + p]
        off += p
    ip = oracle.kv_indptr(lens)
    assert ip.tolist() == _brute_indptr(lens)
    ix = oracle.kv_indices(lens, table, ps)
    assert ix.tolist() == _brute_indices(lens, table, ps, num_pages * ps)
    # invariants: segment lengths, distinct slots, in-page offsets
    assert len(ix) == ip[-1]
    assert len(set(ix.tolist())) == len(ix)
    for b in range(B):
        seg = ix[ip[b]:ip[b + 1]]
        assert len(seg) == lens[b]
        assert all(int(s) % ps == t % ps for t, s in enumerate(seg))


def test_bind_tiny_workload_invariants():
    w = workloads.make("tiny")
    ip, ix = oracle.bind_full(w.seq_lens.numpy(), w.req_to_page.numpy(), w.page_size)
    assert ip.tolist() == [0, 37, 137]
    assert ix.tolist() == _brute_indices(w.seq_lens.tolist(), w.req_to_page.tolist(),
                                         w.page_size, w.num_slots)
    # every gathered row is a real (non-NaN) row of the store
    assert not torch.isnan(w.k_store[0, torch.from_numpy(ix)]).any()


# ------------------------------------------------------------ attention ----

def test_attention_golden_examples():
    ex = _load("attention_examples.json")["examples"]
    env = {"e": math.e, "log": math.log}
    for e in ex:
        K = np.array(e["K"], dtype=np.float64)
        V = np.array(e["V"], dtype=np.float64)
        out, m, lnz = oracle.attention_rows(np.array(e["q"]), K, V, e["scale"])
        want = [eval(x, env) for x in e["out_expr"]]  # noqa: S307 - fixture expressions
        np.testing.assert_allclose(out, want, rtol=0, atol=1e-14, err_msg=e["name"])
        assert abs((m + lnz) - eval(e["lse_expr"], env)) < 1e-14, e["name"]


def _scatter_into_pages(dense_k, dense_v, ps, rng, extra_pages=3):
    """Lay dense per-request K/V [L, Hkv, D] into a shuffled paged store."""
    lens = [k.shape[0] for k in dense_k]
    hkv, d = dense_k[0].shape[1:]
    pages = [-(-L // ps) for L in lens]
    num_pages = sum(pages) + extra_pages
    perm = rng.permutation(num_pages)
    table = -np.ones((len(lens), max(pages)), dtype=np.int64)
    k_store = np.full((num_pages * ps, hkv, d), np.nan)
    v_store = np.full((num_pages * ps, hkv, d), np.nan)
    off = 0
    for b, (kb, vb) in enumerate(zip(dense_k, dense_v)):
        table[b, :pages[b]] = perm[off:off + pages[b]]
        off += pages[b]
        for t in range(lens[b]):
            slot = table[b, t // ps] * ps + t % ps
            k_store[slot] = kb[t]
            v_store[slot] = vb[t]
    return table, k_store, v_store


@pytest.mark.parametrize("G,hkv,D,ps", [(1, 2, 64, 16), (2, 2, 64, 16), (4, 2, 128, 16),
                                        (8, 1, 128, 8), (3, 2, 32, 4)])
def test_attention_matches_torch_sdpa_dense(G, hkv, D, ps):
    rng = np.random.default_rng(G * 100 + D)
    lens = [1, 17, 50]
    H = G * hkv
    bf = lambda a: torch.tensor(a, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    dense_k = [bf(rng.standard_normal((L, hkv, D))) for L in lens]
    dense_v = [bf(rng.standard_normal((L, hkv, D))) for L in lens]
    q = bf(rng.standard_normal((len(lens), H, D)))
    scale = float(np.float32(1 / math.sqrt(D)))
    table, ks, vs = _scatter_into_pages(dense_k, dense_v, ps, rng)
    ip, ix = oracle.bind_full(lens, table, ps)
    out, lse = oracle.decode_attention(q, ks, vs, lens, ip, ix, scale, hkv)
    for b, L in enumerate(lens):
        kq = torch.from_numpy(dense_k[b]).permute(1, 0, 2).repeat_interleave(G, dim=0)  # [H, L, D]
        vq = torch.from_numpy(dense_v[b]).permute(1, 0, 2).repeat_interleave(G, dim=0)
        qb = torch.from_numpy(q[b]).unsqueeze(1)  # [H, 1, D]
        ref = torch.nn.functional.scaled_dot_product_attention(qb, kq, vq, scale=scale)
        np.testing.assert_allclose(out[b], ref[:, 0].numpy(), rtol=0, atol=1e-12)
        # lse against the log-sum-exp of the dense scores
        s = scale * torch.einsum("hld,hd->hl", kq, torch.from_numpy(q[b]))
        np.testing.assert_allclose(lse[b], torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_large_scores_stay_finite():
    """Scores near 1e3 overflow exp() unless the max is subtracted first."""
    K = np.array([[30.0, 0.0], [29.0, 0.0], [0.0, 1.0]])
    V = np.array([[1.0, 0.0], [0.0, 1.0], [5.0, 5.0]])
    out, m, lnz = oracle.attention_rows(np.array([40.0, 0.0]), K, V, 1.0)
    w1 = 1.0 / (1.0 + math.exp(-40.0) + math.exp(-1200.0))
    np.testing.assert_allclose(out, [w1, 1 - w1], atol=1e-15)
    assert m == 1200.0 and abs(lnz - math.log1p(math.exp(-40.0))) < 1e-15


def test_closed_forms():
    rng = np.random.default_rng(7)
    D, L = 16, 9
    q = rng.standard_normal(D)
    V = rng.standard_normal((L, D))
    # single token: out = v, lse = score
    k1 = rng.standard_normal((1, D))
    out, m, lnz = oracle.attention_rows(q, k1, V[:1], 0.5)
    assert np.array_equal(out, V[0]) and abs(m + lnz - 0.5 * float(k1[0] @ q)) < 1e-15
    # all keys equal: out = mean(V), lse = s + ln L
    kc = np.repeat(k1, L, axis=0)
    out, m, lnz = oracle.attention_rows(q, kc, V, 0.5)
    np.testing.assert_allclose(out, V.mean(axis=0), atol=1e-14)
    assert abs(m + lnz - (0.5 * float(k1[0] @ q) + math.log(L))) < 1e-13
    # all values equal c: out = c
    Vc = np.full((L, D), -2.25)
    out, _, _ = oracle.attention_rows(q, rng.standard_normal((L, D)), Vc, 0.7)
    np.testing.assert_allclose(out, Vc[0], atol=1e-14)
    # scale 0: out = mean(V), lse = ln L
    out, m, lnz = oracle.attention_rows(q, rng.standard_normal((L, D)), V, 0.0)
    np.testing.assert_allclose(out, V.mean(axis=0), atol=1e-14)
    assert abs(m + lnz - math.log(L)) < 1e-14
    # empty
    out, m, lnz = oracle.attention_rows(q, np.zeros((0, D)), np.zeros((0, D)), 1.0)
    assert np.all(out == 0) and m == -math.inf


def test_gqa_head_map():
    """Query head h must read kv head h // G: give each kv head a distinct V."""
    hkv, G, D, L, ps = 3, 2, 8, 5, 4
    K = np.zeros((L, hkv, D))
    V = np.zeros((L, hkv, D))
    for g in range(hkv):
        V[:, g, :] = g + 1
    table, ks, vs = _scatter_into_pages([K], [V], ps, np.random.default_rng(0))
    ip, ix = oracle.bind_full([L], table, ps)
    out, _ = oracle.decode_attention(np.ones((1, hkv * G, D)), ks, vs, [L], ip, ix, 1.0, hkv)
    for h in range(hkv * G):
        assert np.all(out[0, h] == h // G + 1)


def test_page_permutation_invariance_bit_exact():
    """Relaying the same logical cache through other pages changes nothing."""
    w = workloads.make("tiny")
    L = w.seq_lens.numpy()
    ip, ix = oracle.bind_full(L, w.req_to_page.numpy(), w.page_size)
    out1, lse1 = oracle.decode_attention(w.q[0], w.k_store[0], w.v_store[0], L, ip, ix, w.scale, w.n_kv_heads)
    rng = np.random.default_rng(11)
    perm = rng.permutation(w.num_pages)
    table2 = w.req_to_page.numpy().copy()
    used = table2 >= 0
    table2[used] = perm[: used.sum()]
    k2 = torch.full_like(w.k_store[0], float("nan"))
    v2 = torch.full_like(w.v_store[0], float("nan"))
    ix2 = oracle.kv_indices(L, table2, w.page_size)
    k2[torch.from_numpy(ix2)] = w.k_store[0, torch.from_numpy(ix)]
    v2[torch.from_numpy(ix2)] = w.v_store[0, torch.from_numpy(ix)]
    out2, lse2 = oracle.decode_attention(w.q[0], k2, v2, L, ip, ix2, w.scale, w.n_kv_heads)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


# --------------------------------------------------------------- splits ----

@pytest.mark.parametrize("name", ["split_example.json", "split_example_team2.json"])
def test_split_plan_golden(name):
    g = _load(name)
    for S, want in g["plans"].items():
        plan = oracle.split_plan(g["seq_lens"], g["page_size"], g["n_kv_heads"], int(S), n_chunks=g["n_chunks"],
                                 team=g["team"])
        got = [[[list(r) for r in plan[b][h]] for h in range(g["n_kv_heads"])] for b in range(2)]
        assert got == want, S
    if plan_args(g["n_kv_heads"]) == {"n_chunks": g["n_chunks"], "team": g["team"]}:
        # this example is the launch's own plan (the header's constants)
        for S, want in g["plans"].items():
            plan = oracle.split_plan(g["seq_lens"], g["page_size"], g["n_kv_heads"], int(S),
                                     **plan_args(g["n_kv_heads"]))
            assert [[[list(r) for r in plan[b][h]] for h in range(2)] for b in range(2)] == want


def test_plan_constants_from_header():
    """The bundle size is gcd(n_kv_heads, PD_PLAN_TEAM_MAX) and the chunk count PD_PLAN_WAVES / T."""
    assert (PLAN_WAVES, PLAN_TEAM_MAX) == (2048, 4)
    assert [plan_args(h)["team"] for h in (1, 2, 3, 4, 6, 8, 12, 16, 5)] == [1, 2, 1, 4, 2, 4, 4, 4, 1]
    assert [plan_args(h)["n_chunks"] for h in (1, 2, 8)] == [2048, 1024, 512]


def _brute_plan(L, ps, hkv, S, n_chunks, team):
    """Same rule, computed another way: chunk id of every (bundle row, page)
    pair, then group each bundle row's pages by chunk id; every head of a
    bundle takes its bundle's ranges."""
    P = [-(-x // ps) for x in L]
    rows = [(b, gs) for b in range(len(L)) for gs in range(hkv // team)]
    flat = [(b, gs, lp) for (b, gs) in rows for lp in range(P[b])]
    if S == 1:
        cid = [rows.index((b, gs)) for (b, gs, lp) in flat]
    else:
        tp, pm = len(flat), max(P + [0])
        qp = max(math.ceil(tp / n_chunks), math.ceil(pm / (S - 1)), 1)
        cid = [i // qp for i in range(len(flat))]
    out = {}
    for (b, gs, lp), k in zip(flat, cid):
        out.setdefault((b, gs), {}).setdefault(k, []).append(lp)
    plan = [[[] for _ in range(hkv)] for _ in L]
    for (b, gs), groups in out.items():
        for k in sorted(groups):
            pages = groups[k]
            for g in range(gs * team, (gs + 1) * team):
                plan[b][g].append((pages[0] * ps, min((pages[-1] + 1) * ps, L[b])))
    return plan


@pytest.mark.parametrize("seed", range(6))
def test_split_plan_brute_force(seed):
    rng = np.random.default_rng(seed)
    ps = int(rng.choice([1, 3, 16]))
    L = [int(x) for x in rng.integers(0, 90, size=int(rng.integers(1, 6)))]
    hkv = int(rng.choice([1, 2, 3, 4, 6, 8]))
    for team in sorted({1, plan_args(hkv)["team"]}):
        for S in (1, 2, 3, 5, 9):
            for nc in (2, 7, 2048 // team):
                got = oracle.split_plan(L, ps, hkv, S, n_chunks=nc, team=team)
                assert got == _brute_plan(L, ps, hkv, S, nc, team), (S, nc, team)
                for b in range(len(L)):
                    for g in range(hkv):
                        rr = got[b][g]
                        assert len(rr) <= S
                        assert sum(hi - lo for lo, hi in rr) == L[b]
                        assert all(lo % ps == 0 and lo < hi for lo, hi in rr)
                        assert all(rr[i][1] == rr[i + 1][0] for i in range(len(rr) - 1))


@pytest.mark.parametrize("S", [1, 2, 4, 7, 32])
def test_split_invariance_and_merge_identity(S):
    w = workloads.make("tiny")
    L = w.seq_lens.numpy()
    ip, ix = oracle.bind_full(L, w.req_to_page.numpy(), w.page_size)
    out, lse = oracle.decode_attention(w.q[0], w.k_store[0], w.v_store[0], L, ip, ix, w.scale, w.n_kv_heads)
    o, m, lsep = oracle.split_partials(w.q[0], w.k_store[0], w.v_store[0], L, ip, ix, w.scale,
                                       w.n_kv_heads, w.page_size, S, **plan_args(w.n_kv_heads))
    mo, mlse = oracle.merge_splits(o, lsep)
    np.testing.assert_allclose(mo, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(mlse, lse, rtol=0, atol=1e-12)
    # partition covers each (request, kv head) exactly once
    plan = oracle.split_plan(L, w.page_size, w.n_kv_heads, S, **plan_args(w.n_kv_heads))
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            rr = plan[b][g]
            assert sum(hi - lo for lo, hi in rr) == L[b] and len(rr) <= S
            for lo, hi in rr:
                assert lo % w.page_size == 0
    # empty splits
    empty = ~np.isfinite(lsep)
    assert np.all(np.isneginf(lsep[empty])) and np.all(np.isneginf(m[empty]))
    assert np.all(o[empty] == 0)


def test_split_partial_equals_attention_over_its_range():
    """Each partial is plain attention over its own token range (checked with SDPA)."""
    w = workloads.make("tiny")
    L = w.seq_lens.numpy()
    ip, ix = oracle.bind_full(L, w.req_to_page.numpy(), w.page_size)
    S = 4
    o, m, lse = oracle.split_partials(w.q[0], w.k_store[0], w.v_store[0], L, ip, ix, w.scale,
                                      w.n_kv_heads, w.page_size, S, **plan_args(w.n_kv_heads))
    G = w.group
    plan = oracle.split_plan(L, w.page_size, w.n_kv_heads, S, **plan_args(w.n_kv_heads))
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            hs = slice(g * G, (g + 1) * G)
            for j, (lo, hi) in enumerate(plan[b][g]):
                slots = torch.from_numpy(ix[ip[b] + lo: ip[b] + hi])
                K = w.k_store[0, slots, g].to(torch.float64).unsqueeze(0).expand(G, -1, -1)
                V = w.v_store[0, slots, g].to(torch.float64).unsqueeze(0).expand(G, -1, -1)
                qb = w.q[0, b, hs].to(torch.float64).unsqueeze(1)
                ref = torch.nn.functional.scaled_dot_product_attention(qb, K, V, scale=w.scale)[:, 0]
                np.testing.assert_allclose(o[b, hs, j], ref.numpy(), atol=1e-12, rtol=0)
                smax = (w.scale * torch.einsum("hld,hd->hl", K, w.q[0, b, hs].to(torch.float64))).max(-1).values
                np.testing.assert_allclose(m[b, hs, j], smax.numpy(), atol=1e-12, rtol=0)


def test_merge_weights_by_lse():
    """Two splits with known lse: weights are exp(lse_j - LSE)."""
    o = np.array([[[1.0, 0.0], [0.0, 1.0], [9.0, 9.0]]])
    lse = np.array([[math.log(3.0), math.log(1.0), -math.inf]])
    out, L = oracle.merge_splits(o, lse)
    np.testing.assert_allclose(out[0], [0.75, 0.25], atol=1e-15)
    assert abs(L[0] - math.log(4.0)) < 1e-15
    out, L = oracle.merge_splits(np.zeros((1, 2, 3)), np.full((1, 2), -math.inf))
    assert np.all(out == 0) and np.isneginf(L[0])


# ------------------------------------------------------------ workloads ----

def test_workload_determinism():
    a = workloads.make("tiny")
    b = workloads.make("tiny")
    for name in ("seq_lens", "req_to_page", "q", "k_store", "v_store"):
        x, y = getattr(a, name), getattr(b, name)
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y), name


def test_workload_shapes():
    w = workloads.make("tiny")
    assert w.seq_lens.tolist() == [37, 100]
    assert w.k_store.shape == (1, 64 * 16, 2, 64)
    assert w.q.shape == (1, 2, 4, 64)
    assert w.scale == 0.125
    # pages no request owns are NaN canaries
    owned = set(w.req_to_page[w.req_to_page >= 0].tolist())
    free = [p for p in range(w.num_pages) if p not in owned]
    assert free and torch.isnan(w.k_store[0, free[0] * 16]).all()


# --------------------------------------------------------------- prefill ----

def test_prefill_single_new_token_is_decode():
    """n_b = 1 for every request: the newest token attends to all L_b tokens."""
    w = workloads.make("tiny")
    L = w.seq_lens.numpy()
    ip, ix = oracle.bind_full(L, w.req_to_page.numpy(), w.page_size)
    ref, ref_lse = oracle.decode_attention(w.q[0], w.k_store[0], w.v_store[0], L, ip, ix, w.scale, w.n_kv_heads)
    out, lse = oracle.prefill_attention(w.q[0], w.k_store[0], w.v_store[0], L, [1] * w.batch, ip, ix, w.scale,
                                        w.n_kv_heads)
    assert np.array_equal(out, ref) and np.array_equal(lse, ref_lse)


@pytest.mark.parametrize("name", ["prefill_tiny"])
def test_prefill_against_sdpa_with_causal_mask(name):
    """torch's float64 SDPA over each request's dense K/V with a boolean mask
    that lets query i see keys 0 .. L_b - n_b + i."""
    w = workloads.make(name)
    L = w.seq_lens.numpy()
    n = w.meta["extend_lens"].numpy()
    ip, ix = oracle.bind_full(L, w.req_to_page.numpy(), w.page_size)
    out, lse = oracle.prefill_attention(w.q[0], w.k_store[0], w.v_store[0], L, n, ip, ix, w.scale, w.n_kv_heads)
    G = w.group
    row = 0
    for b in range(w.batch):
        # dense K/V of the request, built by walking its page list (not the oracle's gather)
        slots = [int(w.req_to_page[b, t // w.page_size]) * w.page_size + t % w.page_size for t in range(L[b])]
        K = w.k_store[0, slots].to(torch.float64).repeat_interleave(G, dim=1).transpose(0, 1)  # [H, L, D]
        V = w.v_store[0, slots].to(torch.float64).repeat_interleave(G, dim=1).transpose(0, 1)
        Q = w.q[0, row:row + n[b]].to(torch.float64).transpose(0, 1)  # [H, n, D]
        mask = torch.arange(L[b])[None, :] <= (L[b] - n[b] + torch.arange(n[b]))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=w.scale)
        np.testing.assert_allclose(out[row:row + n[b]], ref.transpose(0, 1).numpy(), atol=1e-12, rtol=0)
        s = w.scale * torch.einsum("hnd,hld->hnl", Q, K)
        s = s.masked_fill(~mask, float("-inf"))
        np.testing.assert_allclose(lse[row:row + n[b]], torch.logsumexp(s, -1).transpose(0, 1).numpy(),
                                   atol=1e-12, rtol=0)
        row += n[b]


def test_prefill_first_token_of_a_fresh_prompt_is_its_value_row():
    """No prefix: new token 0 sees only itself, so its output is its V row."""
    w = workloads.make("prefill_tiny")
    L = w.seq_lens.numpy()
    n = w.meta["extend_lens"].numpy()
    assert L[0] == n[0]
    ip, ix = oracle.bind_full(L, w.req_to_page.numpy(), w.page_size)
    out, _ = oracle.prefill_attention(w.q[0], w.k_store[0], w.v_store[0], L, n, ip, ix, w.scale, w.n_kv_heads)
    slot0 = int(w.req_to_page[0, 0]) * w.page_size
    for h in range(w.n_heads):
        assert np.array_equal(out[0, h], w.v_store[0, slot0, h // w.group].to(torch.float64).numpy())


def test_qo_indptr():
    assert oracle.qo_indptr([3, 0, 5]).tolist() == [0, 3, 3, 8]
