"""Float64 oracle of one paged decode step (test infrastructure only).

Notation: B requests, H query heads, Hkv kv heads, G = H / Hkv, D head dim,
ps page size, L_b = seq_lens[b], P_b = ceil(L_b / ps), S kv splits.

Readings of the pages taken here (the pages describe the engine in commit
bullets and print no formulas):
  * kv_indptr is token-granular: the exclusive prefix sum of seq_lens
    ([CA] bullet on building kv_indptr once per step from seq_lens).
  * kv_indices lists, request after request, the storage slot of every cached
    token; page p owns slots [p*ps, (p+1)*ps) and a request's t-th token lives
    in its (t // ps)-th page at offset t % ps ([CA] bullets on the request ->
    token pool and on the 4-D [n_layers, size, n_kv_heads, head_dim] store).
  * Query head h reads kv head h // G (contiguous query-head groups).
  * The single new query attends to all L_b cached tokens, its own included;
    there is no mask ([CA] bullets dropping decode_mask / page_table).
  * Softmax is natural-base; ``scale`` is the float32 value the kernel gets.
  * Split partition (the pages fix no rule; any partition yields the same
    merged output).  The kv heads form bundles of T heads; the bundle rows
    (request b, bundle gs) are laid end to end, request-major, each as its
    P_b pages.  With S = 1 every non-empty row is one split.  With S >= 2
    that page sequence is cut into chunks of
    Qp = max(ceil(TP / C), ceil(P_max / (S - 1)), 1) pages (TP = total pages
    of all bundle rows); split j of row (b, g) is the intersection of bundle
    row (b, g // T) with the j-th chunk that touches it.  A row then never has
    more than S splits, and every chunk holds the same number of pages.
    Splits past a row's last chunk are empty.  C and T are parameters: the
    caller passes the values of the launch whose partials it checks.
  * Per-layer KV append ([CA] bullets on the single-index write
    buffer[layer_id, loc] and on moving the slot bookkeeping into
    bind_tasks): the new token is already counted in seq_lens, so it is
    position L_b - 1 and its K/V rows go to that position's slot.
  * Per-split outputs ([WS] bullet on decode_o_part / decode_ml_part): o_j is
    normalised by its own softmax sum; the (m, log-sum) pair is
    m_j = max score, ln l_j with l_j = sum exp(s - m_j), so lse_j = m_j + ln l_j.
    An empty split has m = lse = -inf and o = 0.
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = float("-inf")


def to_f64(t) -> np.ndarray:
    """bf16 / fp32 torch tensor or array -> float64 numpy (exact for bf16)."""
    try:
        import torch

        if isinstance(t, torch.Tensor):
            return t.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(t, dtype=np.float64)


# --------------------------------------------------------------------------
# Bind: [CA] bullets on the steady-state +1 update and on building kv_indptr
# a single time per step; [WS] bullet on updating position_ids, seq_lens and
# kv_indptr in place.
# --------------------------------------------------------------------------

def kv_indptr(seq_lens) -> np.ndarray:
    """Exclusive prefix sum of seq_lens: indptr[0] = 0, indptr[b+1] = indptr[b] + L_b."""
    L = [int(x) for x in np.asarray(seq_lens).reshape(-1)]
    out = np.zeros(len(L) + 1, dtype=np.int64)
    running = 0
    for b, lb in enumerate(L):
        running += lb
        out[b + 1] = running
    assert running < 2 ** 31, "kv_indptr must fit int32"
    return out


def kv_indices(seq_lens, req_to_page, page_size: int) -> np.ndarray:
    """Storage slot of every cached token, request after request.

    kv_indices[indptr[b] + t] = req_to_page[b][t // ps] * ps + t % ps, t < L_b.
    """
    L = np.asarray(seq_lens).reshape(-1).astype(np.int64)
    table = np.asarray(req_to_page).astype(np.int64)
    parts = []
    for b in range(len(L)):
        t = np.arange(L[b], dtype=np.int64)
        parts.append(table[b, t // page_size] * page_size + t % page_size)
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def kv_indices_contiguous(seq_lens, req_base) -> np.ndarray:
    """Contiguous cache ([CA] bullet adding a contiguous per-request buffer next
    to the paged cache): request b's t-th token is at slot req_base[b] + t."""
    L = np.asarray(seq_lens).reshape(-1).astype(np.int64)
    base = np.asarray(req_base).reshape(-1).astype(np.int64)
    parts = [base[b] + np.arange(L[b], dtype=np.int64) for b in range(len(L))]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def bind_steady(seq_lens, position_ids):
    """Steady decode step: every request gained exactly one token."""
    return (np.asarray(seq_lens).astype(np.int64) + 1,
            np.asarray(position_ids).astype(np.int64) + 1)


def bind_full(seq_lens, req_to_page, page_size):
    """(kv_indptr, kv_indices) for the given lengths and page table."""
    return kv_indptr(seq_lens), kv_indices(seq_lens, req_to_page, page_size)


# --------------------------------------------------------------------------
# Per-layer KV append ([CA] bullets on the buffer[layer_id, loc] write).
# --------------------------------------------------------------------------

def append_slots(seq_lens, req_to_page, page_size: int) -> np.ndarray:
    """Slot of each request's newest token, position L_b - 1, or -1 when the
    request has no tokens: req_to_page[b][t // ps] * ps + t % ps, t = L_b - 1."""
    L = np.asarray(seq_lens).reshape(-1).astype(np.int64)
    table = np.asarray(req_to_page).astype(np.int64)
    out = np.full(len(L), -1, dtype=np.int64)
    for b in range(len(L)):
        if L[b] > 0:
            t = L[b] - 1
            out[b] = table[b, t // page_size] * page_size + t % page_size
    return out


def append_kv(store_layer, new_rows, slots):
    """A copy of one layer of a store ([num_slots, Hkv, D]) with new_rows[b]
    ([Hkv, D]) written at slots[b] for every slots[b] >= 0 (a bit copy)."""
    out = store_layer.clone()
    for b, slot in enumerate(np.asarray(slots).reshape(-1)):
        if slot >= 0:
            out[int(slot)] = new_rows[b]
    return out


# --------------------------------------------------------------------------
# Attention: exact softmax attention of each single-token query over all of
# its cached tokens ([WS] bullets on attn_paged_decode writing decode_out).
# --------------------------------------------------------------------------

def gather_rows(store_layer, slots) -> np.ndarray:
    """Rows of one layer's [num_slots, Hkv, D] store at the given slots, float64."""
    return to_f64(store_layer[np.asarray(slots, dtype=np.int64)]) if len(slots) else \
        np.zeros((0,) + tuple(store_layer.shape[1:]), dtype=np.float64)


def attention_rows(q_h, k_rows, v_rows, scale):
    """One query head against its L cached rows (float64).

    s_t = scale * <q, k_t>;  m = max s;  Z = sum exp(s - m);
    out = sum exp(s_t - m) v_t / Z;  returns (out, m, ln Z).
    With L = 0 returns (zeros, -inf, -inf).
    """
    q_h = np.asarray(q_h, dtype=np.float64)
    if k_rows.shape[0] == 0:
        return np.zeros(v_rows.shape[-1], dtype=np.float64), NEG_INF, NEG_INF
    s = float(np.float32(scale)) * (k_rows @ q_h)
    m = float(s.max())
    w = np.exp(s - m)
    z = float(w.sum())
    out = (w @ v_rows) / z
    return out, m, math.log(z)


def decode_attention(q_layer, k_layer, v_layer, seq_lens, indptr, indices, scale,
                     n_kv_heads, pairs=None):
    """Full (unsplit) decode attention for one layer.

    q_layer [B, H, D]; k_layer / v_layer [num_slots, Hkv, D].
    Returns out [B, H, D] and lse [B, H] (float64).  ``pairs`` restricts the
    work to a list of (b, kv_head) pairs; other entries are left NaN.
    """
    q = to_f64(q_layer)
    B, H, D = q.shape
    G = H // n_kv_heads
    out = np.full((B, H, D), np.nan)
    lse = np.full((B, H), np.nan)
    if pairs is None:
        pairs = [(b, g) for b in range(B) for g in range(n_kv_heads)]
    for b, g in pairs:
        slots = indices[indptr[b]:indptr[b + 1]]
        K = gather_rows(k_layer[:, g], slots)
        V = gather_rows(v_layer[:, g], slots)
        for h in range(g * G, (g + 1) * G):
            o, m, lnz = attention_rows(q[b, h], K, V, scale)
            out[b, h] = o
            lse[b, h] = m + lnz
    return out, lse


# --------------------------------------------------------------------------
# Paged prefill / extend ([WS] / [CA] bullets on the prefill qo_indptr built
# once per step in the workspace and reused by every layer's prefill).
# Reading: request b's last n_b = extend_lens[b] cached tokens are new and each
# has a query; q rows are laid out request after request (qo_indptr is the
# exclusive prefix sum of extend_lens).  New token i of request b sits at
# position L_b - n_b + i and attends causally: to cached tokens 0 .. that
# position (the prefix and the new tokens up to itself).
# --------------------------------------------------------------------------

def qo_indptr(extend_lens) -> np.ndarray:
    """Exclusive prefix sum of the new-token counts."""
    return kv_indptr(extend_lens)


def prefill_attention(q_rows, k_layer, v_layer, seq_lens, extend_lens, kv_ptr, indices, scale, n_kv_heads):
    """Causal attention of every new token over its request's cache.

    q_rows [sum n_b, H, D]; returns out [sum n_b, H, D] and lse [sum n_b, H]
    (float64).
    """
    q = to_f64(q_rows)
    T, H, D = q.shape
    G = H // n_kv_heads
    L = np.asarray(seq_lens).reshape(-1).astype(np.int64)
    n = np.asarray(extend_lens).reshape(-1).astype(np.int64)
    qo = qo_indptr(n)
    out = np.full((T, H, D), np.nan)
    lse = np.full((T, H), np.nan)
    for b in range(len(L)):
        slots = indices[kv_ptr[b]:kv_ptr[b + 1]]
        for g in range(n_kv_heads):
            K = gather_rows(k_layer[:, g], slots)
            V = gather_rows(v_layer[:, g], slots)
            for i in range(int(n[b])):
                pos = int(L[b] - n[b] + i)      # this token's position
                for h in range(g * G, (g + 1) * G):
                    o, m, lnz = attention_rows(q[qo[b] + i, h], K[:pos + 1], V[:pos + 1], scale)
                    out[qo[b] + i, h] = o
                    lse[qo[b] + i, h] = m + lnz
    return out, lse


# --------------------------------------------------------------------------
# Split-KV partials and their log-sum-exp merge ([WS] bullets on
# decode_o_part / decode_ml_part and the split partial buffers).
# --------------------------------------------------------------------------

def _pages(seq_lens, page_size):
    return [-(-int(x) // page_size) for x in np.asarray(seq_lens).reshape(-1)]


def chunk_pages(seq_lens, page_size, n_kv_heads, S, n_chunks, team):
    """Qp for S >= 2: max(ceil(TP / C), ceil(P_max / (S - 1)), 1), where the
    bundle rows hold TP = (n_kv_heads / team) * sum P pages and C = n_chunks."""
    P = _pages(seq_lens, page_size)
    tp = (n_kv_heads // int(team)) * sum(P)
    p_max = max(P + [0])
    return max(-(-tp // int(n_chunks)), -(-p_max // (int(S) - 1)), 1)


def split_plan(seq_lens, page_size, n_kv_heads, S, n_chunks, team):
    """Token ranges of the splits: plan[b][g] = [(lo, hi), ...] indexed by j.

    The kv heads form bundles of ``team`` heads (gs = g // team); the bundle
    rows (b, gs) are walked in order, page by page, and a new split starts
    whenever the chunk index of the global page changes (S >= 2) or a row
    begins.  Every head of a bundle gets its bundle row's splits.  The chunk
    count C = ``n_chunks`` and the bundle size ``team`` are the caller's: the
    partition is defined for any C >= 1 and any team dividing n_kv_heads.
    """
    team = int(team)
    assert n_kv_heads % team == 0 and int(n_chunks) >= 1
    hs = n_kv_heads // team
    L = [int(x) for x in np.asarray(seq_lens).reshape(-1)]
    P = _pages(L, page_size)
    qp = None if int(S) == 1 else chunk_pages(L, page_size, n_kv_heads, S, n_chunks, team)
    bundle = [[[] for _ in range(hs)] for _ in L]
    gp = 0  # global page index of the current page
    for b, lb in enumerate(L):
        for gs in range(hs):
            cur = None  # (chunk id, first local page)
            for lp in range(P[b]):
                k = 0 if qp is None else gp // qp
                if cur is None or k != cur[0]:
                    if cur is not None:
                        bundle[b][gs].append((cur[1] * page_size, min(lp * page_size, lb)))
                    cur = (k, lp)
                gp += 1
            if cur is not None:
                bundle[b][gs].append((cur[1] * page_size, lb))
    return [[list(bundle[b][g // team]) for g in range(n_kv_heads)] for b in range(len(L))]


def split_partials(q_layer, k_layer, v_layer, seq_lens, indptr, indices, scale,
                   n_kv_heads, page_size, S, n_chunks, team, pairs=None):
    """Per-split outputs: o [B, H, S, D], m [B, H, S], lse [B, H, S] (float64),
    under split_plan(seq_lens, page_size, n_kv_heads, S, n_chunks, team).

    Empty splits: o = 0, m = lse = -inf.
    """
    q = to_f64(q_layer)
    B, H, D = q.shape
    G = H // n_kv_heads
    plan = split_plan(seq_lens, page_size, n_kv_heads, S, n_chunks, team)
    o = np.full((B, H, S, D), np.nan)
    m = np.full((B, H, S), np.nan)
    lse = np.full((B, H, S), np.nan)
    if pairs is None:
        pairs = [(b, g) for b in range(B) for g in range(n_kv_heads)]
    for b, g in pairs:
        slots_b = indices[indptr[b]:indptr[b + 1]]
        ranges = plan[b][g]
        assert len(ranges) <= S, "more splits than S"
        for j in range(S):
            lo, hi = ranges[j] if j < len(ranges) else (0, 0)
            K = gather_rows(k_layer[:, g], slots_b[lo:hi])
            V = gather_rows(v_layer[:, g], slots_b[lo:hi])
            for h in range(g * G, (g + 1) * G):
                oj, mj, lnz = attention_rows(q[b, h], K, V, scale)
                o[b, h, j] = oj
                m[b, h, j] = mj
                lse[b, h, j] = mj + lnz
    return o, m, lse


def merge_splits(o_part, lse_part):
    """Combine splits: LSE = log sum_j exp(lse_j); out = sum_j exp(lse_j - LSE) o_j.

    Empty splits (lse = -inf) get weight 0.  All splits empty -> out = 0,
    LSE = -inf.  Shapes: o_part [..., S, D], lse_part [..., S].
    """
    o_part = np.asarray(o_part, dtype=np.float64)
    lse_part = np.asarray(lse_part, dtype=np.float64)
    top = np.max(lse_part, axis=-1, keepdims=True)
    finite = np.isfinite(top)
    top_safe = np.where(finite, top, 0.0)
    w = np.where(np.isfinite(lse_part), np.exp(lse_part - top_safe), 0.0)
    wsum = w.sum(axis=-1, keepdims=True)
    o_clean = np.where(np.isfinite(lse_part)[..., None], o_part, 0.0)
    out = np.where(wsum > 0,
                   (w[..., None] * o_clean).sum(axis=-2) / np.where(wsum > 0, wsum, 1.0),
                   0.0)
    lse = np.where(finite[..., 0], top_safe[..., 0] + np.log(np.where(wsum[..., 0] > 0, wsum[..., 0], 1.0)),
                   NEG_INF)
    return out, lse
