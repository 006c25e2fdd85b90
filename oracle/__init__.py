"""CPU oracle for split-KV paged decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this package; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library: it is a plain, slow, float64 restatement of what a decode step
computes, written so it can be checked against its sources by eye.

Sources (web pages, each a commit view of the AstrAI engine):
  [WS]  AstrAI commit 0b661bae, astrai/inference/core/workspace.py view
  [CA]  AstrAI commit cbc58447, astrai/inference/core/cache.py view
  [EX]  AstrAI commit e0f7fa8e, astrai/inference/core/executor.py view
The pages are commit-message bullet lists; they are cited by the bullet's
subject.  Where they are silent, the reading taken is stated at the function.

Every function here is pinned by CPU tests against something other than
itself (brute force, closed forms, torch's float64 SDPA, hand-derived
examples); no function is "parity unpinned".
"""
from .paged_attention import (  # noqa: F401
    NEG_INF,
    append_kv,
    append_slots,
    attention_rows,
    bind_full,
    bind_steady,
    decode_attention,
    gather_rows,
    kv_indices,
    kv_indices_contiguous,
    kv_indptr,
    merge_splits,
    prefill_attention,
    qo_indptr,
    chunk_pages,
    split_partials,
    split_plan,
    to_f64,
)
