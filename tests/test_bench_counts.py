"""The bench's closed-form count of non-empty split partials (used for the
algorithmic bytes of the roofline) against the oracle's split plan, which
walks the pages one by one.  CPU only."""
import numpy as np
import pytest

import bench
import oracle
from tests.plan_params import plan_args


@pytest.mark.parametrize("seed", range(40))
def test_row_splits_match_oracle_plan(seed):
    rng = np.random.default_rng(seed)
    n_kv_heads = int(rng.choice([1, 2, 3, 4, 8]))
    page_size = int(rng.choice([1, 7, 16, 32]))
    B = int(rng.integers(1, 40))
    hi = int(rng.choice([40, 700, 5000]))
    L = rng.integers(0, hi, size=B)
    S = int(rng.choice([1, 2, 3, 17, 64, 256]))
    got = bench.row_splits(L, page_size, n_kv_heads, S)
    plan = oracle.split_plan(L, page_size, n_kv_heads, S, **plan_args(n_kv_heads))
    want = np.array([[len(plan[b][g]) for g in range(n_kv_heads)] for b in range(B)])
    assert np.array_equal(got, want), (L.tolist(), page_size, n_kv_heads, S)
    assert bench.split_segments(L, page_size, n_kv_heads, S) == int(want.sum())
    if S > 1:
        assert want.max() <= S
