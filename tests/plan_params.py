"""The split plan's launch constants as include/paged_decode.h states them
(PD_PLAN_WAVES, PD_PLAN_TEAM_MAX), turned into the chunk count and bundle
size that the oracle's split_plan / split_partials take.  Read from the
header text, so the tests check the kernel against its documented contract."""
import math
import os
import re

_HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "paged_decode.h")


def _define(name: str) -> int:
    with open(_HEADER) as f:
        m = re.search(rf"^#define\s+{name}\s+(\d+)\s*$", f.read(), flags=re.M)
    assert m, f"{name} is not defined in {_HEADER}"
    return int(m.group(1))


PLAN_WAVES = _define("PD_PLAN_WAVES")
PLAN_TEAM_MAX = _define("PD_PLAN_TEAM_MAX")


def plan_args(n_kv_heads: int) -> dict:
    """{'n_chunks': C, 'team': T}: T = gcd(n_kv_heads, PD_PLAN_TEAM_MAX), C = PD_PLAN_WAVES / T."""
    team = math.gcd(int(n_kv_heads), PLAN_TEAM_MAX)
    return {"n_chunks": PLAN_WAVES // team, "team": team}
