"""The C ABI library loads and exports what include/paged_decode.h declares (no GPU).

Only pure-host entry points are called here: sizing, strerror, argument
validation that fails before any HIP call.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_decode.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(paged_decode_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def abi():
    from paged_kv_decode_10_amd import _abi
    if not os.path.exists(_abi.LIB_PATH):
        pytest.fail("libpaged_decode.so is not built (run python -m paged_kv_decode_10_amd.build)")
    return _abi


def test_header_matches_binding_list(abi):
    assert _declared_functions() == sorted(abi.EXPORTS)


def test_library_exports_every_declared_symbol(abi):
    out = subprocess.run(["nm", "-D", "--defined-only", abi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (paged_decode_\w+)", out))
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(abi.lib(), name)


def _cfg(abi, **kw):
    base = dict(n_layers=2, n_heads=32, n_kv_heads=8, head_dim=128, page_size=16, max_batch=4,
                max_splits=8, max_pages_per_req=16, num_slots=1024, max_total_tokens=1000)
    base.update(kw)
    return abi.PdConfig(*[base[f] for f, _ in abi.PdConfig._fields_])


def test_workspace_bytes_and_validation(abi):
    L = abi.lib()
    n = ctypes.c_size_t(0)
    c = _cfg(abi)
    assert L.paged_decode_workspace_bytes(ctypes.byref(c), ctypes.byref(n)) == abi.PD_OK
    rows = 4 * 32 * 8
    # kv_indptr, kv_indices, page_indptr, o_part, ml_part, qo_indptr, item_indptr, req_order, meta,
    # error word, each 256-aligned
    al = lambda x: -(-x // 256) * 256
    want = (al(5 * 4) + al(1000 * 4) + al(5 * 4) + al(rows * 128 * 4) + al(rows * 2 * 4) + al(5 * 4) + al(5 * 4)
            + al(4 * 4) + al(64) + al(4))
    assert n.value == want
    for bad, code in [(dict(head_dim=96), abi.PD_E_UNSUPPORTED), (dict(n_heads=30), abi.PD_E_UNSUPPORTED),
                      (dict(n_heads=8 * 17), abi.PD_E_UNSUPPORTED), (dict(page_size=0), abi.PD_E_INVALID),
                      (dict(max_batch=0), abi.PD_E_INVALID), (dict(max_batch=2048), abi.PD_E_UNSUPPORTED),
                      (dict(num_slots=8), abi.PD_E_INVALID), (dict(max_splits=1000), abi.PD_E_UNSUPPORTED)]:
        c = _cfg(abi, **bad)
        assert L.paged_decode_workspace_bytes(ctypes.byref(c), ctypes.byref(n)) == code, bad
    assert L.paged_decode_workspace_bytes(None, ctypes.byref(n)) == abi.PD_E_INVALID


def test_host_side_rejections(abi):
    L = abi.lib()
    c = _cfg(abi)
    h = ctypes.c_void_p()
    assert L.paged_decode_init_workspace(ctypes.byref(c), None, 1 << 20, ctypes.byref(h)) == abi.PD_E_INVALID
    assert L.paged_decode_init_workspace(ctypes.byref(c), ctypes.c_void_p(0x1001), 1 << 30,
                                         ctypes.byref(h)) == abi.PD_E_INVALID  # misaligned
    assert L.paged_decode_init_workspace(ctypes.byref(c), ctypes.c_void_p(0x100000), 16,
                                         ctypes.byref(h)) == abi.PD_E_CAPACITY  # arena too small
    s = ctypes.c_int32()
    assert L.paged_decode_num_splits(None, 1, 0, ctypes.byref(s)) == abi.PD_E_INVALID
    assert L.paged_decode_bind(None, 1, 0, None, None, None, None) == abi.PD_E_INVALID
    assert L.paged_decode_bind_contiguous(None, 1, 0, None, None, None, None) == abi.PD_E_INVALID
    assert L.paged_decode_attn(None, 1, 0, 1, None, None, None, 1.0, None) == abi.PD_E_INVALID
    assert L.paged_decode_merge(None, 1, 1, None, None) == abi.PD_E_INVALID
    assert L.paged_decode_bind_extend(None, 1, None, None, None, None, None) == abi.PD_E_INVALID
    assert L.paged_decode_prefill_attn(None, 1, 0, None, 0, None, None, 1.0, None, None) == abi.PD_E_INVALID
    assert L.paged_decode_append_kv(None, 1, 0, None, None, None, None, None) == abi.PD_E_INVALID
    assert L.paged_decode_append_attn(None, 1, 0, 1, None, None, None, None, None, 1.0, None) == abi.PD_E_INVALID
    assert L.paged_decode_graph_pool_create(None, None, 0, ctypes.byref(h)) == abi.PD_E_INVALID
    assert L.paged_decode_graph_pool_warmup(None) == abi.PD_E_INVALID
    assert L.paged_decode_graph_pool_step(None, 1, None) == abi.PD_E_INVALID
    assert L.paged_decode_graph_pool_destroy(None) == abi.PD_E_INVALID
    assert L.paged_decode_destroy(None) == abi.PD_E_INVALID
    for code in range(5):
        assert L.paged_decode_strerror(code)
    assert L.paged_decode_strerror(99) == b"unknown status"


def test_product_path_has_no_oracle_or_fallback():
    """The package must not import the oracle nor carry a CPU path."""
    pkg = os.path.join(ROOT, "paged_kv_decode_10_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "workloads" not in text or f == "build.py", f


def test_plan_constants_match_header(abi):
    text = open(HEADER).read()
    for name in ("PD_PLAN_WAVES", "PD_PLAN_TEAM_MAX"):
        m = re.search(rf"^#define\s+{name}\s+(\d+)\s*$", text, flags=re.M)
        assert m and int(m.group(1)) == getattr(abi, name), name
