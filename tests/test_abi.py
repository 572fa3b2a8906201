"""The C ABI library loads, exports every declared entry point, and validates configurations
on the host (no GPU work)."""
import ctypes
import os
import re

import pytest

from sparse_mla_attention_score_amd import hisparse as hsb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hisparse.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:hs_status|const char\*)\s+(\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = hsb.lib()
    declared = _declared()
    assert len(declared) >= 15
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(hsb.EXPORTED) == declared


def _cfg(**kw):
    base = dict(topk=2048, max_batch=64, max_queries=4, max_pages_per_req=2049,
                num_gpu_blocks=30000, num_idx_blocks=131200, num_host_blocks=118000)
    base.update(kw)
    return hsb.make_config(**base)


def test_workspace_and_pool_sizes():
    cfg = _cfg()
    ws = hsb.hs_workspace_bytes(cfg)
    lmax = 2049 * 64
    assert ws > 64 * 4 * lmax * 4          # at least the score scratch
    assert ws < 4 * 2 ** 30
    assert hsb.hs_host_pool_bytes(cfg) == 118000 * 64 * 656
    cfg2 = _cfg(n_layers=4, kv_dtype=hsb.HS_BF16)
    assert hsb.hs_host_pool_bytes(cfg2) == 4 * 118000 * 64 * 1152


@pytest.mark.parametrize("field,value,status", [
    ("block_size", 32, hsb.HS_ERR_UNSUPPORTED),
    ("n_heads", 128, hsb.HS_ERR_UNSUPPORTED),
    ("d_qk", 512, hsb.HS_ERR_UNSUPPORTED),
    ("topk", 4096, hsb.HS_ERR_UNSUPPORTED),
    ("topk", 0, hsb.HS_ERR_UNSUPPORTED),
    ("max_queries", 5, hsb.HS_ERR_UNSUPPORTED),
    ("max_batch", 0, hsb.HS_ERR_INVALID_ARG),
    ("n_layers", 0, hsb.HS_ERR_INVALID_ARG),
    ("hot_rows_per_req", 100, hsb.HS_ERR_INVALID_ARG),      # not a multiple of 64
    ("hot_rows_per_req", 4096, hsb.HS_ERR_INVALID_ARG),     # < S * K = 8192
    ("kv_dtype", 7, hsb.HS_ERR_UNSUPPORTED),
    ("num_gpu_blocks", 0, hsb.HS_ERR_INVALID_ARG),
    ("num_gpu_blocks", 1 << 26, hsb.HS_ERR_INVALID_ARG),     # row ids would overflow int32
    ("hot_leasing", 2, hsb.HS_ERR_INVALID_ARG),
])
def test_config_validation(field, value, status):
    cfg = _cfg()
    setattr(cfg, field, value)
    with pytest.raises(hsb.HiSparseError) as e:
        hsb.hs_workspace_bytes(cfg)
    assert e.value.status == status
    assert hsb.hs_last_error()


def test_default_hot_buffer_follows_the_pages_rule():
    # 0 selects (S + 1) x top-K: 2 x K without MTP, (spec + 2) x K with MTP3
    assert hsb.hs_workspace_bytes(_cfg(hot_rows_per_req=0)) == hsb.hs_workspace_bytes(_cfg(hot_rows_per_req=10240))
    c1 = _cfg(max_queries=1, max_batch=32)
    assert hsb.hs_workspace_bytes(c1) == hsb.hs_workspace_bytes(_cfg(max_queries=1, max_batch=32, hot_rows_per_req=4096))


def test_status_strings():
    assert hsb.hs_status_string(0) == "HS_OK"
    assert hsb.hs_status_string(-2) == "HS_ERR_UNSUPPORTED"
    lib = hsb.lib()
    assert lib.hs_destroy(None) == hsb.HS_ERR_INVALID_ARG


def test_kernel_timing_argument_checks():
    lib = hsb.lib()
    assert lib.hs_kernel_timing(None, 1) == hsb.HS_ERR_INVALID_ARG
    ms = (ctypes.c_double * hsb.HS_KERNEL_COUNT)()
    n = (ctypes.c_int64 * hsb.HS_KERNEL_COUNT)()
    assert lib.hs_kernel_times(None, ms, n, hsb.HS_KERNEL_COUNT) == hsb.HS_ERR_INVALID_ARG


def test_kernel_ids_match_header():
    text = open(HEADER).read()
    ids = dict((m[0], int(m[1])) for m in re.findall(r"(HS_KERNEL_\w+)\s*=\s*(\d+)", text))
    assert ids["HS_KERNEL_COUNT"] == hsb.HS_KERNEL_COUNT
    for i, name in enumerate(hsb.KERNEL_NAMES):
        assert ids[f"HS_KERNEL_{name.upper()}"] == i


def test_write_side_argument_checks():
    # a NULL context is refused on the host, before any HIP call
    lib = hsb.lib()
    pages = (ctypes.c_int32 * 2)(0, 0)
    lens = (ctypes.c_int32 * 1)(65)
    freed = (ctypes.c_int32 * 1)()
    assert lib.hisparse_materialize_pages(None, pages, 1, None) == hsb.HS_ERR_INVALID_ARG
    assert "ctx is NULL" in hsb.hs_last_error()
    assert lib.hisparse_release_pages(None, pages, 1, lens, freed, None) == hsb.HS_ERR_INVALID_ARG
    assert "ctx is NULL" in hsb.hs_last_error()
    a, b = ctypes.c_int64(), ctypes.c_int64()
    assert lib.hs_select_paths(None, ctypes.byref(a), ctypes.byref(b)) == hsb.HS_ERR_INVALID_ARG


def test_leasing_argument_checks():
    # NULL contexts and lists are refused on the host; leasing needs a host pool
    lib = hsb.lib()
    lst = (ctypes.c_int32 * 2)(0, 1)
    assert lib.hs_hot_release(None, lst, 2, None) == hsb.HS_ERR_INVALID_ARG
    assert lib.hs_hot_pool_give(None, lst, 2, None) == hsb.HS_ERR_INVALID_ARG
    n = ctypes.c_int32()
    assert lib.hs_hot_pool_read(None, lst, 2, ctypes.byref(n)) == hsb.HS_ERR_INVALID_ARG
    assert lib.hisparse_resolve_plan(None, None, None, 1, 1, None, None, None, None) == hsb.HS_ERR_INVALID_ARG
    with pytest.raises(hsb.HiSparseError) as e:
        hsb.hs_workspace_bytes(_cfg(hot_leasing=1, num_host_blocks=0))
    assert e.value.status == hsb.HS_ERR_INVALID_ARG and "host pool" in hsb.hs_last_error()
    # the pool's ring takes one int32 per GPU block
    assert hsb.hs_workspace_bytes(_cfg(num_gpu_blocks=4096)) >= hsb.hs_workspace_bytes(_cfg(num_gpu_blocks=2048)) + 8192 - 256
