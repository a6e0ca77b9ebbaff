"""The C ABI library loads on a machine without a GPU, exports every function
include/sekv.h declares, and rejects invalid arguments on the host before any
HIP call."""
import ctypes
import os
import re

import pytest

import compressed_kv_attention_sekv_amd as S

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "sekv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sekv_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(S.library_path()):
        pytest.skip("libsekv.so not built")
    return S.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(S.EXPORTED_SYMBOLS)


def test_config_struct_layout_matches_header():
    # int32 x8, double x2, int32 x2, uint64, int32 x2 -> 72 bytes with natural alignment
    assert ctypes.sizeof(S.SekvConfig) == 72
    assert ctypes.sizeof(S.SekvRouteOut) == 48


def _cfg(**kw):
    c = S.make_config(2, 8, 2)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value,msg", [
    ("head_dim", 64, "head_dim"),
    ("n_q_heads", 7, "multiple"),
    ("n_kv_heads", 0, "multiple"),
    ("route_dim", 0, "route_dim"),
    ("route_dim", 65, "route_dim"),
    ("max_rank", 0, "max_rank"),
    ("max_rank", 129, "max_rank"),
    ("min_span_len", 0, "min_span_len"),
    ("window", -1, "window"),
    ("n_layers", 0, "n_layers"),
    ("kv_dtype", 7, "kv_dtype"),
    ("factor_tier", 3, "factor_tier"),
    ("alpha", float("nan"), "finite"),
    ("svd_mode", 2, "svd_mode"),
    ("append_capacity", -1, "append_capacity"),
])
def test_build_rejects_bad_config(L, field, value, msg):
    cfg = _cfg(**{field: value})
    out = ctypes.c_void_p(123)
    st = L.sekv_build_spans(ctypes.byref(cfg), 100, ctypes.c_void_p(8), ctypes.c_void_p(8),
                            ctypes.c_void_p(8), ctypes.c_void_p(8), None, None, ctypes.byref(out))
    assert st == S.SEKV_ERR_INVALID
    assert msg in L.sekv_last_error().decode()
    assert out.value is None


def test_build_rejects_null_inputs_and_sizes(L):
    cfg = _cfg()
    out = ctypes.c_void_p()
    assert L.sekv_build_spans(ctypes.byref(cfg), 100, None, ctypes.c_void_p(8), ctypes.c_void_p(8),
                              ctypes.c_void_p(8), None, None, ctypes.byref(out)) == S.SEKV_ERR_INVALID
    assert L.sekv_build_spans(ctypes.byref(cfg), 0, ctypes.c_void_p(8), ctypes.c_void_p(8),
                              ctypes.c_void_p(8), ctypes.c_void_p(8), None, None,
                              ctypes.byref(out)) == S.SEKV_ERR_INVALID
    assert L.sekv_build_spans(ctypes.byref(cfg), 10, ctypes.c_void_p(8), ctypes.c_void_p(8),
                              ctypes.c_void_p(8), ctypes.c_void_p(8), None, None,
                              None) == S.SEKV_ERR_INVALID
    assert L.sekv_segment(None, 10, ctypes.c_void_p(8), None, None, None, None) == S.SEKV_ERR_INVALID


def test_calls_on_null_cache_are_rejected(L):
    ro = S.SekvRouteOut()
    assert L.sekv_route(None, 0, None, None, None, ctypes.byref(ro), None) == S.SEKV_ERR_INVALID
    assert L.sekv_decode_attn(None, 0, None, ctypes.byref(ro), None, None, 0, None,
                              None) == S.SEKV_ERR_INVALID
    assert L.sekv_cap_budget(None, ctypes.byref(ro), 0, None) == S.SEKV_ERR_INVALID
    assert L.sekv_cap_budget_layer(None, ctypes.byref(ro), 0, None) == S.SEKV_ERR_INVALID
    assert L.sekv_set_residency(None, 1 << 20, 1 << 16) == S.SEKV_ERR_INVALID
    assert L.sekv_set_fetch_mode(None, S.SEKV_FETCH_MEMCPY) == S.SEKV_ERR_INVALID
    assert L.sekv_apply_gates(None, ctypes.c_void_p(8), ctypes.c_void_p(8), 0.5,
                              None) == S.SEKV_ERR_INVALID
    out6 = (ctypes.c_uint64 * 6)()
    assert L.sekv_residency_stats(None, out6, 0) == S.SEKV_ERR_INVALID
    assert L.sekv_decode_workspace_bytes(None) == 0
    info = S.SekvCacheInfo()
    assert L.sekv_cache_info_get(None, ctypes.byref(info)) == S.SEKV_ERR_INVALID
    L.sekv_cache_destroy(None)  # no-op


def test_fetch_failure_hook_arguments(L):
    assert L.sekv_test_fail_fetch(-1) == S.SEKV_ERR_INVALID
    assert b"n must be" in L.sekv_last_error()
    assert L.sekv_test_fail_fetch(0) == S.SEKV_OK


def test_batch_calls_reject_bad_arguments(L):
    P, SZ = ctypes.c_void_p, ctypes.c_size_t
    n = 2
    nulls = (P * n)()
    ros = (S.SekvRouteOut * n)()
    sizes = (SZ * n)()
    for fn, extra in ((L.sekv_route_attn_batch, (P(8), P(8))), (L.sekv_decode_attn_batch, ())):
        def call(caches, batch):
            return fn(caches, batch, 0, nulls, *extra, ros, nulls, nulls, sizes, None)
        assert call(None, n) == S.SEKV_ERR_INVALID              # no cache array
        for batch in (0, -1, S.SEKV_MAX_BATCH + 1):             # batch size out of range
            assert call(nulls, batch) == S.SEKV_ERR_INVALID
            assert b"batch" in L.sekv_last_error()
        assert call(nulls, n) == S.SEKV_ERR_INVALID             # NULL caches in the array
    # the shared projection and thresholds are required by the routing variant
    assert L.sekv_route_attn_batch(nulls, n, 0, nulls, None, None, ros, nulls, nulls, sizes,
                                   None) == S.SEKV_ERR_INVALID


def test_binding_checks_tensor_arguments():
    import torch
    cfg = S.make_config(1, 4, 1, kv_dtype="f32")
    with pytest.raises(ValueError, match="device tensor"):
        S.sekv_build_spans(cfg, torch.zeros(10), torch.zeros(1, 1, 10, 128),
                           torch.zeros(1, 1, 10, 128), torch.zeros(1, 4, 32, 128))
