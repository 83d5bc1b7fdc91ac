"""Host-side checks of the C ABI (no GPU needed, no compute launched).

The library must load, export every function include/mla.h declares, and
reject invalid arguments on the host before touching a device.
"""
import ctypes

import pytest

import int2_quantized_absorbed_amd as M
from int2_quantized_absorbed_amd import binding as Bd

DS = M.Dims(512, 64, 128, 128, 128, 32, 0)


def test_library_exports_every_declared_symbol():
    lib = M.lib()
    names = M.header_functions()
    assert "mla_decode_absorbed" in names and "mla_append_quant" in names
    assert "mla_calibrate_rotation" in names and "mla_fit_clip" in names
    for n in names:
        assert hasattr(lib, n), n
    assert M.mla_abi_version() == 3


def test_status_strings():
    for st in range(6):
        assert isinstance(M.mla_status_string(st), str)
    assert M.mla_status_string(0) == "ok"


def _dims(**kw):
    base = dict(kv_lora_rank=512, qk_rope_head_dim=64, qk_nope_head_dim=128, v_head_dim=128,
                num_heads=128, group_size=32, index_head_dim=0, rope_bits=0)
    base.update(kw)
    return Bd.mla_dims(*base.values())


BAD_DIMS = [
    dict(kv_lora_rank=0), dict(kv_lora_rank=100), dict(group_size=8), dict(group_size=64),
    dict(kv_lora_rank=48, group_size=32), dict(qk_rope_head_dim=0), dict(qk_rope_head_dim=3),
    dict(num_heads=0), dict(index_head_dim=-2), dict(v_head_dim=0),
    dict(rope_bits=2), dict(rope_bits=8), dict(rope_bits=4, qk_rope_head_dim=40),
]


@pytest.mark.parametrize("bad", BAD_DIMS)
def test_invalid_dims_rejected_everywhere(bad):
    lib = M.lib()
    d = _dims(**bad)
    P = ctypes.c_void_p(16)
    cache = Bd.mla_cache(16, 16, 16, 0, 10)
    assert lib.mla_prepare_rotation(ctypes.byref(d), P, P, None) == Bd.MLA_ERR_INVALID_ARG
    assert lib.mla_append_quant(ctypes.byref(d), P, 0, P, None, P, 4, P, P, ctypes.byref(cache), None) \
        == Bd.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_workspace_size(ctypes.byref(d), 1, 1) == 0
    assert lib.mla_decode_absorbed(ctypes.byref(d), P, P, P, P, ctypes.byref(cache), P, P, 1, 1, 1, 0.1, P,
                                   1 << 30, P, P, None) == Bd.MLA_ERR_INVALID_ARG
    assert lib.mla_calibrate_rotation(ctypes.byref(d), P, 0, 10, P, None, None) == Bd.MLA_ERR_INVALID_ARG
    assert M.mla_last_error() != ""


def test_null_dims():
    lib = M.lib()
    assert lib.mla_prepare_rotation(None, None, None, None) == Bd.MLA_ERR_INVALID_ARG
    assert "NULL" in M.mla_last_error()


def test_decode_argument_checks():
    lib = M.lib()
    d = _dims()
    P = ctypes.c_void_p(256)
    cache = Bd.mla_cache(256, 256, 256, 0, 1000)
    call = lambda **kw: lib.mla_decode_absorbed(
        ctypes.byref(d), kw.get("qn", P), P, P, P, ctypes.byref(cache), P, P, kw.get("B", 2), kw.get("tq", 1),
        kw.get("causal", 1), kw.get("scale", 0.07), kw.get("ws", P), kw.get("wsb", 1 << 40), P, P, None)
    assert call(tq=0) == Bd.MLA_ERR_INVALID_ARG
    assert call(tq=65) == Bd.MLA_ERR_INVALID_ARG
    assert call(causal=2) == Bd.MLA_ERR_INVALID_ARG
    assert call(B=-1) == Bd.MLA_ERR_INVALID_ARG
    assert call(scale=float("nan")) == Bd.MLA_ERR_INVALID_ARG
    assert call(qn=ctypes.c_void_p(0)) == Bd.MLA_ERR_INVALID_ARG
    assert call(qn=ctypes.c_void_p(258)) == Bd.MLA_ERR_INVALID_ARG       # misaligned
    assert call(wsb=16) == Bd.MLA_ERR_WORKSPACE
    assert "workspace" in M.mla_last_error()
    assert call(B=0) == Bd.MLA_OK                                         # nothing to do
    d2 = _dims(kv_lora_rank=1024)
    assert lib.mla_decode_absorbed(ctypes.byref(d2), P, P, P, P, ctypes.byref(cache), P, P, 2, 1, 1, 0.07, P,
                                   1 << 40, P, P, None) == Bd.MLA_ERR_UNSUPPORTED


def test_decode_noalloc_argument_checks():
    """The static-scratch decode checks its arguments and its workspace need
    on the host: a decode larger than the scratch is refused before anything
    is launched."""
    lib = M.lib()
    d = _dims()
    P = ctypes.c_void_p(256)
    cache = Bd.mla_cache(256, 256, 256, 0, 1000)
    call = lambda **kw: lib.mla_decode_absorbed_noalloc(
        ctypes.byref(d), kw.get("qn", P), P, P, P, ctypes.byref(cache), P, P, kw.get("B", 2), kw.get("tq", 1),
        kw.get("causal", 1), 0.07, P, P, None)
    assert M.mla_decode_noalloc_max_workspace() == 48 << 20
    assert call(tq=0) == Bd.MLA_ERR_INVALID_ARG
    assert call(B=-1) == Bd.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_absorbed_noalloc(None, P, P, P, P, ctypes.byref(cache), P, P, 2, 1, 1, 0.07, P, P,
                                           None) == Bd.MLA_ERR_INVALID_ARG
    big_b = 256  # 256 sequences of 128 heads x 8 queries: far beyond 48 MiB of workspace
    assert M.mla_decode_workspace_size(DS, big_b, 8) > M.mla_decode_noalloc_max_workspace()
    assert call(B=big_b, tq=8) == Bd.MLA_ERR_WORKSPACE
    assert "static scratch" in M.mla_last_error()


def test_index_topk_argument_checks():
    lib = M.lib()
    d = _dims(index_head_dim=64)
    P = ctypes.c_void_p(256)
    cache = Bd.mla_cache(256, 256, 256, 256, 1000)
    call = lambda **kw: lib.mla_index_topk(
        ctypes.byref(kw.get("d", d)), kw.get("q", P), ctypes.byref(kw.get("cache", cache)), P, P, kw.get("B", 2),
        kw.get("k", 64), P, kw.get("wsb", 1 << 40), kw.get("sel", P), P, None)
    assert call(d=_dims(index_head_dim=0)) == Bd.MLA_ERR_INVALID_ARG       # no indexer key
    assert call(d=_dims(index_head_dim=12)) == Bd.MLA_ERR_UNSUPPORTED
    assert call(k=0) == Bd.MLA_ERR_INVALID_ARG
    assert call(B=-1) == Bd.MLA_ERR_INVALID_ARG
    assert call(q=ctypes.c_void_p(0)) == Bd.MLA_ERR_INVALID_ARG
    assert call(sel=ctypes.c_void_p(260)) == Bd.MLA_ERR_INVALID_ARG       # misaligned
    assert call(cache=Bd.mla_cache(256, 256, 256, 0, 1000)) == Bd.MLA_ERR_INVALID_ARG
    assert call(wsb=16) == Bd.MLA_ERR_WORKSPACE
    assert call(B=0) == Bd.MLA_OK
    # one score per cache slot, and a histogram and chunk counts per sequence
    w1 = lib.mla_index_topk_workspace_size(ctypes.byref(d), 1, 1000)
    assert w1 >= 4000 and lib.mla_index_topk_workspace_size(ctypes.byref(d), 2, 1000) > w1
    assert lib.mla_index_topk_workspace_size(ctypes.byref(d), -1, 1000) == 0


def test_decode_sparse_argument_checks():
    lib = M.lib()
    d = _dims()
    P = ctypes.c_void_p(256)
    cache = Bd.mla_cache(256, 256, 256, 0, 1000)
    call = lambda **kw: lib.mla_decode_sparse(
        ctypes.byref(d), P, P, P, P, ctypes.byref(cache), P, kw.get("sel", P), kw.get("n_sel", P), kw.get("B", 2),
        kw.get("k", 64), 0.07, P, kw.get("wsb", 1 << 40), P, P, None)
    assert call(k=0) == Bd.MLA_ERR_INVALID_ARG
    assert call(sel=ctypes.c_void_p(0)) == Bd.MLA_ERR_INVALID_ARG
    assert call(n_sel=ctypes.c_void_p(264)) == Bd.MLA_ERR_INVALID_ARG     # misaligned
    assert call(B=-1) == Bd.MLA_ERR_INVALID_ARG
    assert call(wsb=16) == Bd.MLA_ERR_WORKSPACE
    assert "mla_decode_sparse" in M.mla_last_error()
    assert call(B=0) == Bd.MLA_OK


def test_append_argument_checks():
    lib = M.lib()
    d = _dims()
    P = ctypes.c_void_p(256)
    cache = Bd.mla_cache(256, 256, 256, 0, 1000)
    call = lambda **kw: lib.mla_append_quant(
        ctypes.byref(kw.get("d", d)), P, kw.get("dt", 0), P, kw.get("idx", None), P, kw.get("n", 8), P, P,
        ctypes.byref(kw.get("cache", cache)), None)
    assert call(n=0) == Bd.MLA_OK
    assert call(n=-1) == Bd.MLA_ERR_INVALID_ARG
    assert call(dt=7) == Bd.MLA_ERR_INVALID_ARG
    assert call(idx=P) == Bd.MLA_ERR_INVALID_ARG          # idx key without index_head_dim
    d_idx = _dims(index_head_dim=64)
    assert call(d=d_idx) == Bd.MLA_ERR_INVALID_ARG        # index_head_dim without idx key
    assert call(cache=Bd.mla_cache(0, 256, 256, 0, 10)) == Bd.MLA_ERR_INVALID_ARG
    assert call(cache=Bd.mla_cache(256, 256, 256, 0, -1)) == Bd.MLA_ERR_INVALID_ARG


def test_decode_step_argument_checks():
    """Every argument of the combined step is checked before anything is
    launched: with no GPU here a launch would report MLA_ERR_HIP, so a
    check error (or MLA_OK with nothing to do) shows nothing ran."""
    lib = M.lib()
    d = _dims()
    P = ctypes.c_void_p(256)
    cache = Bd.mla_cache(256, 256, 256, 0, 1000)
    call = lambda **kw: lib.mla_decode_step(
        ctypes.byref(d), kw.get("lat", P), kw.get("dt", 0), P, kw.get("idx", None), P, kw.get("n", 8), P, P,
        kw.get("qn", P), P, P, P, ctypes.byref(cache), P, P, kw.get("B", 2), kw.get("tq", 1), 1, 0.07, P,
        kw.get("wsb", 1 << 40), P, P, None)
    assert call(n=-1) == Bd.MLA_ERR_INVALID_ARG
    assert call(dt=7) == Bd.MLA_ERR_INVALID_ARG
    assert call(lat=ctypes.c_void_p(0)) == Bd.MLA_ERR_INVALID_ARG
    assert call(idx=P) == Bd.MLA_ERR_INVALID_ARG           # idx key without index_head_dim
    assert "mla_decode_step" in M.mla_last_error()
    # valid append, invalid decode: rejected before the append is launched
    assert call(tq=0) == Bd.MLA_ERR_INVALID_ARG
    assert call(qn=ctypes.c_void_p(258)) == Bd.MLA_ERR_INVALID_ARG
    assert call(wsb=16) == Bd.MLA_ERR_WORKSPACE
    assert call(n=0, B=0) == Bd.MLA_OK                     # nothing to do


def test_calibration_argument_checks():
    lib = M.lib()
    d = _dims()
    P = ctypes.c_void_p(256)
    assert lib.mla_calibrate_rotation(ctypes.byref(d), P, 0, 0, P, None, None) == Bd.MLA_ERR_INVALID_ARG
    assert lib.mla_calibrate_rotation(ctypes.byref(d), P, 5, 10, P, None, None) == Bd.MLA_ERR_INVALID_ARG
    W = lib.mla_calibrate_rotation_weighted
    assert W(ctypes.byref(d), P, 0, 0, P, P, P, None, None) == Bd.MLA_ERR_INVALID_ARG      # n_cal < 1
    assert W(ctypes.byref(d), P, 5, 10, P, P, P, None, None) == Bd.MLA_ERR_INVALID_ARG     # dtype
    assert W(ctypes.byref(d), P, 0, 10, None, P, P, None, None) == Bd.MLA_ERR_INVALID_ARG  # w_uk NULL
    assert W(ctypes.byref(d), P, 0, 10, P, None, P, None, None) == Bd.MLA_ERR_INVALID_ARG  # w_uv NULL
    assert W(None, P, 0, 10, P, P, P, None, None) == Bd.MLA_ERR_INVALID_ARG                # dims NULL
    grid = (ctypes.c_float * 2)(1.0, 1.5)
    assert lib.mla_fit_clip(ctypes.byref(d), P, 0, 10, P, grid, 2, P, None, None) == Bd.MLA_ERR_INVALID_ARG
    assert lib.mla_fit_clip(ctypes.byref(d), P, 0, 10, P, grid, 0, P, None, None) == Bd.MLA_ERR_INVALID_ARG
    assert lib.mla_set_decode_variant(3) == Bd.MLA_ERR_INVALID_ARG
    assert lib.mla_set_decode_variant(0) == Bd.MLA_OK


def test_workspace_size_is_monotone():
    s1 = M.mla_decode_workspace_size(DS, 8, 1)
    s2 = M.mla_decode_workspace_size(DS, 16, 1)
    s3 = M.mla_decode_workspace_size(DS, 8, 8)
    assert 0 < s1 < s2 and s1 < s3
    assert M.mla_decode_workspace_size(DS, 8, 0) == 0


def _gdims(**kw):
    a = dict(head_dim=128, num_q_heads=32, num_kv_heads=8, group_size=32, k_rotation=0)
    a.update(kw)
    return Bd.gqa_dims(a["head_dim"], a["num_q_heads"], a["num_kv_heads"], a["group_size"], a["k_rotation"])


@pytest.mark.parametrize("bad", [dict(head_dim=100), dict(head_dim=512), dict(group_size=8),
                                 dict(num_q_heads=30), dict(num_kv_heads=0), dict(num_q_heads=4, num_kv_heads=8),
                                 dict(k_rotation=2), dict(k_rotation=-1)])
def test_gqa_dims_rejected(bad):
    lib = M.lib()
    d = _gdims(**bad)
    P = ctypes.c_void_p(256)
    assert lib.gqa_decode_workspace_size(ctypes.byref(d), 2, 1) == 0
    assert lib.gqa_prepare_rotation(ctypes.byref(d), P, P, None) == Bd.MLA_ERR_INVALID_ARG
    assert "gqa_prepare_rotation" in M.mla_last_error()


def test_gqa_workspace_grows_with_batch():
    lib = M.lib()
    d = _gdims()
    w1 = lib.gqa_decode_workspace_size(ctypes.byref(d), 1, 1)
    w8 = lib.gqa_decode_workspace_size(ctypes.byref(d), 8, 1)
    assert 0 < w1 < w8 and w8 % 256 == 0
    assert lib.gqa_decode_workspace_size(ctypes.byref(d), 8, 0) == 0


def test_gqa_decode_argument_checks():
    lib = M.lib()
    d = _gdims()
    P = ctypes.c_void_p(256)
    cache = Bd.gqa_cache(256, 256, 256, 256, 1000)
    call = lambda **kw: lib.gqa_decode(
        ctypes.byref(d), kw.get("q", P), ctypes.byref(kw.get("cache", cache)), P, P, P, P, kw.get("B", 2),
        kw.get("tq", 1), kw.get("causal", 1), kw.get("scale", 0.09), P, kw.get("wsb", 1 << 40), P, P, None)
    assert call(tq=0) == Bd.MLA_ERR_INVALID_ARG
    assert call(causal=2) == Bd.MLA_ERR_INVALID_ARG
    assert call(scale=float("nan")) == Bd.MLA_ERR_INVALID_ARG
    assert call(B=-1) == Bd.MLA_ERR_INVALID_ARG
    assert call(q=ctypes.c_void_p(0)) == Bd.MLA_ERR_INVALID_ARG
    assert call(q=ctypes.c_void_p(264)) == Bd.MLA_ERR_INVALID_ARG         # misaligned
    assert call(cache=Bd.gqa_cache(256, 0, 256, 256, 1000)) == Bd.MLA_ERR_INVALID_ARG
    assert call(wsb=16) == Bd.MLA_ERR_WORKSPACE
    assert "gqa_decode" in M.mla_last_error()
    assert call(B=0) == Bd.MLA_OK


def test_gqa_append_and_calibrate_argument_checks():
    lib = M.lib()
    d = _gdims()
    P = ctypes.c_void_p(256)
    cache = Bd.gqa_cache(256, 256, 256, 256, 1000)
    app = lambda **kw: lib.gqa_append_quant(ctypes.byref(d), kw.get("k", P), P, P, kw.get("n", 8), P, P, P, P,
                                            ctypes.byref(cache), None)
    assert app(n=0) == Bd.MLA_OK
    assert app(n=-1) == Bd.MLA_ERR_INVALID_ARG
    assert app(k=ctypes.c_void_p(0)) == Bd.MLA_ERR_INVALID_ARG
    assert app(k=ctypes.c_void_p(258)) == Bd.MLA_ERR_INVALID_ARG
    cal = lambda **kw: lib.gqa_calibrate(ctypes.byref(d), P, P, P, kw.get("n", 64), kw.get("scale", 0.09), P, P,
                                         None, None, None)
    assert cal(n=0) == Bd.MLA_ERR_INVALID_ARG
    assert cal(n=65537) == Bd.MLA_ERR_INVALID_ARG
    assert cal(scale=float("inf")) == Bd.MLA_ERR_INVALID_ARG
    grid = (ctypes.c_float * 2)(1.0, 0.0)
    fit = lambda ng: lib.gqa_fit_clip(ctypes.byref(d), P, 64, P, grid, ng, P, None)
    assert fit(0) == Bd.MLA_ERR_INVALID_ARG
    assert fit(2) == Bd.MLA_ERR_INVALID_ARG                             # grid value 0 is outside (0, 1]
