"""The C-ABI library loads without a GPU, exports every function that
include/qsa.h declares, and its host-only checks behave as documented."""
import ctypes
import os
import re

import pytest

import learned_sparse_attention_amd as qsa
import workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "qsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("qsa_index_topk", "qsa_decode", "qsa_prefill", "qsa_validate"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = qsa.load()
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_validate_and_sizes():
    g = workload.geometry()
    assert qsa.validate(g) == 0
    for field, bad in (("head_dim", 128), ("page_size", 32), ("compress_ratio", 8),
                       ("idx_heads", 4), ("idx_dim", 128), ("topk_groups", 4096),
                       ("topk_groups", 0), ("kv_dtype", 7), ("num_kv_heads", 3)):
        assert qsa.validate(dict(g, **{field: bad})) == -2, field
    # the group budget: any K in 1..2048 (the exact top-K has no further
    # limit; the set {512, 1024, 2048} binds only a heuristic selector)
    for K in (1, 3, 511, 512, 777, 1024, 2047, 2048):
        assert qsa.validate(dict(g, topk_groups=K)) == 0, K
    for K in (-1, 0, 2049, 4096):
        assert qsa.validate(dict(g, topk_groups=K)) == -2, K
    # indexer forms: 8 x 64 with a key per head, or 4 x 128 sharing one key
    assert qsa.validate(dict(g, idx_key_heads=0)) == 0
    assert qsa.validate(workload.geometry(indexer="mqa")) == 0
    for hi, di, hk in ((4, 128, 4), (8, 64, 1), (4, 64, 1), (8, 128, 1)):
        assert qsa.validate(dict(g, idx_heads=hi, idx_dim=di, idx_key_heads=hk)) == -2
    assert qsa.validate(dict(g, k_scale=0.0)) == -1
    assert qsa.validate(dict(g, v_scale=float("nan"))) == -1
    assert qsa.token_width(g, 1) == 4 * 512 + 3
    assert qsa.token_width(dict(g, topk_groups=2048), 3) == 4 * 2048 + 5
    assert qsa.token_width(g, 5) == 0
    assert qsa.decode_workspace_size(g, 8, 1, 262144) > 8 * 65536 * 4
    assert qsa.decode_workspace_size(g, 8, 1, 262145) == 0
    assert qsa.prefill_workspace_size(g, 4096, 32768) >= 4096 * 8192 * 4
    assert qsa.index_topk_workspace_size(g, 3, 1000) > 0
    # 12 heads per KV head x 4 positions = 48 rows is fine; 16 x 5 is not
    assert qsa.decode_workspace_size(dict(g, num_q_heads=24), 4, 4, 1000) > 0


def test_entry_points_reject_bad_arguments_before_any_launch():
    lib = qsa.load()
    g = qsa._geom(workload.geometry())
    c = qsa.PagedCache(None, None, None, None, 0, 0)
    # null cache pointers: refused on the host, nothing is enqueued
    assert lib.qsa_decode(ctypes.byref(g), ctypes.byref(c), 1, 1, 100, *([None] * 8), None, 0,
                          None) == -1
    assert lib.qsa_prefill(ctypes.byref(g), ctypes.byref(c), 0, 0, 1, *([None] * 7), None, 0,
                           None) == -1
    assert lib.qsa_index_topk(ctypes.byref(g), ctypes.byref(c), 1, 100, *([None] * 6), None, 0,
                              None) == -1
    bad = qsa._geom(dict(workload.geometry(), head_dim=64))
    assert lib.qsa_decode(ctypes.byref(bad), ctypes.byref(c), 1, 1, 100, *([None] * 8), None, 0,
                          None) == -2
    assert lib.qsa_status_string(-3) == b"workspace missing, too small or misaligned"


def test_append_argument_checks():
    lib = qsa.load()
    g = qsa._geom(workload.geometry(kv_dtype="fp8", k_scale=0.5, v_scale=0.5))
    nul = [None] * 4
    # null caches / tensors with work to do: refused before any launch
    assert lib.qsa_append_kv(ctypes.byref(g), *nul, 4, 4, 1, None, None, 3, None, None, None,
                             None) == -1
    # nothing to append: success without touching any pointer
    assert lib.qsa_append_kv(ctypes.byref(g), *nul, 4, 4, 0, None, None, 3, None, None, None,
                             None) == 0
    assert lib.qsa_append_kv(ctypes.byref(g), *nul, 4, 4, 2, None, None, 0, None, None, None,
                             None) == 0
    assert lib.qsa_append_kv(ctypes.byref(g), *nul, 4, 4, -1, None, None, 3, None, None, None,
                             None) == -1
    bad = qsa._geom(dict(workload.geometry(), num_kv_heads=3))
    assert lib.qsa_append_kv(ctypes.byref(bad), *nul, 4, 4, 1, None, None, 3, None, None, None,
                             None) == -2
    assert [qsa.append_khat_slots(n) for n in (-1, 0, 1, 4, 5, 8, 4096)] == [0, 0, 1, 1, 2, 2,
                                                                           1024]


def test_empty_inputs_succeed_without_touching_buffers():
    # batch / chunk / row count 0: success, decided on the host before any
    # pointer is read (the cache pointers are placeholders that are never
    # dereferenced, and every tensor pointer is null)
    lib = qsa.load()
    g = qsa._geom(workload.geometry())
    fake = ctypes.c_void_p(0x1000)
    c = qsa.PagedCache(fake, fake, fake, fake, 4, 4)
    assert lib.qsa_decode(ctypes.byref(g), ctypes.byref(c), 0, 1, 256, *([None] * 8), None, 0,
                          None) == 0
    assert lib.qsa_prefill(ctypes.byref(g), ctypes.byref(c), 0, 100, 0, *([None] * 7), None, 0,
                           None) == 0
    assert lib.qsa_index_topk(ctypes.byref(g), ctypes.byref(c), 0, 256, *([None] * 6), None, 0,
                              None) == 0
    assert lib.qsa_index_score(ctypes.byref(g), ctypes.byref(c), 0, 256, *([None] * 5),
                               None) == 0
    assert lib.qsa_index_score_prefill(ctypes.byref(g), ctypes.byref(c), 0, 100, 0, None, None,
                                       None, None) == 0
    # the same calls with work to do and null tensors are refused
    assert lib.qsa_decode(ctypes.byref(g), ctypes.byref(c), 1, 1, 256, *([None] * 8), None, 0,
                          None) == -1
    assert lib.qsa_prefill(ctypes.byref(g), ctypes.byref(c), 0, 100, 1, *([None] * 7), None, 0,
                           None) == -1
    # a context beyond the page table's reach is refused even when empty
    assert lib.qsa_decode(ctypes.byref(g), ctypes.byref(c), 0, 1, 4 * 64 + 1, *([None] * 8),
                          None, 0, None) == -1
