"""A seeded sweep of decode and prefill configurations through the C ABI,
each compared with the oracle like the fixed cases: head shapes of the
local GQA pairs, BF16 and FP8 caches, budgets from 1 to 2,048 groups
(including the three of the heuristic selector's prerequisite), ragged
and empty contexts at page and group boundaries, 1 to 4 MTP positions and
page-table entries out of range.  The case parameters come from one fixed
generator, so every run checks the same cases; the data come from the
seeded workload generators."""
import numpy as np
import pytest

import workload
from tests.test_gpu_parity import _decode_check
from tests.test_gpu_prefill import _prefill_check

pytestmark = pytest.mark.gpu

HEADS = [(16, 2), (24, 2), (12, 1), (8, 1), (16, 1), (6, 1), (3, 1), (8, 2)]
BUDGETS = [1, 3, 17, 100, 255, 512, 777, 1024, 2048]
EDGE_LENS = [0, 1, 3, 4, 5, 63, 64, 65, 255, 256, 257, 4095, 4096, 4097]


def _decode_cases(n=48):
    r = np.random.RandomState(20261203)
    cases = []
    for i in range(n):
        hq, hkv = HEADS[r.randint(len(HEADS))]
        gq = hq // hkv
        Q = int(r.randint(1, 5))
        while Q * gq > 48:
            Q -= 1
        B = int(r.randint(1, 7))
        lens = [int(r.choice(EDGE_LENS)) if r.rand() < 0.3 else int(r.randint(0, 40000))
                for _ in range(B)]
        cases.append(dict(seed=7000 + i, hq=hq, hkv=hkv, Q=Q, lens=lens,
                          K=int(BUDGETS[r.randint(len(BUDGETS))]),
                          kv="fp8" if r.rand() < 0.5 else "bf16", bad=r.rand() < 0.3))
    return cases


def _prefill_cases(n=24):
    r = np.random.RandomState(20261204)
    cases = []
    for i in range(n):
        hq, hkv = HEADS[r.randint(len(HEADS))]
        first = int(r.choice(EDGE_LENS)) if r.rand() < 0.3 else int(r.randint(0, 20000))
        cases.append(dict(seed=7500 + i, hq=hq, hkv=hkv, first=first,
                          n_q=int(r.randint(1, 300)), K=int(BUDGETS[r.randint(len(BUDGETS))]),
                          kv="fp8" if r.rand() < 0.5 else "bf16", bad=r.rand() < 0.3))
    return cases


def _break_pages(wl, seed):
    """About one page in twelve of every row out of range (-1 or past the
    pool), at positions fixed by the case seed."""
    r = np.random.RandomState(seed)
    rows, cols = wl.page_table.shape
    for b in range(rows):
        for c in range(cols):
            if r.rand() < 1.0 / 12:
                wl.page_table[b, c] = -1 if r.rand() < 0.5 else wl.num_pages + int(r.randint(8))


@pytest.mark.parametrize("case", _decode_cases(), ids=lambda c: f"d{c['seed']}")
def test_random_decode(gpu, case):
    c = case
    wl = workload.decode_workload(c["seed"], c["lens"], q_per_req=c["Q"], num_q_heads=c["hq"],
                                  num_kv_heads=c["hkv"], topk_groups=c["K"], kv_dtype=c["kv"])
    if c["bad"]:
        _break_pages(wl, c["seed"])
    _decode_check(wl, gpu)


@pytest.mark.parametrize("case", _prefill_cases(), ids=lambda c: f"p{c['seed']}")
def test_random_prefill(gpu, case):
    c = case
    wl = workload.prefill_workload(c["seed"], c["first"], c["n_q"], num_q_heads=c["hq"],
                                   num_kv_heads=c["hkv"], topk_groups=c["K"], kv_dtype=c["kv"])
    if c["bad"]:
        _break_pages(wl, c["seed"])
    _prefill_check(wl, gpu, np.arange(wl.n_q))


# KV head counts of 3, 4 and 8 (an XCD then serves one KV head only when the
# count divides 8): a second fixed generator, so the cases above stay as
# they are
HEADS_KV = [(24, 3), (16, 4), (32, 8), (48, 3), (32, 4)]


def _kv_head_cases(n_dec=12, n_pf=8):
    r = np.random.RandomState(20261205)
    dec, pf = [], []
    for i in range(n_dec):
        hq, hkv = HEADS_KV[r.randint(len(HEADS_KV))]
        Q = int(r.randint(1, 5))
        while Q * (hq // hkv) > 48:
            Q -= 1
        lens = [int(r.randint(0, 40000)) for _ in range(int(r.randint(1, 5)))]
        dec.append(dict(seed=8000 + i, hq=hq, hkv=hkv, Q=Q, lens=lens,
                        K=int(BUDGETS[r.randint(len(BUDGETS))]),
                        kv="fp8" if r.rand() < 0.5 else "bf16", bad=r.rand() < 0.3))
    for i in range(n_pf):
        hq, hkv = HEADS_KV[r.randint(len(HEADS_KV))]
        pf.append(dict(seed=8500 + i, hq=hq, hkv=hkv, first=int(r.randint(0, 20000)),
                       n_q=int(r.randint(1, 200)), K=int(BUDGETS[r.randint(len(BUDGETS))]),
                       kv="fp8" if r.rand() < 0.5 else "bf16", bad=r.rand() < 0.3))
    return dec, pf


@pytest.mark.parametrize("case", _kv_head_cases()[0], ids=lambda c: f"d{c['seed']}")
def test_random_decode_kv_heads(gpu, case):
    test_random_decode(gpu, case)


@pytest.mark.parametrize("case", _kv_head_cases()[1], ids=lambda c: f"p{c['seed']}")
def test_random_prefill_kv_heads(gpu, case):
    test_random_prefill(gpu, case)
