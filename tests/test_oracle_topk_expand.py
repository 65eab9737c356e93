"""Pins of the oracle's exact top-K and expansion: brute force on tiny
rows, invariants at scale, and the counts printed on the pages."""
import itertools
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def golden():
    vals = {}
    for line in open(os.path.join(HERE, "golden", "page_closed_forms.txt")):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split()
            vals[k] = v
    return vals


def brute_topk(s, K):
    """Exhaustive: the unique K-subset whose every member outranks every
    non-member under (score desc, index asc)."""
    G = len(s)
    if G <= K:
        return list(range(G))

    def beats(a, b):
        return s[a] > s[b] or (s[a] == s[b] and a < b)

    hits = []
    for sub in itertools.combinations(range(G), K):
        rest = set(range(G)) - set(sub)
        if all(beats(a, b) for a in sub for b in rest):
            hits.append(list(sub))
    assert len(hits) == 1
    return hits[0]


def test_topk_matches_exhaustive_search_with_ties():
    rng = np.random.default_rng(0)
    pool = np.array([0.0, -0.0, 1.0, 2.0, 2.0, 3.5, -1.0, -np.inf], np.float32)
    for trial in range(60):
        G = int(rng.integers(1, 11))
        K = int(rng.integers(1, 8))
        s = rng.choice(pool, G).astype(np.float32)
        row = np.full((1, 12), -np.inf, np.float32)
        row[0, :G] = s
        got = oracle.topk(row, [G], K)[0]
        want = brute_topk(list(s), K)
        assert list(got[got >= 0]) == want, (s, K)
        assert np.all(got[len(want):] == -1)


def test_topk_matches_sorted_order_on_random_rows():
    rng = np.random.default_rng(1)
    for G, K in ((64, 16), (300, 64), (1000, 999), (2048, 512)):
        s = np.round(rng.standard_normal(G) * 4).astype(np.float32)  # many ties
        got = oracle.topk(s[None], [G], K)[0]
        want = sorted(sorted(range(G), key=lambda g: (-s[g], g))[:K])
        assert list(got) == want


def test_topk_invariants_large_row():
    rng = np.random.default_rng(2)
    G, K = 65536, 2048
    s = rng.random(G).astype(np.float32)
    s[::97] = 0.0
    got = oracle.topk(s[None], [G], K)[0]
    assert len(got) == K and np.all(np.diff(got) > 0)
    sel = np.zeros(G, bool)
    sel[got] = True
    worst_in = s[sel].min()
    best_out = s[~sel].max()
    assert worst_in >= best_out
    # ties at the boundary go to the lowest indices
    tied_out = np.flatnonzero(~sel & (s == worst_in))
    tied_in = np.flatnonzero(sel & (s == worst_in))
    if len(tied_out) and len(tied_in):
        assert tied_in.max() < tied_out.min()


def test_topk_short_rows_keep_everything():
    s = np.arange(10, dtype=np.float32)[None]
    got = oracle.topk(s, [7], 512)[0]
    assert list(got[:7]) == list(range(7)) and np.all(got[7:] == -1)
    got = oracle.topk(s, [0], 4)[0]
    assert np.all(got == -1)


def test_topk_rejects_nan():
    s = np.array([[1.0, np.nan, 2.0]], np.float32)
    with pytest.raises(ValueError):
        oracle.topk(s, [3], 1)


def test_expand_counts_and_tail():
    K = 512
    for r in (0, 1, 2, 3):
        G = 2048
        L = 4 * G + r
        groups = np.sort(np.random.default_rng(r).choice(G, K, replace=False)).astype(np.int32)
        W = oracle.token_width(K)
        t = oracle.position_tokens(groups, L, 0, W)
        n = int((t >= 0).sum())
        assert n == 4 * K + r
        v = t[:n]
        assert np.all(np.diff(v) > 0) and v.max() < L
        assert set(range(4 * G, L)) <= set(v.tolist())
        assert set((v[v < 4 * G] // 4).tolist()) == set(groups.tolist())


def test_page_printed_counts():
    gd = golden()
    K_tokens = int(gd["token_budget_tokens"])
    assert K_tokens / 16384 == float(gd["token_budget_fraction_at_16k"])
    ratio = int(gd["compress_ratio"])
    budgets = [int(x) for x in gd["group_budgets"].split(",")]
    assert K_tokens // ratio in budgets
    # width of one query's token list = 4K + largest tail
    assert oracle.token_width(512) == int(gd["max_selected_slots_k512"])
    assert max(int(x) for x in gd["causal_tail_lengths"].split(",")) == ratio - 1
    # packed BF16 K+V bytes at capacity, two KV heads, head dim 256
    cap, D = int(gd["kv_capacity_tokens"]), int(gd["head_dim"])
    assert cap * 2 * D * 2 * 2 == int(gd["packed_bf16_kv_mib_262144"]) * 2 ** 20


def test_mtp_shared_selection_invariants():
    # S_j = S0 + groups completed since the base position; |T_j| = 4(K + G_j - G0) + r_j
    K = 8
    G0 = 40
    S0 = np.sort(np.random.default_rng(3).choice(G0, K, replace=False)).astype(np.int32)
    W = oracle.token_width(K, 3)
    for r0 in (0, 1, 2, 3):
        L0 = 4 * G0 + r0
        for j in range(3):
            Lj = L0 + j
            Gj, rj = Lj // 4, Lj % 4
            t = oracle.position_tokens(S0, L0, j, W)
            v = t[t >= 0]
            assert len(v) == 4 * (K + Gj - G0) + rj
            groups_j = set((v[v < 4 * Gj] // 4).tolist())
            assert set(S0.tolist()) <= groups_j
            assert groups_j - set(S0.tolist()) == set(range(G0, Gj))
            if Lj > 4 * G0:  # the current token is attended unless it closes a group
                assert v.max() == Lj - 1
