"""Pins of the oracle's indexer score (assumed per-head ReLU-weighted form).

The pages print no indexer formula, so these pins fix the code against the
assumed form  s_g = sum_h w_h * max(0, q_h . k̂_{g,h})  through special cases
and closed forms that a dropped term, a wrong head/dim index, a transposed
operand or a wrong page mapping would break.  The form itself stays
"parity unpinned" with respect to the pages.
"""
import numpy as np

import oracle

GPP = 16  # groups per 64-token page at ratio 4


def khat_from_groups(kg: np.ndarray, perm=None):
    """Place logical groups [G, Hi, Di] into pages via a page table."""
    G, Hi, Di = kg.shape
    n_pages = (G + GPP - 1) // GPP
    perm = np.arange(n_pages) if perm is None else np.asarray(perm)
    kh = np.full((n_pages, GPP, Hi, Di), np.nan, np.float32)
    for g in range(G):
        kh[perm[g // GPP], g % GPP] = kg[g]
    return kh, perm.astype(np.int32)[None, :]


def run(q, w, kg, L=None, perm=None, bf16=False):
    G = kg.shape[0]
    L = 4 * G if L is None else L
    kh, pt = khat_from_groups(kg, perm)
    gstride = ((L // 4) + 3) // 4 * 4 if L // 4 > 0 else 4
    gstride = max(gstride, kh.shape[0] * GPP)
    return oracle.scores([0], [L], q[None], w[None], kh, pt, kh.shape[0], gstride,
                         round_bf16_inputs=bf16)[0]


def test_one_hot_keys_select_relu_of_query_entries():
    # H_i = 1, w = 1, k̂_g = e_{j(g)}  =>  s_g = max(q_j, 0)
    Di = 64
    q = np.linspace(-3, 3, Di).astype(np.float32)[None]
    G = 48
    j = (np.arange(G) * 7) % Di
    kg = np.zeros((G, 1, Di), np.float32)
    kg[np.arange(G), 0, j] = 1.0
    s = run(q, np.ones(1, np.float32), kg)
    assert np.array_equal(s[:G], np.maximum(q[0, j], 0).astype(np.float32))


def test_single_active_head_and_weight():
    # only head h carries a key: s = w_h * ReLU(q_h . k_h), other heads ignored
    rng = np.random.default_rng(1)
    Hi, Di, G = 8, 64, 32
    q = rng.integers(-3, 4, (Hi, Di)).astype(np.float32)
    w = np.arange(1, Hi + 1).astype(np.float32) / 4
    for h in (0, 5, 7):
        kg = np.zeros((G, Hi, Di), np.float32)
        kg[:, h, :] = rng.integers(-2, 3, (G, Di))
        s = run(q, w, kg)[:G]
        dots = kg[:, h, :].astype(np.int64) @ q[h].astype(np.int64)
        assert np.array_equal(s, (w[h] * np.maximum(dots, 0)).astype(np.float32))


def test_aligned_keys_closed_form():
    # k̂_{g,h} = a_g q_h  =>  s_g = max(a_g, 0) * sum_h w_h |q_h|^2
    rng = np.random.default_rng(2)
    Hi, Di, G = 8, 64, 40
    q = rng.integers(-2, 3, (Hi, Di)).astype(np.float32)
    w = rng.integers(0, 4, Hi).astype(np.float32)
    a = np.arange(G, dtype=np.float32) - 20
    kg = a[:, None, None] * q[None]
    s = run(q, w, kg)[:G]
    c = float((w * (q.astype(np.float64) ** 2).sum(1)).sum())
    assert np.array_equal(s, (np.maximum(a, 0) * c).astype(np.float32))


def test_negative_weight_and_negative_dots():
    Hi, Di = 8, 64
    q = np.ones((Hi, Di), np.float32)
    kg = np.stack([np.full((Hi, Di), v, np.float32) for v in (1.0, -1.0)])
    w = np.full(Hi, -0.5, np.float32)
    s = run(q, w, kg)
    assert s[0] == -0.5 * 64 * 8          # negative weight keeps its sign
    assert s[1] == 0.0 and not np.signbit(s[1])  # ReLU zero, canonical +0


def test_single_rounding_of_exact_sum():
    # 1 + 2^-24 + 2^-25 = 1 + 0.75 ulp(1): correctly rounded to 1 + 2^-23;
    # sequential fp32 accumulation would give 1.0
    Hi, Di = 1, 64
    q = np.zeros((Hi, Di), np.float32)
    q[0, :3] = [1.0, 2.0 ** -24, 2.0 ** -25]
    kg = np.zeros((4, Hi, Di), np.float32)
    kg[:, 0, :3] = 1.0
    s = run(q, np.ones(1, np.float32), kg)
    assert s[0] == np.float32(1.0 + 2.0 ** -23)


def test_bf16_rounding_of_indexer_inputs():
    Hi, Di = 1, 64
    q = np.zeros((Hi, Di), np.float32)
    q[0, 0] = 1.0 + 2.0 ** -10  # not bf16-exact; rounds to 1.0
    kg = np.zeros((4, Hi, Di), np.float32)
    kg[:, 0, 0] = 3.0 + 2.0 ** -9  # rounds to 3.0 (tie -> even)
    s32 = run(q, np.ones(1, np.float32), kg)
    s16 = run(q, np.ones(1, np.float32), kg, bf16=True)
    assert s16[0] == 3.0 and s32[0] != 3.0


def test_causal_mask_and_page_permutation():
    rng = np.random.default_rng(5)
    Hi, Di, G = 8, 64, 70
    q = rng.standard_normal((Hi, Di)).astype(np.float32)
    w = rng.random(Hi).astype(np.float32)
    kg = rng.standard_normal((G, Hi, Di)).astype(np.float32)
    L = 4 * 61 + 3  # 61 complete groups; groups >= 61 are not candidates
    kg_poison = kg.copy()
    kg_poison[61:] = np.nan
    a = run(q, w, kg, L=L)
    b = run(q, w, kg_poison, L=L, perm=[4, 0, 3, 1, 2])
    assert np.array_equal(a, b)
    assert np.all(np.isneginf(a[61:])) and np.all(np.isfinite(a[:61]))


def test_out_of_range_page_scores_minus_inf():
    Hi, Di, G = 8, 64, 32
    kg = np.ones((G, Hi, Di), np.float32)
    kh, pt = khat_from_groups(kg)
    pt = pt.copy()
    pt[0, 1] = 99  # groups 16..31 on an invalid page
    s = oracle.scores([0], [4 * G], np.ones((1, Hi, Di), np.float32),
                      np.ones((1, Hi), np.float32), kh, pt, kh.shape[0], G)[0]
    assert np.all(s[:16] == 64 * 8) and np.all(np.isneginf(s[16:]))


# --- the multi-query indexer form (OrcaRouter article on PR #41855, "Warum QSA
# der heikle Teil ist - in Zahlen": 4 query heads share 1 key head, dim 128)

def test_mqa_equals_per_head_form_with_replicated_key():
    # one shared key head == the per-head form with that key in every head
    rng = np.random.default_rng(11)
    Hi, Di, G = 4, 128, 40
    q = rng.normal(size=(Hi, Di)).astype(np.float32)
    w = rng.uniform(0, 1, Hi).astype(np.float32)
    k1 = rng.normal(size=(G, 1, Di)).astype(np.float32)
    a = run(q, w, k1)
    b = run(q, w, np.repeat(k1, Hi, axis=1))
    assert np.array_equal(a, b)


def test_mqa_one_hot_key_reads_every_query_head():
    # k̂_g = e_{j(g)} shared by all heads  =>  s_g = sum_h w_h max(q_h[j(g)], 0)
    rng = np.random.default_rng(12)
    Hi, Di, G = 4, 128, 64
    q = rng.integers(-4, 5, (Hi, Di)).astype(np.float32)
    w = np.array([0.5, 1.0, 2.0, 4.0], np.float32)
    j = (np.arange(G) * 37) % Di
    kg = np.zeros((G, 1, Di), np.float32)
    kg[np.arange(G), 0, j] = 1.0
    s = run(q, w, kg)[:G]
    want = (np.maximum(q[:, j], 0) * w[:, None]).sum(axis=0)   # exact small integers / 2
    assert np.array_equal(s, want.astype(np.float32))


def test_mqa_relu_keeps_only_aligned_heads():
    # q_h = sign_h * c_h * k (one key for all groups): heads with a negative
    # sign contribute 0, the others w_h c_h |k|^2
    rng = np.random.default_rng(13)
    Di, G = 128, 20
    k = rng.integers(-2, 3, Di).astype(np.float32)
    sign = np.array([1, -1, 1, -1], np.float32)
    c = np.array([1, 2, 3, 4], np.float32)
    q = (sign * c)[:, None] * k[None, :]
    w = np.array([1.0, 1.0, 0.25, 1.0], np.float32)
    kg = np.repeat(k[None, None, :], G, axis=0)
    s = run(q, w, kg)[:G]
    n2 = float(k @ k)
    assert np.all(s == np.float32((1.0 * 1 + 0.25 * 3) * n2))
