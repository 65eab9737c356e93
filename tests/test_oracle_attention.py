"""Pins of the oracle's sparse attention and composed layer step.

Reference points that do not come from the oracle: torch's CPU
scaled_dot_product_attention (a library routine, fp64, GQA) over K/V that
the test dequantizes itself with torch casts; closed forms (one token,
constant V, zero query); invariances the pages state (page-table
permutation, two requests sharing a prefix, zero output for empty rows)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workload


def dequant(cache: np.ndarray, dtype: int, scale: float) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(cache))
    if dtype == 0:
        v = t.view(torch.int16).view(torch.bfloat16).to(torch.float64)
    else:
        v = t.view(torch.float8_e4m3fn).to(torch.float64)
    return v * float(np.float32(scale))


def gather(wl, req, tokens):
    """[n, Hkv, D] K and V rows of logical tokens of request `req`."""
    tokens = np.asarray(tokens)
    phys = wl.page_table[req, tokens // 64]
    slot = tokens % 64
    g = wl.geom
    K = dequant(wl.k_cache, g["kv_dtype"], g["k_scale"])[phys, slot]
    V = dequant(wl.v_cache, g["kv_dtype"], g["v_scale"])[phys, slot]
    return K, V


def sdpa(q_bits, K, V, geom, mask=None):
    """q_bits [R, Hq, D] bf16 bits, K/V [n, Hkv, D] -> [R, Hq, D] fp64."""
    q = torch.from_numpy(workload.bf16_bits_to_f32(q_bits)).to(torch.float64)
    scale = geom["sm_scale"] if geom["sm_scale"] > 0 else 1.0 / math.sqrt(geom["head_dim"])
    scale = float(np.float32(scale))
    qq = q.permute(1, 0, 2)[None]            # [1, Hq, R, D]
    kk = K.permute(1, 0, 2)[None]            # [1, Hkv, n, D]
    vv = V.permute(1, 0, 2)[None]
    o = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=scale, enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


HEAD_PAIRS = [(16, 2), (24, 2), (12, 1), (6, 1), (3, 1)]


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("L", [1, 5, 63, 64, 65, 130, 1027])
def test_budget_covers_context_equals_dense(kv, L):
    wl = workload.decode_workload(100 + L, [L], kv_dtype=kv, topk_groups=512)
    r = oracle.decode(wl)
    K, V = gather(wl, 0, np.arange(L))
    ref = sdpa(wl.q[0], K, V, wl.geom)
    np.testing.assert_allclose(r["out"][0], ref, rtol=0, atol=1e-12)
    assert int((r["tokens"] >= 0).sum()) == L


@pytest.mark.parametrize("hq,hkv", HEAD_PAIRS)
def test_head_pairs_dense_mtp(hq, hkv):
    L0 = 4 * 37 + 2
    wl = workload.decode_workload(7, [L0, L0 - 5], q_per_req=3, num_q_heads=hq, num_kv_heads=hkv,
                                  kv_dtype="fp8", topk_groups=1024)
    r = oracle.decode(wl)
    for b in range(2):
        for j in range(3):
            Lj = int(wl.ctx_lens[b]) + j
            K, V = gather(wl, b, np.arange(Lj))
            ref = sdpa(wl.q[b, j][None], K, V, wl.geom)[0]
            np.testing.assert_allclose(r["out"][b, j], ref, rtol=0, atol=1e-12)


def test_prefill_dense_causal():
    wl = workload.prefill_workload(9, first_pos=60, n_q=9, topk_groups=512)
    r = oracle.prefill(wl)
    L = wl.first_pos + wl.n_q
    K, V = gather(wl, 0, np.arange(L))
    pos = np.arange(wl.first_pos, L)
    mask = torch.from_numpy(np.arange(L)[None, :] <= pos[:, None])
    ref = sdpa(wl.q, K, V, wl.geom, mask=mask[None, None])
    np.testing.assert_allclose(r["out"], ref, rtol=0, atol=1e-12)


def test_sparse_selection_matches_sdpa_on_selected_tokens():
    wl = workload.decode_workload(21, [4 * 300 + 3], kv_dtype="bf16", topk_groups=64)
    r = oracle.decode(wl)
    toks = r["tokens"][0, 0]
    toks = toks[toks >= 0]
    assert len(toks) == 4 * 64 + 3
    K, V = gather(wl, 0, toks)
    ref = sdpa(wl.q[0], K, V, wl.geom)
    np.testing.assert_allclose(r["out"][0], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("width", [1, 63, 64, 65, 2051])
def test_unordered_physical_slots(width):
    # token lists of the widths the pages test, over a randomly paged cache
    wl = workload.decode_workload(33, [4096], kv_dtype="bf16", topk_groups=512)
    rng = np.random.default_rng(width)
    toks = np.sort(rng.choice(4096, width, replace=False)).astype(np.int32)
    out = oracle.attend(wl.geom, [0], toks[None], wl.q[0, 0][None], wl.k_cache, wl.v_cache,
                        wl.page_table, wl.num_pages)
    K, V = gather(wl, 0, toks)
    np.testing.assert_allclose(out[0], sdpa(wl.q[0, 0][None], K, V, wl.geom)[0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("hq,hkv", HEAD_PAIRS)
@pytest.mark.parametrize("rows", [1, 257])
def test_local_head_shapes(hq, hkv, rows):
    wl = workload.decode_workload(44, [700], num_q_heads=hq, num_kv_heads=hkv, kv_dtype="bf16")
    rng = np.random.default_rng(rows + hq)
    q = workload.normal_bf16(45, 3, (rows, hq, 256))
    toks = np.sort(rng.choice(700, 65, replace=False)).astype(np.int32)
    out = oracle.attend(wl.geom, np.zeros(rows, np.int32), np.tile(toks, (rows, 1)), q,
                        wl.k_cache, wl.v_cache, wl.page_table, wl.num_pages)
    K, V = gather(wl, 0, toks)
    np.testing.assert_allclose(out, sdpa(q, K, V, wl.geom), rtol=0, atol=1e-12)


def test_single_token_constant_v_and_zero_query():
    wl = workload.decode_workload(5, [900], kv_dtype="bf16")
    g = wl.geom
    # one token: the output is that token's V exactly
    out = oracle.attend(g, [0], np.array([[321]], np.int32), wl.q[0, 0][None], wl.k_cache,
                        wl.v_cache, wl.page_table, wl.num_pages)
    K, V = gather(wl, 0, [321])
    kh = np.arange(g["num_q_heads"]) // (g["num_q_heads"] // g["num_kv_heads"])
    assert np.array_equal(out[0], V[0].numpy()[kh])
    # zero query: uniform weights, output = mean of the selected V rows
    toks = np.arange(100, 180, dtype=np.int32)
    qz = np.zeros_like(wl.q[0, 0])[None]
    out = oracle.attend(g, [0], toks[None], qz, wl.k_cache, wl.v_cache, wl.page_table,
                        wl.num_pages)
    K, V = gather(wl, 0, toks)
    np.testing.assert_allclose(out[0], V.numpy().mean(0)[kh], rtol=1e-13, atol=1e-15)
    # constant V: output is that constant whatever the scores
    vc = np.full_like(wl.v_cache, 0x3FC0)  # bf16 1.5
    out = oracle.attend(g, [0], toks[None], wl.q[0, 0][None], wl.k_cache, vc, wl.page_table,
                        wl.num_pages)
    np.testing.assert_allclose(out, 1.5, rtol=1e-14)


def test_empty_rows_are_exact_zero():
    wl = workload.decode_workload(6, [400, 0], kv_dtype="bf16")
    r = oracle.decode(wl)
    assert np.all(r["out"][1] == 0.0)
    assert np.all(r["groups"][1] == -1)
    out = oracle.attend(wl.geom, [0], np.full((1, 8), -1, np.int32), wl.q[0, 0][None],
                        wl.k_cache, wl.v_cache, wl.page_table, wl.num_pages)
    assert np.all(out == 0.0)


def test_page_permutation_invariance():
    a = workload.decode_workload(8, [3000, 2500], kv_dtype="fp8", topk_groups=128,
                                 random_pages=True)
    b = workload.decode_workload(8, [3000, 2500], kv_dtype="fp8", topk_groups=128,
                                 random_pages=False)
    assert not np.array_equal(a.page_table, b.page_table)
    ra, rb = oracle.decode(a), oracle.decode(b)
    assert np.array_equal(ra["groups"], rb["groups"])
    assert np.array_equal(ra["out"], rb["out"])


def test_two_requests_sharing_a_prefix():
    wl = workload.decode_workload(12, [2000, 2000], kv_dtype="bf16", topk_groups=64)
    # request 1 maps its pages onto request 0's physical pages and asks the
    # same query: the physical mapping must not change anything
    wl.page_table[1] = wl.page_table[0]
    wl.q[1] = wl.q[0]
    wl.q_idx[1] = wl.q_idx[0]
    wl.w_idx[1] = wl.w_idx[0]
    r = oracle.decode(wl)
    assert np.array_equal(r["groups"][0], r["groups"][1])
    assert np.array_equal(r["out"][0], r["out"][1])


def test_scales():
    wl = workload.decode_workload(13, [777], kv_dtype="bf16")
    g = wl.geom
    toks = np.arange(0, 777, 3, dtype=np.int32)[None]
    base = oracle.attend(g, [0], toks, wl.q[0, 0][None], wl.k_cache, wl.v_cache, wl.page_table,
                         wl.num_pages)
    g16 = dict(g, sm_scale=1.0 / 16)
    assert np.array_equal(base, oracle.attend(g16, [0], toks, wl.q[0, 0][None], wl.k_cache,
                                              wl.v_cache, wl.page_table, wl.num_pages))
    g2 = dict(g, v_scale=2.0)
    np.testing.assert_allclose(oracle.attend(g2, [0], toks, wl.q[0, 0][None], wl.k_cache,
                                             wl.v_cache, wl.page_table, wl.num_pages),
                               2 * base, rtol=1e-14)
    gk = dict(g, k_scale=2.0)
    gs = dict(g, sm_scale=2.0 / 16)
    np.testing.assert_allclose(
        oracle.attend(gk, [0], toks, wl.q[0, 0][None], wl.k_cache, wl.v_cache, wl.page_table,
                      wl.num_pages),
        oracle.attend(gs, [0], toks, wl.q[0, 0][None], wl.k_cache, wl.v_cache, wl.page_table,
                      wl.num_pages), rtol=1e-12)
    g3 = dict(g, sm_scale=0.3)
    K, V = gather(wl, 0, toks[0])
    np.testing.assert_allclose(
        oracle.attend(g3, [0], toks, wl.q[0, 0][None], wl.k_cache, wl.v_cache, wl.page_table,
                      wl.num_pages)[0], sdpa(wl.q[0, 0][None], K, V, g3)[0], rtol=0, atol=1e-12)
