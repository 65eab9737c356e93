"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
seeded inputs — scores, exact top-K (tie window 1e-6 of the K-th score),
token lists (bit-exact) and attention outputs on the GPU's own selection
(max-abs 2e-3 BF16 KV, 2e-2 FP8 KV)."""
import numpy as np
import pytest

import oracle
import workload
from tests import qsa_gpu as H

pytestmark = pytest.mark.gpu


def _decode_check(wl, gpu):
    import torch
    d = H.to_dev(wl, gpu)
    res = H.run_decode(wl, d)
    torch.cuda.synchronize()
    g = wl.geom
    K, Q = g["topk_groups"], wl.q_per_req
    gs = res["scores"].cpu().numpy()
    gg = res["groups"].cpu().numpy()
    gt = res["tokens"].cpu().numpy()
    go = res["out"].cpu().numpy()
    L0 = wl.ctx_lens
    valid = (L0 >= 0) & (L0 <= wl.max_ctx - (Q - 1))
    G = np.where(valid, L0 // 4, 0).astype(np.int32)
    ora_s = oracle.scores(wl.row_req, wl.row_len, wl.q_idx, wl.w_idx, wl.khat, wl.page_table,
                          wl.num_pages, wl.gstride)
    H.check_scores(gs, ora_s, G, H.score_bound(wl))
    ora_g = oracle.topk(ora_s, G, K)
    H.check_topk(gg, gs, ora_g, ora_s, G, K)
    W = oracle.token_width(K, Q)
    H.check_tokens(gt, gg, L0, W, wl.max_ctx, Q)
    # attention on the GPU's own selection
    toks = gt.reshape(-1, W)
    ora_o = oracle.attend(g, np.repeat(wl.row_req, Q), toks,
                          wl.q.reshape(-1, g["num_q_heads"], g["head_dim"]), wl.k_cache,
                          wl.v_cache, wl.page_table, wl.num_pages)
    return H.check_attention(go.reshape(ora_o.shape), ora_o, g["kv_dtype"])


def test_library_loads_on_gpu(gpu):
    import learned_sparse_attention_amd as qsa
    qsa.load()
    assert qsa.validate(workload.geometry()) == 0


@pytest.mark.parametrize("tail", [1, 2, 3])
def test_decode_small_bf16(gpu, tail):
    wl = workload.decode_workload(201 + tail, [4 * 700 + tail], kv_dtype="bf16", topk_groups=512,
                                  random_pages=True)
    _decode_check(wl, gpu)


@pytest.mark.parametrize("L", [0, 1, 3, 4, 5, 63, 64, 65, 130, 2051])
def test_decode_dense_when_budget_covers_context(gpu, L):
    wl = workload.decode_workload(300 + L, [L, max(L - 1, 0)], kv_dtype="bf16", topk_groups=512)
    _decode_check(wl, gpu)


def test_decode_fp8_random_pages_batch(gpu):
    lens = [5000, 4097, 12345, 8192, 3, 20000]
    wl = workload.decode_workload(77, lens, kv_dtype="fp8", topk_groups=512, max_ctx=20480)
    _decode_check(wl, gpu)


@pytest.mark.parametrize("K", [1, 16, 100, 1024, 2048])
def test_decode_budgets(gpu, K):
    wl = workload.decode_workload(400 + K, [4 * 3000 + 2, 4 * 2500], kv_dtype="fp8", topk_groups=K)
    _decode_check(wl, gpu)


def test_decode_all_scores_tied(gpu):
    # w = 0: every score is +0, so the lowest K group indices are selected
    wl = workload.decode_workload(9, [4 * 1500 + 1], kv_dtype="bf16", topk_groups=512)
    wl.w_idx[:] = 0.0
    _decode_check(wl, gpu)


def test_decode_few_distinct_scores(gpu):
    # integer-valued indexer inputs give many exactly equal scores
    wl = workload.decode_workload(10, [4 * 4000 + 3, 4 * 3000], kv_dtype="bf16", topk_groups=512)
    wl.khat[:] = np.round(wl.khat * 0.7)
    wl.q_idx[:] = np.sign(wl.q_idx)
    wl.w_idx[:] = 1.0
    _decode_check(wl, gpu)


@pytest.mark.parametrize("hq,hkv", [(16, 2), (24, 2), (12, 1), (6, 1), (3, 1)])
def test_decode_mtp_head_shapes(gpu, hq, hkv):
    lens = [4 * 2000 + 1, 4 * 2000 + 2, 4 * 2000 + 3, 4 * 2000]
    wl = workload.decode_workload(500 + hq, lens, q_per_req=3, num_q_heads=hq, num_kv_heads=hkv,
                                  kv_dtype="fp8", topk_groups=1024)
    _decode_check(wl, gpu)


def test_decode_invalid_lengths_give_zero(gpu):
    wl = workload.decode_workload(11, [2000, 2000], kv_dtype="bf16")
    wl.ctx_lens[1] = wl.max_ctx + 5  # out of range: empty selection, zero output
    wl.row_len[1] = wl.ctx_lens[1]
    import torch
    d = H.to_dev(wl, gpu)
    res = H.run_decode(wl, d)
    torch.cuda.synchronize()
    assert np.all(res["out"][1].cpu().numpy() == 0.0)
    assert np.all(res["groups"][1].cpu().numpy() == -1)


def test_fp8_v_conversion_all_codes(gpu):
    # one token whose V row holds every finite E4M3 code: the output is that
    # row exactly (times v_scale), which pins the device FP8 decoder
    wl = workload.decode_workload(12, [1], kv_dtype="fp8", topk_groups=512)
    codes = np.arange(256, dtype=np.uint8)
    codes[codes == 0x7F] = 0
    codes[codes == 0xFF] = 0
    wl.v_cache[0, 0, :, :] = codes[None, :]
    import torch
    d = H.to_dev(wl, gpu)
    out = H.run_decode(wl, d)["out"].cpu().numpy()
    torch.cuda.synchronize()
    want = np.array([oracle.fp8_e4m3_value(c) for c in codes]) * np.float32(wl.geom["v_scale"])
    for h in range(wl.geom["num_q_heads"]):
        np.testing.assert_array_equal(out[0, 0, h].astype(np.float64), want.astype(np.float32))


def test_prefill_small(gpu):
    import torch
    wl = workload.prefill_workload(13, first_pos=3000, n_q=70, kv_dtype="bf16", topk_groups=512)
    d = H.to_dev(wl, gpu)
    res = H.run_prefill(wl, d)
    torch.cuda.synchronize()
    r = oracle.prefill(wl)
    gstride = (wl.first_pos + wl.n_q) // 4
    G = (wl.row_len // 4).astype(np.int32)
    gs = res["scores"].cpu().numpy()
    H.check_scores(gs, r["scores"], G, H.score_bound(wl, gstride=gstride, round_bf16=True))
    gg = res["groups"].cpu().numpy()
    H.check_topk(gg, gs, r["groups"], r["scores"], G, 512)
    gt = res["tokens"].cpu().numpy()
    W = oracle.token_width(512)
    for i in range(wl.n_q):
        assert np.array_equal(gt[i], oracle.position_tokens(gg[i], int(wl.row_len[i]), 0, W))
    ora_o = oracle.attend(wl.geom, wl.row_req, gt, wl.q, wl.k_cache, wl.v_cache, wl.page_table,
                          wl.num_pages)
    H.check_attention(res["out"].cpu().numpy(), ora_o, 0)


def test_index_topk_entry_point(gpu):
    import torch
    import learned_sparse_attention_amd as qsa
    wl = workload.decode_workload(14, [4 * 3000 + 1, 4 * 2999, 40], kv_dtype="bf16",
                                  topk_groups=256)
    d = H.to_dev(wl, gpu)
    grp, sc = qsa.qsa_index_topk(wl.geom, d["khat"], d["pt"], d["row_req"], d["row_len"],
                                 d["q_idx"], d["w_idx"], wl.max_ctx, want_scores=True,
                                 num_pages=wl.num_pages)
    torch.cuda.synchronize()
    ora_s = oracle.scores(wl.row_req, wl.row_len, wl.q_idx, wl.w_idx, wl.khat, wl.page_table,
                          wl.num_pages, wl.gstride)
    G = (wl.row_len // 4).astype(np.int32)
    H.check_scores(sc.cpu().numpy(), ora_s, G, H.score_bound(wl))
    H.check_topk(grp.cpu().numpy(), sc.cpu().numpy(), oracle.topk(ora_s, G, 256), ora_s, G, 256)


@pytest.mark.parametrize("K", [512, 2048])
def test_decode_long_rows_pruned_topk(gpu, K):
    # rows longer than 16,384 groups take the sample-pruned two-step top-K
    lens = [262144, 4 * 17000 + 1, 100003, 70000]
    wl = workload.decode_workload(600 + K, lens, kv_dtype="fp8", topk_groups=K)
    _decode_check(wl, gpu)


def test_decode_long_rows_all_tied(gpu):
    # all scores +0: the pruning threshold keeps every group, the slices
    # overflow and the exact full-row path must pick the lowest K indices
    wl = workload.decode_workload(610, [262144, 200001], kv_dtype="fp8", topk_groups=2048)
    wl.w_idx[:] = 0.0
    _decode_check(wl, gpu)


def test_decode_long_rows_sample_miss(gpu):
    # the evenly spaced sample positions are made the top scorers, so the
    # sample-derived threshold keeps fewer than K groups and the exact
    # full-row path must take over
    wl = workload.decode_workload(611, [262144], kv_dtype="fp8", topk_groups=2048)
    G = 262144 // 4
    gpp = 16
    for i in range(512):
        g = (i * G) // 512
        page = wl.page_table[0, g // gpp]
        wl.khat[page, g % gpp] = 4.0 * wl.q_idx[0]
    _decode_check(wl, gpu)


def test_decode_long_rows_coarse_scores(gpu):
    # scores on a coarse grid: many exact ties at the K-th score
    wl = workload.decode_workload(612, [262144, 150000], kv_dtype="bf16", topk_groups=2048)
    wl.khat[:] = np.round(wl.khat)
    wl.q_idx[:] = np.round(wl.q_idx)
    wl.w_idx[:] = 0.5
    _decode_check(wl, gpu)


# Rows of up to 8,192 groups (prefill queries, shorter decode) take the
# one-workgroup pruned top-K: a sampled guess, candidates compacted into
# LDS, and the whole row ranked instead when the guess misses.

def test_decode_short_rows_sample_miss(gpu):
    # the 512 sample positions of an 8,192-group row are its top scorers,
    # so at K = 1,024 the guess keeps about 100 candidates and the whole-row
    # ranking must take over
    wl = workload.decode_workload(620, [32768, 32768 - 5], kv_dtype="fp8", topk_groups=1024)
    gpp = 16
    for b, L in enumerate(wl.ctx_lens):
        G = int(L) // 4
        for i in range(512):
            g = (i * G) // 512
            page = wl.page_table[b, g // gpp]
            wl.khat[page, g % gpp] = 4.0 * wl.q_idx[b]
    _decode_check(wl, gpu)


def test_decode_short_rows_all_tied(gpu):
    # all scores +0: every group is a candidate, the waves' LDS regions
    # overflow, and the whole-row ranking must keep the lowest K indices
    wl = workload.decode_workload(621, [32768, 20001], kv_dtype="bf16", topk_groups=2048)
    wl.w_idx[:] = 0.0
    _decode_check(wl, gpu)


def test_decode_short_rows_coarse_scores(gpu):
    # scores on a coarse grid: long runs of exact ties at the K-th score
    wl = workload.decode_workload(622, [32768, 24000, 9001], kv_dtype="bf16", topk_groups=512)
    wl.khat[:] = np.round(wl.khat)
    wl.q_idx[:] = np.round(wl.q_idx)
    wl.w_idx[:] = 0.5
    _decode_check(wl, gpu)


def test_decode_short_rows_odd_stride(gpu):
    # a score row stride that is not a multiple of 4 (scalar loads in the
    # short-row top-K), with rows at, just above and well above K groups
    wl = workload.decode_workload(623, [4 * 5001 + 3, 4 * 512, 4 * 513 + 1, 4 * 3000],
                                  kv_dtype="fp8", topk_groups=512)
    assert wl.gstride % 4 != 0
    _decode_check(wl, gpu)


# Rows of up to 2,048 groups take one wavefront each (exact radix select
# over the row's key span, selection emitted from per-lane bit masks).

def test_decode_wave_rows_coarse_scores(gpu):
    # long runs of exact ties at the K-th score
    wl = workload.decode_workload(630, [8192, 6001, 4099], kv_dtype="bf16", topk_groups=512)
    wl.khat[:] = np.round(wl.khat)
    wl.q_idx[:] = np.round(wl.q_idx)
    wl.w_idx[:] = 0.5
    _decode_check(wl, gpu)


def test_decode_wave_rows_all_tied(gpu):
    # every score +0: the lowest K indices
    wl = workload.decode_workload(631, [8192, 5003], kv_dtype="fp8", topk_groups=1024)
    wl.w_idx[:] = 0.0
    _decode_check(wl, gpu)


def test_decode_wave_rows_odd_stride(gpu):
    # a score row stride that is not a multiple of 4 (scalar loads), rows
    # at, just above and well above K groups
    wl = workload.decode_workload(632, [4 * 2001 + 3, 4 * 512, 4 * 513 + 1, 4 * 1500],
                                  kv_dtype="fp8", topk_groups=512)
    assert wl.gstride % 4 != 0 and wl.gstride <= 2048
    _decode_check(wl, gpu)


# Rows of 8,193 to 16,384 groups: the pruned row kernel with 512 threads.

def test_decode_16k_rows_sample_miss(gpu):
    # the sample positions are the top scorers: the guess keeps ~100
    # candidates for K = 1,024 and the whole-row ranking takes over
    wl = workload.decode_workload(640, [65536, 40001], kv_dtype="fp8", topk_groups=1024)
    gpp = 16
    for b, L in enumerate(wl.ctx_lens):
        G = int(L) // 4
        for i in range(512):
            g = (i * G) // 512
            wl.khat[wl.page_table[b, g // gpp], g % gpp] = 4.0 * wl.q_idx[b]
    _decode_check(wl, gpu)


def test_decode_16k_rows_ties_and_pruned(gpu):
    # coarse scores (tie runs at the K-th score) on one row, all scores +0
    # (overflowing candidate regions) on another, normal scores on a third
    wl = workload.decode_workload(641, [65536, 50000, 36001], kv_dtype="bf16", topk_groups=2048)
    for b in (0,):
        pages = wl.page_table[b, :(int(wl.ctx_lens[b]) + 63) // 64]
        wl.khat[pages] = np.round(wl.khat[pages])
    wl.q_idx[0] = np.round(wl.q_idx[0])
    wl.w_idx[1] = 0.0
    _decode_check(wl, gpu)


@pytest.mark.parametrize("K", [1, 7, 100])
@pytest.mark.parametrize("lens", [[8000, 6003], [60000, 40003], [200001]],
                         ids=["wave-rows", "rows-512-threads", "long-rows"])
def test_decode_small_budgets_each_topk_path(gpu, K, lens):
    wl = workload.decode_workload(650 + K, lens, kv_dtype="fp8", topk_groups=K)
    _decode_check(wl, gpu)
