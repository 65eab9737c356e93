"""GPU parity of the prefill path: the matrix-core indexer scores (alone,
through qsa_index_score_prefill, and inside qsa_prefill) against the oracle
on bf16-rounded indexer inputs, at small ragged sizes that span several
256-query x 32-group tiles with partial ones, and at the long-prefill chunk
(4,096 queries at positions 28,672 .. 32,767) on sampled query rows."""
import numpy as np
import pytest

import oracle
import workload
from tests import qsa_gpu as H

pytestmark = pytest.mark.gpu


def _scores(wl, gpu):
    import torch
    import learned_sparse_attention_amd as qsa
    d = H.to_dev(wl, gpu)
    sc = qsa.qsa_index_score_prefill(wl.geom, d["khat"], d["pt"], wl.req, wl.first_pos,
                                     d["q_idx"], d["w_idx"], num_pages=wl.num_pages)
    torch.cuda.synchronize()
    return sc.cpu().numpy()


def _check_scores(wl, gs, rows):
    rows = np.asarray(rows)
    gstride = (wl.first_pos + wl.n_q) // 4
    assert gs.shape == (wl.n_q, gstride)
    ora = oracle.scores(wl.row_req[rows], wl.row_len[rows], wl.q_idx[rows], wl.w_idx[rows],
                        wl.khat, wl.page_table, wl.num_pages, gstride, round_bf16_inputs=True)
    G = (wl.row_len[rows] // 4).astype(np.int32)
    H.check_scores(gs[rows], ora, G, H.score_bound(wl, rows=rows, gstride=gstride,
                                                    round_bf16=True))
    return ora, G


# (first_pos, n_q): gstride = (first_pos + n_q) / 4 both a multiple of 4
# (16-byte stores) and not; query counts below, at and past one 256-query tile
@pytest.mark.parametrize("first_pos,n_q", [(3, 5), (100, 31), (1000, 257), (2999, 300),
                                           (5000, 513), (0, 64)])
def test_prefill_scores_ragged(gpu, first_pos, n_q):
    wl = workload.prefill_workload(700 + n_q, first_pos, n_q, idx_bf16_exact=False)
    gs = _scores(wl, gpu)
    _check_scores(wl, gs, np.arange(n_q))


def test_prefill_scores_out_of_range_pages(gpu):
    # page ids outside [0, num_pages) are never read: their groups score -inf
    wl = workload.prefill_workload(720, 2000, 200, idx_bf16_exact=False)
    wl.page_table[0, 5] = wl.num_pages + 7
    wl.page_table[0, 9] = -3
    gs = _scores(wl, gpu)
    _check_scores(wl, gs, np.arange(wl.n_q))
    assert np.all(np.isneginf(gs[:, 5 * 16:6 * 16])) and np.all(np.isneginf(gs[:, 9 * 16:10 * 16]))


def test_prefill_scores_equal_inside_prefill(gpu):
    # the scores qsa_prefill ranks are the ones the scoring entry point returns
    import torch
    wl = workload.prefill_workload(721, 1500, 96, idx_bf16_exact=False)
    gs = _scores(wl, gpu)
    d = H.to_dev(wl, gpu)
    res = H.run_prefill(wl, d)
    torch.cuda.synchronize()
    assert np.array_equal(res["scores"].cpu().numpy(), gs)


def _sample_rows(n_q, seed):
    fixed = [0, 1, 2, 3, 31, 32, 255, 256, 257, 1023, 1024, 2047, 2048, 3071, 3072, 4064, 4093,
             4094, 4095, n_q - 2, n_q - 1]
    rng = np.random.default_rng(seed)
    extra = rng.choice(n_q, 16, replace=False).tolist()
    return np.array(sorted(set(r for r in fixed + extra if 0 <= r < n_q)))


def _prefill_check(wl, gpu, rows):
    """qsa_prefill on the whole chunk; scores, top-K, token lists and
    attention compared with the oracle on `rows`; the -inf mask on every
    row; every output finite."""
    import torch
    d = H.to_dev(wl, gpu)
    res = H.run_prefill(wl, d)
    torch.cuda.synchronize()
    r = oracle.prefill(wl, rows=rows)
    gs = res["scores"].cpu().numpy()
    G = (wl.row_len[rows] // 4).astype(np.int32)
    gstride = (wl.first_pos + wl.n_q) // 4
    H.check_scores(gs[rows], r["scores"], G,
                   H.score_bound(wl, rows=rows, gstride=gstride, round_bf16=True))
    gg = res["groups"].cpu().numpy()[rows]
    K = wl.geom["topk_groups"]
    H.check_topk(gg, gs[rows], r["groups"], r["scores"], G, K)
    gt = res["tokens"].cpu().numpy()[rows]
    W = oracle.token_width(K)
    for i, p in enumerate(rows):
        assert np.array_equal(gt[i], oracle.position_tokens(gg[i], int(wl.row_len[p]), 0, W))
    out = res["out"].cpu().numpy()
    assert np.all(np.isfinite(out))
    ora_o = oracle.attend(wl.geom, wl.row_req[rows], gt, wl.q[rows], wl.k_cache, wl.v_cache,
                          wl.page_table, wl.num_pages)
    H.check_attention(out[rows], ora_o, 0 if wl.geom["kv_dtype"] == 0 else 1)
    # every row's scores, not only the sampled ones: -inf exactly past G
    Gall = wl.row_len // 4
    cols = np.arange(gstride)[None, :]
    assert np.array_equal(np.isneginf(gs), cols >= Gall[:, None])


def test_prefill_long_chunk_sampled(gpu):
    # the long-prefill chunk at full size, in the launch configuration the
    # benchmark times; checked on sampled query rows the oracle computes
    wl = workload.config(4)
    _prefill_check(wl, gpu, _sample_rows(wl.n_q, 4))


def test_prefill_long_7810_queries_over_65536(gpu):
    # the operator suite's long-prefill case (PR #41855 article, Tests):
    # 7,810 queries ending a 65,536-token cache, 2,051 selected slots each
    # (K = 512 groups plus the current block), on sampled rows
    wl = workload.prefill_workload(830, 65536 - 7810, 7810, kv_dtype="bf16", topk_groups=512)
    assert 4 * wl.geom["topk_groups"] + 3 == 2051
    _prefill_check(wl, gpu, _sample_rows(wl.n_q, 5))


@pytest.mark.parametrize("hq,hkv", [(16, 2), (24, 2), (12, 1), (6, 1), (3, 1)])
@pytest.mark.parametrize("n_q,kv", [(1, "fp8"), (257, "bf16")])
def test_prefill_head_shapes(gpu, hq, hkv, n_q, kv):
    # the operator suite's local head shapes at 1 and 257 query rows
    wl = workload.prefill_workload(840 + 7 * hq + hkv + n_q, 2500, n_q, num_q_heads=hq,
                                   num_kv_heads=hkv, kv_dtype=kv, topk_groups=512)
    _prefill_check(wl, gpu, np.arange(n_q))


@pytest.mark.parametrize("first_pos,n_q,K,kv", [
    (4096, 1024, 1024, "bf16"),    # rows of <= 2,048 groups: one wavefront per row
    (24576, 2048, 2048, "fp8"),    # 2,049..8,192 groups: the 256-thread pruned top-K
    (40960, 1024, 1024, "fp8"),    # 8,193..16,384 groups: the 1,024-thread finish kernel
])
def test_prefill_topk_paths_and_budgets(gpu, first_pos, n_q, K, kv):
    wl = workload.prefill_workload(840 + K, first_pos, n_q, kv_dtype=kv, topk_groups=K)
    _prefill_check(wl, gpu, _sample_rows(wl.n_q, 6))
