"""GPU parity of the prefill path: the matrix-core indexer scores (alone,
through qsa_index_score_prefill, and inside qsa_prefill) against the oracle
on bf16-rounded indexer inputs, at small ragged sizes that span several
256-query x 32-group tiles with partial ones, and at the long-prefill chunk
(4,096 queries at positions 28,672 .. 32,767), the operator suite's
7,810-query case and chunks past 65,536 tokens: scores and top-K on every
query row, attention on sampled rows."""
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


def _prefill_check(wl, gpu, attn_rows, score_rows=None):
    """qsa_prefill on the whole chunk.  Scores and the exact top-K are
    compared with the oracle on `score_rows` (default: every query row),
    token lists on those rows, attention on `attn_rows` (the oracle's
    fp64 attention is the expensive part); the -inf mask and finiteness of
    the outputs on every row fetched."""
    import torch
    d = H.to_dev(wl, gpu)
    res = H.run_prefill(wl, d)
    torch.cuda.synchronize()
    K = wl.geom["topk_groups"]
    gstride = (wl.first_pos + wl.n_q) // 4
    all_rows = score_rows is None
    rows = np.arange(wl.n_q) if all_rows else np.asarray(score_rows)
    if all_rows:
        gs, gg = res["scores"].cpu().numpy(), res["groups"].cpu().numpy()
        gt, out = res["tokens"].cpu().numpy(), res["out"].cpu().numpy()
    else:  # only the checked rows leave the GPU
        ri = torch.from_numpy(rows).to(gpu)
        gs, gg = res["scores"][ri].cpu().numpy(), res["groups"][ri].cpu().numpy()
        gt, out = res["tokens"][ri].cpu().numpy(), res["out"][ri].cpu().numpy()
    del res, d
    G = (wl.row_len[rows] // 4).astype(np.int32)
    ora_s = oracle.scores(wl.row_req[rows], wl.row_len[rows], wl.q_idx[rows], wl.w_idx[rows],
                          wl.khat, wl.page_table, wl.num_pages, gstride, round_bf16_inputs=True)
    H.check_scores(gs, ora_s, G, H.score_bound_matmul(wl, rows, gstride))
    H.check_topk(gg, gs, oracle.topk(ora_s, G, K), ora_s, G, K)
    del ora_s
    W = oracle.token_width(K)
    for i, p in enumerate(rows):
        assert np.array_equal(gt[i], oracle.position_tokens(gg[i], int(wl.row_len[p]), 0, W)), p
    assert np.all(np.isfinite(out))
    # attention on the GPU's own selection, on the sampled rows
    pos = {int(p): i for i, p in enumerate(rows)}
    ai = np.array([pos[int(p)] for p in attn_rows])
    ora_o = oracle.attend(wl.geom, wl.row_req[attn_rows], gt[ai], wl.q[attn_rows], wl.k_cache,
                          wl.v_cache, wl.page_table, wl.num_pages)
    H.check_attention(out[ai], ora_o, 0 if wl.geom["kv_dtype"] == 0 else 1)
    # -inf exactly past each row's complete groups and on groups whose page
    # id is out of range
    cols = np.arange(gstride)
    pages = wl.page_table[wl.req][np.minimum(cols // 16, wl.page_table.shape[1] - 1)]
    bad = (pages < 0) | (pages >= wl.num_pages)
    want = (cols[None, :] >= (wl.row_len[rows] // 4)[:, None]) | bad[None, :]
    assert np.array_equal(np.isneginf(gs), want)
    return gs, gg


def test_prefill_long_chunk_every_row(gpu):
    # the long-prefill chunk at full size, in the launch configuration the
    # benchmark times: scores, top-K and attention on every one of the
    # 4,096 query rows
    wl = workload.config(4)
    _prefill_check(wl, gpu, np.arange(wl.n_q))


def test_prefill_long_7810_queries_over_65536(gpu):
    # the operator suite's long-prefill case (PR #41855 article, Tests):
    # 7,810 queries ending a 65,536-token cache, 2,051 selected slots each
    # (K = 512 groups plus the current block).  Scores, top-K and attention
    # on every row (the article's own test samples rows for the attention).
    # The score rows are 16,384 groups long: the 512-thread row kernel.
    wl = workload.prefill_workload(830, 65536 - 7810, 7810, kv_dtype="bf16", topk_groups=512)
    assert 4 * wl.geom["topk_groups"] + 3 == 2051 and wl.gstride == 16384
    _prefill_check(wl, gpu, np.arange(wl.n_q))


# Score rows longer than 16,384 groups (prefill past 65,536 tokens, up to
# the 262,144-token capacity of the qsa-hisparse offload contract) take the
# two-launch top-K (per-slice extraction, then one workgroup per row).  In
# prefill it runs without the scoring kernel's sample buffer: the guess is
# read from the score rows themselves.

def test_prefill_past_65536_tokens_every_row(gpu):
    # scores, top-K and attention (8,195 tokens each) on every row
    wl = workload.prefill_workload(850, 131072, 1024, kv_dtype="fp8", topk_groups=2048)
    assert (wl.first_pos + wl.n_q) // 4 > 16384
    _prefill_check(wl, gpu, np.arange(wl.n_q))


def test_prefill_past_65536_tokens_k512_bf16(gpu):
    # rows of 15,750 .. 16,749 groups in a 16,750-group stride: the last
    # slice of each row is partial and some rows leave it empty
    wl = workload.prefill_workload(851, 63000, 4000, kv_dtype="bf16", topk_groups=512)
    assert wl.gstride > 16384
    _prefill_check(wl, gpu, _sample_rows(wl.n_q, 8))


def test_prefill_past_65536_tokens_sample_miss(gpu):
    # every query shares one indexer query, and the groups at the evenly
    # spaced guess positions of every row score far above the rest: the
    # guess keeps only those (under K), so each row's exact full-row
    # ranking must take over
    wl = workload.prefill_workload(852, 131072, 8, kv_dtype="fp8", topk_groups=2048)
    wl.q_idx[:] = wl.q_idx[0]
    wl.w_idx[:] = wl.w_idx[0]
    hot = set()
    for L in wl.row_len:
        G = int(L) // 4
        hot |= {(i * G) // 512 for i in range(512)}
    assert len(hot) < 2048
    for g in hot:
        wl.khat[wl.page_table[0, g // 16], g % 16] = 4.0 * wl.q_idx[0]
    _prefill_check(wl, gpu, np.arange(wl.n_q))


def test_prefill_past_65536_tokens_all_tied(gpu):
    # w = 0: every score +0, every slice overflows its candidate area, and
    # each row must keep its lowest K group indices
    wl = workload.prefill_workload(853, 131072, 64, kv_dtype="fp8", topk_groups=2048)
    wl.w_idx[:] = 0.0
    _, gg = _prefill_check(wl, gpu, np.array([0, 31, 63]))
    assert np.array_equal(gg, np.tile(np.arange(2048, dtype=np.int32), (64, 1)))


def test_prefill_rows_of_every_length_past_16384_groups(gpu):
    # one chunk of 65,540 queries from position 0: its score stride is
    # 16,385 groups, so every row takes the two-launch top-K while the rows
    # hold anywhere from 0 to 16,385 groups (rows at or under K = 512
    # groups keep all of them; under 512 groups the guess repeats
    # positions).  Checked on sampled rows, which alone are copied back.
    wl = workload.prefill_workload(854, 0, 65540, kv_dtype="fp8", topk_groups=512)
    assert wl.gstride == 16385
    rows = np.array(sorted({0, 1, 2, 3, 4, 7, 100, 511, 2047, 2048, 2051, 2052, 4096, 8191,
                            8192, 12000, 20000, 32767, 40000, 50000, 60000, 65535, 65536,
                            65537, 65538, 65539}))
    _prefill_check(wl, gpu, rows[::3], score_rows=rows)


@pytest.mark.parametrize("hq,hkv", [(16, 2), (24, 2), (12, 1), (6, 1), (3, 1), (16, 1)])
@pytest.mark.parametrize("n_q,kv", [(1, "fp8"), (257, "bf16")])
def test_prefill_head_shapes(gpu, hq, hkv, n_q, kv):
    # the operator suite's local head shapes at 1 and 257 query rows, and
    # the widest group (16 query heads per KV head: the output rows then
    # take two LDS passes); one KV head spreads its queries over all 8 XCDs
    wl = workload.prefill_workload(840 + 7 * hq + hkv + n_q, 2500, n_q, num_q_heads=hq,
                                   num_kv_heads=hkv, kv_dtype=kv, topk_groups=512)
    _prefill_check(wl, gpu, np.arange(n_q))


@pytest.mark.parametrize("first_pos,n_q,K,kv", [
    (4096, 1024, 1024, "bf16"),    # score stride <= 2,048 groups: one wavefront per row
    (24576, 2048, 2048, "fp8"),    # 2,049..8,192 groups: the 256-thread pruned row kernel
    (40960, 1024, 1024, "fp8"),    # 8,193..16,384 groups: the 512-thread pruned row kernel
])
def test_prefill_topk_paths_and_budgets(gpu, first_pos, n_q, K, kv):
    wl = workload.prefill_workload(840 + K, first_pos, n_q, kv_dtype=kv, topk_groups=K)
    _prefill_check(wl, gpu, _sample_rows(wl.n_q, 6))


@pytest.mark.parametrize("hq,hkv,kv", [(24, 3, "bf16"), (16, 4, "fp8"), (16, 8, "bf16"),
                                        (32, 16, "fp8")])
def test_prefill_kv_head_counts(gpu, hq, hkv, kv):
    # KV head counts that divide the 8 XCDs (4, 8: each XCD serves one head)
    # and that do not (3, 16: workgroups in plain (query block, head) order)
    wl = workload.prefill_workload(880 + hq + hkv, 2500, 257, num_q_heads=hq, num_kv_heads=hkv,
                                   kv_dtype=kv, topk_groups=512)
    _prefill_check(wl, gpu, np.arange(wl.n_q))


@pytest.mark.parametrize("K,first_pos", [(256, 4095), (256, 4092), (255, 4095), (257, 4093)])
def test_prefill_translation_step_edges(gpu, K, first_pos):
    # token streams of 4K + (L mod 4) entries ending on, just before and just
    # past a 1,024-entry translation step (the K prefetch past a step's last
    # sub-tile then reads the step's padding entries)
    wl = workload.prefill_workload(890 + K + first_pos % 4, first_pos, 9, kv_dtype="bf16",
                                   topk_groups=K)
    lens = first_pos + np.arange(wl.n_q) + 1
    streams = 4 * K + lens % 4  # 1,020-1,031 entries over the cases
    assert np.all((streams >= 1020) & (streams <= 1031))
    _prefill_check(wl, gpu, np.arange(wl.n_q))


# Prefill attention walks each query's whole selection in token order, one
# wavefront per (query, KV head); the cases below stress the token stream:
# few selected groups, the longest selections at full capacity, and
# selections piled into one 8,192-token region that every query reads.

@pytest.mark.parametrize("K", [1, 7, 100])
def test_prefill_small_budgets(gpu, K):
    wl = workload.prefill_workload(860 + K, 20000, 300, kv_dtype="bf16", topk_groups=K)
    _prefill_check(wl, gpu, np.arange(wl.n_q))


def test_prefill_at_full_capacity(gpu):
    # 64 queries ending a 262,144-token request, 2,048 groups each
    wl = workload.prefill_workload(863, 262144 - 64, 64, kv_dtype="bf16", topk_groups=2048)
    assert wl.first_pos + wl.n_q == 262144
    _prefill_check(wl, gpu, np.arange(wl.n_q))


def test_prefill_selection_in_one_region(gpu):
    # every query shares one indexer query, and the groups of tokens
    # 16,384 .. 24,575 score far above the rest: each selection lies wholly
    # in that region, then comes the query's current block
    wl = workload.prefill_workload(864, 30000, 96, kv_dtype="bf16", topk_groups=512)
    wl.q_idx[:] = wl.q_idx[0]
    wl.w_idx[:] = wl.w_idx[0]
    for g in range(16384 // 4, 24576 // 4):
        wl.khat[wl.page_table[0, g // 16], g % 16] = 4.0 * wl.q_idx[0]
    _, gg = _prefill_check(wl, gpu, np.arange(wl.n_q))
    assert np.all((gg >= 16384 // 4) & (gg < 24576 // 4))


def _paced_regime(wl):
    # the library paces a BF16 or FP8 chunk's sweep when G / sqrt(n) groups
    # of one KV head's K and V (4 tokens x 256 dims x 2 for K and V, x2
    # bytes for BF16) exceed 1 MiB and every query keeps n >= 128 groups
    G = (wl.first_pos + wl.n_q) / 4
    n = min(wl.geom["topk_groups"], G)
    gb = 2 * 4 * 256 * (1 if wl.geom["kv_dtype"] == 1 else 2)
    return n >= 128 and G / np.sqrt(n) * gb > (1 << 20)


def test_prefill_paced_sweep_every_row(gpu):
    # a BF16 chunk in the paced regime with a ragged query count: scores,
    # top-K and attention on every row, then a second call bitwise equal
    # (the waits change timing only)
    import torch
    wl = workload.prefill_workload(861, 16384, 203, kv_dtype="bf16", topk_groups=128)
    assert _paced_regime(wl)
    _prefill_check(wl, gpu, np.arange(wl.n_q))
    d = H.to_dev(wl, gpu)
    a = H.run_prefill(wl, d)["out"].clone()
    b = H.run_prefill(wl, d)["out"]
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("hq,hkv,kv", [(24, 3, "bf16"), (12, 1, "bf16"), (16, 2, "fp8")])
def test_prefill_paced_sweep_head_layouts(gpu, hq, hkv, kv):
    # the paced sweep with 3 KV heads (the workgroups take the plain order,
    # 8 XCDs not being a multiple of 3), with 12 query heads on one KV head,
    # and over an FP8 cache (its rows are half the bytes, so it needs a
    # longer context to reach the paced regime); every row checked
    n_q = 77
    first_pos = 16384 if kv == "bf16" else 65536
    wl = workload.prefill_workload(870 + hq + hkv, first_pos, n_q, num_q_heads=hq,
                                   num_kv_heads=hkv, kv_dtype=kv, topk_groups=128)
    assert _paced_regime(wl)
    _prefill_check(wl, gpu, np.arange(wl.n_q))
