"""GPU parity of the multi-query indexer form (OrcaRouter article on PR
#41855, "Warum QSA der heikle Teil ist - in Zahlen": 4 query heads share one
key head of dimension 128, 512 B of k-hat per group): the decode GEMV and the
prefill matrix-core scoring against the oracle, through the top-K,
expansion and attention of qsa_decode / qsa_prefill, at small ragged sizes,
with out-of-range pages, and at the Flash-Next decode shape (B8 at 262,144
tokens, Hq 24 / Hkv 2, FP8 KV, K = 2,048 groups)."""
import numpy as np
import pytest

import oracle
import workload
from tests import qsa_gpu as H
from tests.test_gpu_parity import _decode_check
from tests.test_gpu_prefill import _prefill_check, _sample_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("lens,K", [([4 * 300 + 1], 64), ([4 * 2048 + 3, 4 * 999 + 2, 17], 512),
                                    ([4 * 20000 + 1, 4 * 16385], 1024)])
def test_mqa_decode(gpu, lens, K):
    wl = workload.decode_workload(900 + len(lens), lens, kv_dtype="fp8", topk_groups=K,
                                  indexer="mqa")
    _decode_check(wl, gpu)


def test_mqa_decode_out_of_range_pages(gpu):
    wl = workload.decode_workload(910, [4 * 3000 + 1, 4 * 2500], kv_dtype="bf16",
                                  topk_groups=256, indexer="mqa")
    wl.page_table[0, 3] = wl.num_pages + 5
    wl.page_table[1, 7] = -1
    _decode_check(wl, gpu)


def test_mqa_index_score_entry_point(gpu):
    import torch
    import learned_sparse_attention_amd as qsa
    wl = workload.decode_workload(911, [4 * 1000 + 2, 61, 4 * 777], kv_dtype="bf16",
                                  indexer="mqa")
    d = H.to_dev(wl, gpu)
    sc = qsa.qsa_index_score(wl.geom, d["khat"], d["pt"], d["row_req"], d["row_len"],
                             d["q_idx"], d["w_idx"], wl.max_ctx, num_pages=wl.num_pages)
    torch.cuda.synchronize()
    ora = oracle.scores(wl.row_req, wl.row_len, wl.q_idx, wl.w_idx, wl.khat, wl.page_table,
                        wl.num_pages, wl.gstride)
    G = (wl.row_len // 4).astype(np.int32)
    H.check_scores(sc.cpu().numpy(), ora, G, H.score_bound(wl))


def test_mqa_decode_flash_next_shape(gpu):
    # the Flash-Next attention shape with its indexer and budget
    wl = workload.decode_workload(912, [262144] * 8, num_q_heads=24, num_kv_heads=2,
                                  kv_dtype="fp8", topk_groups=2048, indexer="mqa")
    _decode_check(wl, gpu)


@pytest.mark.parametrize("first_pos,n_q", [(3, 5), (1000, 257), (2999, 300), (0, 64)])
def test_mqa_prefill_ragged(gpu, first_pos, n_q):
    wl = workload.prefill_workload(920 + n_q, first_pos, n_q, kv_dtype="bf16", topk_groups=128,
                                   indexer="mqa", idx_bf16_exact=False)
    _prefill_check(wl, gpu, np.arange(n_q))


def test_mqa_prefill_long_chunk(gpu):
    wl = workload.prefill_workload(930, 28672, 4096, kv_dtype="bf16", topk_groups=512,
                                   indexer="mqa")
    _prefill_check(wl, gpu, _sample_rows(wl.n_q, 6))
