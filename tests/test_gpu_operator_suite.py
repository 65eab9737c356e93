"""GPU parity on the remaining cases of the operator suite described in the
OrcaRouter article on SGLang PR #41855 ("Neun bestandene Tests und eine
Geschwindigkeitszahl ..."): default and explicit softmax scales,
non-contiguous tensors, the physical mapping of two requests that share a
prefix, cache-content reuse, zero query rows, selection width zero and
fully masked rows (exact zeros).  Every case runs through the C ABI and is
compared with the oracle."""
import ctypes

import numpy as np
import pytest

import oracle
import workload
from tests import qsa_gpu as H
from tests.test_gpu_parity import _decode_check
from tests.test_gpu_prefill import _prefill_check

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_explicit_scale_decode(gpu, kv):
    # an explicit softmax scale (0.3) instead of the default 1/sqrt(256)
    wl = workload.decode_workload(900, [4 * 3000 + 1, 4 * 2100 + 3], kv_dtype=kv,
                                  topk_groups=512, sm_scale=0.3)
    assert wl.geom["sm_scale"] == pytest.approx(0.3)
    _decode_check(wl, gpu)


def test_explicit_scale_prefill(gpu):
    wl = workload.prefill_workload(901, 3000, 70, kv_dtype="bf16", topk_groups=512,
                                   sm_scale=0.3)
    _prefill_check(wl, gpu, np.arange(wl.n_q))


def test_default_scale_is_one_over_sqrt_head_dim(gpu):
    # sm_scale <= 0 selects 1/sqrt(256) = 1/16: bitwise the explicit value
    import torch
    outs = []
    for sm in (0.0, -1.0, 1.0 / 16):
        wl = workload.decode_workload(902, [4 * 1200 + 2], kv_dtype="fp8", topk_groups=512,
                                      sm_scale=sm)
        outs.append(H.run_decode(wl, H.to_dev(wl, gpu))["out"].cpu().numpy())
    torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def _strided_copy(t, pad_last):
    """The same values as `t` in a non-contiguous view (a slice of a wider
    buffer)."""
    import torch
    wide = torch.zeros((*t.shape[:-1], t.shape[-1] + pad_last), dtype=t.dtype, device=t.device)
    wide[..., :t.shape[-1]] = t
    v = wide[..., :t.shape[-1]]
    assert not v.is_contiguous()
    return v


def test_non_contiguous_tensors(gpu):
    # q, q_idx, w_idx, the lengths and the page table passed as strided
    # views give bitwise the result of the contiguous tensors
    import torch
    import learned_sparse_attention_amd as qsa
    wl = workload.decode_workload(903, [4 * 2000 + 1, 4 * 1500 + 2, 777], kv_dtype="fp8",
                                  topk_groups=256)
    d = H.to_dev(wl, gpu)
    ref = H.run_decode(wl, d)
    nd = dict(d)
    for k in ("q", "q_idx", "w_idx", "pt"):
        nd[k] = _strided_copy(d[k], 3)
    nd["ctx"] = torch.stack([d["ctx"], d["ctx"]], 1)[:, 0]
    assert not nd["ctx"].is_contiguous()
    got = H.run_decode(wl, nd)
    torch.cuda.synchronize()
    for k in ("out", "groups", "tokens", "scores"):
        assert torch.equal(ref[k], got[k]), k
    # prefill with strided q / q_idx
    pw = workload.prefill_workload(904, 1000, 40, kv_dtype="bf16", topk_groups=128)
    pd = H.to_dev(pw, gpu)
    pref = H.run_prefill(pw, pd)
    npd = dict(pd, q=_strided_copy(pd["q"], 5), q_idx=_strided_copy(pd["q_idx"], 1))
    pgot = H.run_prefill(pw, npd)
    torch.cuda.synchronize()
    for k in ("out", "groups", "tokens", "scores"):
        assert torch.equal(pref[k], pgot[k]), k
    del qsa


def test_two_requests_sharing_a_prefix(gpu):
    # request 1's page table maps its first 40 pages onto request 0's
    # physical pages (a shared prefix) and asks the same query; past the
    # prefix each request has its own pages.  Both match the oracle, and
    # the shared-prefix mapping itself changes nothing: with the whole
    # table shared, the two outputs are bitwise equal.
    wl = workload.decode_workload(905, [4 * 16 * 60 + 1, 4 * 16 * 60 + 1], kv_dtype="bf16",
                                  topk_groups=512)
    wl.page_table[1, :40] = wl.page_table[0, :40]
    for a in (wl.q, wl.q_idx, wl.w_idx):
        a[1] = a[0]
    _decode_check(wl, gpu)
    import torch
    wl.page_table[1] = wl.page_table[0]
    res = H.run_decode(wl, H.to_dev(wl, gpu))
    torch.cuda.synchronize()
    out, grp = res["out"].cpu().numpy(), res["groups"].cpu().numpy()
    assert np.array_equal(grp[0], grp[1]) and np.array_equal(out[0], out[1])
    _decode_check(wl, gpu)


def test_cache_content_reuse(gpu):
    # the step only reads the caches: their bytes are unchanged after a
    # call, and a second call over the same cache contents (here by a
    # request mapped onto the first one's pages) reproduces the first
    import torch
    wl = workload.decode_workload(906, [4 * 5000 + 3], kv_dtype="fp8", topk_groups=1024)
    d = H.to_dev(wl, gpu)
    before = [d[k].clone() for k in ("k", "v", "khat", "pt")]
    r1 = H.run_decode(wl, d)
    r2 = H.run_decode(wl, d)
    torch.cuda.synchronize()
    for b, k in zip(before, ("k", "v", "khat", "pt")):
        # compared as bytes: unused cache slots hold NaN on purpose
        assert torch.equal(b.view(torch.uint8), d[k].view(torch.uint8)), k
    for k in ("out", "groups", "tokens", "scores"):
        assert torch.equal(r1[k], r2[k]), k
    _decode_check(wl, gpu)


def test_zero_query_rows(gpu):
    # zero query rows (batch 0 / chunk of 0 queries / 0 indexer rows): the
    # call succeeds and writes nothing
    import torch
    import learned_sparse_attention_amd as qsa
    wl = workload.decode_workload(907, [900], kv_dtype="bf16", topk_groups=128)
    d = H.to_dev(wl, gpu)
    g = qsa._geom(wl.geom)
    c, keep = qsa._cache(d["k"], d["v"], d["khat"], d["pt"], wl.num_pages)
    sentinel = torch.full((4, 16, 256), 7.0, dtype=torch.float32, device=gpu)
    grp = torch.full((4, 128), 5, dtype=torch.int32, device=gpu)
    lib = qsa.load()
    stream = qsa._stream(gpu)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    assert lib.qsa_decode(ctypes.byref(g), ctypes.byref(c), 0, 1, wl.max_ctx, p(d["ctx"]),
                          p(d["q_idx"]), p(d["w_idx"]), p(d["q"]), p(sentinel), p(grp), None,
                          None, None, 0, stream) == 0
    assert lib.qsa_prefill(ctypes.byref(g), ctypes.byref(c), 0, 100, 0, p(d["q_idx"]),
                           p(d["w_idx"]), p(d["q"]), p(sentinel), p(grp), None, None, None, 0,
                           stream) == 0
    assert lib.qsa_index_topk(ctypes.byref(g), ctypes.byref(c), 0, wl.max_ctx, p(d["row_req"]),
                              p(d["row_len"]), p(d["q_idx"]), p(d["w_idx"]), p(grp), None, None,
                              0, stream) == 0
    torch.cuda.synchronize()
    assert torch.all(sentinel == 7.0) and torch.all(grp == 5)
    # through the binding: empty outputs, no error
    pw = workload.prefill_workload(908, 500, 1, kv_dtype="bf16", topk_groups=128)
    pd = H.to_dev(pw, gpu)
    res = qsa.qsa_prefill(pw.geom, pd["k"], pd["v"], pd["khat"], pd["pt"], 0, 500,
                          pd["q_idx"][:0], pd["w_idx"][:0], pd["q"][:0], want_groups=True,
                          num_pages=pw.num_pages)
    torch.cuda.synchronize()
    assert res["out"].shape == (0, 16, 256) and res["groups"].shape == (0, 128)


def test_selection_width_zero_in_a_batch(gpu):
    # a request at L0 = 0 selects nothing (width 0): its output is exactly
    # zero and its lists are all -1, beside requests with full selections
    import torch
    wl = workload.decode_workload(909, [0, 4 * 1500 + 2, 0, 4 * 700 + 3], kv_dtype="fp8",
                                  topk_groups=512)
    _decode_check(wl, gpu)
    res = H.run_decode(wl, H.to_dev(wl, gpu))
    torch.cuda.synchronize()
    for b in (0, 2):
        assert np.all(res["out"][b].cpu().numpy() == 0.0)
        assert np.all(res["groups"][b].cpu().numpy() == -1)
        assert np.all(res["tokens"][b].cpu().numpy() == -1)


def test_fully_masked_prefill_rows_are_exact_zero(gpu):
    # every page id of the request out of range: no selected token can be
    # read, so every query row is fully masked and outputs exact zeros
    # (the zero-output convention for fully masked rows); its scores are
    # all -inf and the oracle agrees
    wl = workload.prefill_workload(910, 700, 50, kv_dtype="bf16", topk_groups=64)
    wl.page_table[0, :] = wl.num_pages + np.arange(wl.page_table.shape[1])
    gs, _ = _prefill_check(wl, gpu, np.arange(wl.n_q))
    assert np.all(np.isneginf(gs))
    import torch
    res = H.run_prefill(wl, H.to_dev(wl, gpu))
    torch.cuda.synchronize()
    assert np.all(res["out"].cpu().numpy() == 0.0)


def test_partly_masked_prefill_rows(gpu):
    # some pages out of range, including the one holding the chunk's last
    # queries: their groups never score, their tokens are skipped, and rows
    # whose every selected token is masked output exact zeros
    wl = workload.prefill_workload(911, 1200, 100, kv_dtype="fp8", topk_groups=64)
    wl.page_table[0, 3] = -1
    wl.page_table[0, 7] = wl.num_pages + 2
    wl.page_table[0, (wl.first_pos + wl.n_q - 1) // 64] = -5
    _prefill_check(wl, gpu, np.arange(wl.n_q))
    r = oracle.prefill(wl, rows=[0])
    assert np.all(np.isfinite(r["out"]))
