"""Repeatability of the HIP path: the same inputs give bitwise the same
scores, selections and outputs on every call (no atomics decide a value or
an order), and a decode step captured in a HIP graph (the calls enqueue
kernels only: no allocation, memset or host synchronisation) replays to the
eager result, also after its device inputs change between replays."""
import numpy as np
import pytest

import workload
from tests import qsa_gpu as H

pytestmark = pytest.mark.gpu


def _np(res):
    return {k: v.cpu().numpy() for k, v in res.items() if v is not None}


def test_decode_repeats_bitwise(gpu):
    import torch
    wl = workload.config(2)
    d = H.to_dev(wl, gpu)
    first = _np(H.run_decode(wl, d))
    for _ in range(2):
        again = _np(H.run_decode(wl, d))
        torch.cuda.synchronize()
        for k in first:
            assert np.array_equal(first[k].view(np.uint8), again[k].view(np.uint8)), k


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_prefill_repeats_bitwise(gpu, kv):
    # both element types: scoring, top-K, and attention with one wavefront
    # per (query, KV head)
    import torch
    wl = workload.prefill_workload(950, 3000, 300, kv_dtype=kv, topk_groups=256)
    d = H.to_dev(wl, gpu)
    first = _np(H.run_prefill(wl, d))
    again = _np(H.run_prefill(wl, d))
    torch.cuda.synchronize()
    for k in first:
        assert np.array_equal(first[k].view(np.uint8), again[k].view(np.uint8)), k


def test_decode_graph_replay_matches_eager(gpu):
    import torch
    import learned_sparse_attention_amd as qsa
    wl = workload.decode_workload(951, [4 * 9000 + 1, 4 * 7000 + 2, 4 * 8000], kv_dtype="fp8",
                                  topk_groups=512, max_ctx=4 * 9000 + 4)
    d = H.to_dev(wl, gpu)
    g = wl.geom
    B = wl.batch
    out = torch.empty((B, 1, g["num_q_heads"], g["head_dim"]), dtype=torch.float32, device=gpu)
    ws = torch.empty(qsa.decode_workspace_size(g, B, 1, wl.max_ctx), dtype=torch.uint8,
                     device=gpu)
    ctx = d["ctx"].clone()

    def step():
        return qsa.qsa_decode(g, d["k"], d["v"], d["khat"], d["pt"], ctx, d["q_idx"], d["w_idx"],
                              d["q"], wl.max_ctx, out=out, want_groups=True, workspace=ws,
                              num_pages=wl.num_pages)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = step()
    torch.cuda.synchronize()

    def eager_reference():
        o = torch.empty_like(out)
        w2 = torch.empty_like(ws)
        r = qsa.qsa_decode(g, d["k"], d["v"], d["khat"], d["pt"], ctx, d["q_idx"], d["w_idx"],
                           d["q"], wl.max_ctx, out=o, want_groups=True, workspace=w2,
                           num_pages=wl.num_pages)
        torch.cuda.synchronize()
        return o.cpu().numpy(), r["groups"].cpu().numpy()

    # lengths within what each request has stored
    lengths = [wl.ctx_lens, wl.ctx_lens - 1, np.array([4 * 5000 + 3, 17, 4 * 8000 - 1], np.int32)]
    for rep, lens in enumerate(lengths * 2):
        ctx.copy_(torch.from_numpy(np.ascontiguousarray(lens, np.int32)).to(gpu))
        torch.cuda.synchronize()
        want_o, want_g = eager_reference()        # eager work between the replays
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint8), want_o.view(np.uint8)), rep
        assert np.array_equal(captured["groups"].cpu().numpy(), want_g), rep


def test_prefill_graph_replay_matches_eager(gpu):
    # a BF16 prefill step (scoring, top-K, attention) captured in a HIP
    # graph replays to the eager result, with the query rows changed and
    # eager prefill calls between the replays
    import torch
    import learned_sparse_attention_amd as qsa
    wl = workload.prefill_workload(952, 5000, 300, kv_dtype="bf16", topk_groups=256)
    d = H.to_dev(wl, gpu)
    g = wl.geom
    out = torch.empty((wl.n_q, g["num_q_heads"], g["head_dim"]), dtype=torch.float32, device=gpu)
    total = wl.first_pos + wl.n_q
    ws = torch.empty(qsa.prefill_workspace_size(g, wl.n_q, total), dtype=torch.uint8, device=gpu)
    q = d["q"].clone()

    def step(o, w):
        return qsa.qsa_prefill(g, d["k"], d["v"], d["khat"], d["pt"], 0, wl.first_pos,
                               d["q_idx"], d["w_idx"], q, out=o, want_groups=True, workspace=w,
                               num_pages=wl.num_pages)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out, ws)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = step(out, ws)
    torch.cuda.synchronize()
    for rep in range(4):
        # new query rows for the attention (the selection stays)
        new_q = workload.normal_bf16(952 + rep, 9, (wl.n_q, g["num_q_heads"], g["head_dim"]))
        q.copy_(torch.from_numpy(new_q.view(np.int16)).to(gpu))
        torch.cuda.synchronize()
        o2, w2 = torch.empty_like(out), torch.empty_like(ws)
        want = step(o2, w2)  # eager work between the replays
        torch.cuda.synchronize()
        want_o, want_g = o2.cpu().numpy(), want["groups"].cpu().numpy()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint8), want_o.view(np.uint8)), rep
        assert np.array_equal(captured["groups"].cpu().numpy(), want_g), rep
