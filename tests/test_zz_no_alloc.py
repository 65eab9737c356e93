"""qsa_decode_noalloc (the decode entry point that uses the library's static
device scratch instead of a caller workspace) against qsa_decode, through
the C ABI: two calls in a row, the second with a smaller input, each
bitwise equal to qsa_decode on the same inputs; and the size limit."""
import ctypes

import numpy as np
import pytest

import workload
from tests import qsa_gpu as H

pytestmark = pytest.mark.gpu


def _noalloc(wl, d, gpu):
    import torch
    import learned_sparse_attention_amd as qsa
    g = wl.geom
    B, Q, K = wl.batch, wl.q_per_req, g["topk_groups"]
    out = torch.full((B, Q, g["num_q_heads"], g["head_dim"]), float("nan"), device=gpu)
    groups = torch.full((B, K), -7, dtype=torch.int32, device=gpu)
    tokens = torch.full((B, Q, qsa.token_width(g, Q)), -7, dtype=torch.int32, device=gpu)
    scores = torch.full((B, wl.max_ctx // 4), float("nan"), device=gpu)
    return qsa.qsa_decode_noalloc(g, d["k"], d["v"], d["khat"], d["pt"], d["ctx"], d["q_idx"],
                                  d["w_idx"], d["q"], wl.max_ctx, q_per_req=Q, out=out,
                                  groups=groups, tokens=tokens, scores=scores,
                                  num_pages=wl.num_pages)


def test_noalloc_matches_decode_on_two_calls(gpu):
    import torch
    # first call: 8 requests at 262,144 tokens, K = 2,048 (the long-row
    # two-launch top-K); second call: a smaller batch with MTP positions,
    # which leaves the first call's contents in the scratch behind it
    wls = [workload.decode_workload(960, [262144] * 3 + [200001, 150003, 65536, 40001, 9],
                                    kv_dtype="fp8", topk_groups=2048),
           workload.decode_workload(961, [4 * 3000 + 1, 4 * 2000 + 2, 777], q_per_req=3,
                                    num_q_heads=24, kv_dtype="fp8", topk_groups=1024)]
    for wl in wls:
        d = H.to_dev(wl, gpu)
        got = _noalloc(wl, d, gpu)
        torch.cuda.synchronize()
        ref = H.run_decode(wl, d)
        torch.cuda.synchronize()
        for k in ("out", "groups", "tokens", "scores"):
            a, b = got[k].cpu().numpy(), ref[k].cpu().numpy()
            assert a.shape == b.shape, k
            assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  b.view(np.uint32) if b.dtype == np.float32 else b), k


def test_noalloc_refuses_calls_beyond_its_scratch(gpu):
    import torch
    import learned_sparse_attention_amd as qsa
    g = workload.geometry(kv_dtype="fp8", topk_groups=2048)
    cap = qsa.noalloc_scratch_bytes()
    assert cap == 32 << 20
    B = 8
    while qsa.decode_workspace_size(g, B, 1, 262144) <= cap:
        B *= 2
    lib = qsa.load()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: refused on the host
    c = qsa.PagedCache(fake, fake, fake, fake, 4096, 4096)
    gg = qsa._geom(g)
    assert lib.qsa_decode_noalloc(ctypes.byref(gg), ctypes.byref(c), B, 1, 262144,
                                  *([fake] * 5), None, None, None, None) == -5
    assert lib.qsa_decode_noalloc(ctypes.byref(gg), ctypes.byref(c), 0, 1, 262144,
                                  *([None] * 8), None) == 0
    torch.cuda.synchronize()
