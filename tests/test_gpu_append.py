"""GPU parity of the cache append (qsa_append_kv): the paged K/V caches and
the k-hat cache after the append are byte-identical to the oracle's, for
every bf16 input pattern into FP8 and BF16 caches at several scales, for
decode-style and prefill-style appends over random page tables with
out-of-range entries, and the appended tokens feed qsa_decode."""
import numpy as np
import pytest

import oracle
import workload
from tests import qsa_gpu as H
from tests.test_gpu_parity import _decode_check

pytestmark = pytest.mark.gpu


def _run(geom, kc, vc, kh, pt, P, req_rows, start, kn, vn, khn, gpu):
    import torch
    import learned_sparse_attention_amd as qsa
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu)
    dk, dv, dkh, dpt = t(kc), t(vc), t(kh), t(pt)
    qsa.qsa_append_kv(geom, dk, dv, dkh, dpt, t(np.asarray(req_rows, np.int32)),
                      t(np.asarray(start, np.int32)), t(kn.view(np.int16)), t(vn.view(np.int16)),
                      None if khn is None else t(khn), num_pages=P)
    torch.cuda.synchronize()
    return dk.cpu().numpy(), dv.cpu().numpy(), dkh.cpu().numpy()


def _compare(geom, kc, vc, kh, pt, P, req_rows, start, kn, vn, khn, gpu):
    got = _run(geom, kc, vc, kh, pt, P, req_rows, start, kn, vn, khn, gpu)
    want = oracle.append(geom, kc, vc, kh, pt, P, req_rows, start, kn, vn, khn)
    for name, g, w in zip(("k", "v", "khat"), got, want):
        bad = np.argwhere(g.view(np.uint8) != w.view(np.uint8)) if g.dtype != np.float32 else \
            np.argwhere(g.view(np.uint32) != w.view(np.uint32))
        assert bad.size == 0, f"{name} cache differs at {bad[:5].tolist()}"
    return got


def _all_bf16_patterns(geom):
    """128 tokens x [Hkv=2, D=256] holding each of the 65,536 bf16 bit
    patterns once (K ascending, V descending)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    kn = bits.reshape(1, 128, geom["num_kv_heads"], geom["head_dim"])
    vn = bits[::-1].copy().reshape(kn.shape)
    return kn, vn


@pytest.mark.parametrize("kv,scale", [("fp8", 1.0), ("fp8", 0.37), ("fp8", 3.0),
                                      ("bf16", 1.0), ("bf16", 0.5), ("bf16", 0.3)])
def test_append_every_bf16_pattern(gpu, kv, scale):
    geom = workload.geometry(kv_dtype=kv, k_scale=scale, v_scale=scale * 1.5)
    kn, vn = _all_bf16_patterns(geom)
    P = 3
    dt = np.uint8 if kv == "fp8" else np.uint16
    kc = np.full((P, 64, 2, 256), 0x11, dt)
    vc = np.full((P, 64, 2, 256), 0x22, dt)
    kh = np.zeros((P, 16, 8, 64), np.float32)
    pt = np.array([[2, 0]], np.int32)
    _compare(geom, kc, vc, kh, pt, P, [0], [0], kn, vn, None, gpu)


def _random_case(seed, kv, n_req, n_tokens, starts, pages_per_req):
    rng = np.random.default_rng(seed)
    geom = workload.geometry(kv_dtype=kv, k_scale=0.21 if kv == "fp8" else 1.0,
                             v_scale=0.043 if kv == "fp8" else 1.0)
    P = n_req * pages_per_req + 5
    dt = np.uint8 if kv == "fp8" else np.uint16
    kc = rng.integers(0, 0x7E, (P, 64, 2, 256)).astype(dt)
    vc = rng.integers(0, 0x7E, (P, 64, 2, 256)).astype(dt)
    kh = rng.normal(size=(P, 16, 8, 64)).astype(np.float32)
    pt = rng.permutation(P)[:n_req * pages_per_req].reshape(n_req, pages_per_req).astype(np.int32)
    kn = workload.normal_bf16(seed, 1, (n_req, n_tokens, 2, 256))
    vn = workload.normal_bf16(seed, 2, (n_req, n_tokens, 2, 256))
    khn = rng.normal(size=(n_req, oracle.append_khat_slots(n_tokens), 8, 64)).astype(np.float32)
    return geom, kc, vc, kh, pt, P, np.asarray(starts, np.int32), kn, vn, khn


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_append_decode_style(gpu, kv):
    # 8 requests x 3 new tokens at unaligned positions, one starting at a
    # negative position, one page id out of range, one past the page table
    starts = [0, 61, 127, 1000, 4093, -2, 2045, 4 * 16 * 64 - 2]
    geom, kc, vc, kh, pt, P, sp, kn, vn, khn = _random_case(40, kv, 8, 3, starts, 64)
    pt[3, 1000 // 64] = P + 11
    pt[4, 4095 // 64] = -1
    _compare(geom, kc, vc, kh, pt, P, np.arange(8), sp, kn, vn, khn, gpu)


@pytest.mark.parametrize("kv,start,n", [("fp8", 28672, 4096), ("bf16", 3, 4093), ("fp8", 5, 1)])
def test_append_prefill_style(gpu, kv, start, n):
    geom, kc, vc, kh, pt, P, sp, kn, vn, khn = _random_case(41 + n, kv, 1, n, [start],
                                                           (start + n) // 64 + 1)
    _compare(geom, kc, vc, kh, pt, P, [0], sp, kn, vn, khn, gpu)


def test_append_then_decode(gpu):
    # three new tokens appended behind each request's context on the GPU,
    # then a decode step over the grown context reads them
    base = [4 * 700 + 1, 4 * 650]
    wl = workload.decode_workload(42, base, kv_dtype="fp8", topk_groups=128,
                                  max_ctx=max(base) + 3)
    n = 3
    kn = workload.normal_bf16(42, 9, (2, n, 2, 256))
    vn = workload.normal_bf16(42, 10, (2, n, 2, 256))
    khn = workload.normal_f32(42, 11, (2, oracle.append_khat_slots(n), 8, 64))
    start = np.asarray(base, np.int32)
    assert all((b % 64) + n <= 64 for b in base)  # the new tokens stay in allocated pages
    kc, vc, kh = _compare(wl.geom, wl.k_cache, wl.v_cache, wl.khat, wl.page_table, wl.num_pages,
                          np.arange(2), start, kn, vn, khn, gpu)
    wl.k_cache, wl.v_cache, wl.khat = kc, vc, kh
    wl.ctx_lens = start + n
    wl.row_len = wl.ctx_lens.copy()
    wl.stored_lens = wl.ctx_lens.copy()
    _decode_check(wl, gpu)
