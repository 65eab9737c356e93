"""Seeded synthetic QSA workloads.

Builds every input of a QSA layer step (paged K/V caches, the paged
compressed-key cache k̂, page tables, indexer queries and weights, attention
queries) from a seed, in the layouts of the C ABI in ``include/qsa.h``.
Generation is done by ``gen.c`` (SplitMix64 counter streams + Box–Muller);
this module only chooses shapes, lengths and tensor ids.  It holds none of
the method's arithmetic; the oracle and the HIP library both consume its
arrays, and neither imports the other.

Value recipe (shared by every workload):
  q           N(0,1) rounded to bf16                      [rows, Q, Hq, D]
  K, V        N(0,1) as bf16, or as OCP FP8 E4M3 of x/s with a per-tensor
              scale s = amax/448 (separate for K and V)   [P, 64, Hkv, D]
  q_idx, k̂    N(0,1) fp32 (bf16-exact values for prefill workloads)
  w_idx       U(0,1) fp32
  page table  identity, or a seeded Fisher–Yates permutation of the pool
  Unused cache slots (beyond a request's stored length) hold NaN codes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libqsa_workload.so")

# tensor ids of the counter streams
T_QIDX, T_WIDX, T_Q, T_K, T_V, T_KHAT, T_PAGES, T_LENS = 1, 2, 3, 4, 5, 6, 7, 8

PAGE = 64
RATIO = 4
HI, DI = 8, 64
# indexer forms: (query heads, key heads, dims) -- a key per head, or one
# key head shared by 4 query heads of 128 dims (multi-query form)
INDEXER = {"per_head": (8, 8, 64), "mqa": (4, 1, 128)}
HEAD_DIM = 256
CAPACITY = 262_144  # tokens per request (qsa-hisparse offload contract)


def build() -> str:
    """Compile gen.c into libqsa_workload.so (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"],
                   check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        u64, i64, i32, vp, dbl, flt = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_double, ctypes.c_float)
        L.wl_stream_key.restype = u64
        L.wl_stream_key.argtypes = [u64, u64]
        L.wl_fill_normal_f32.argtypes = [u64, i64, vp, ctypes.c_int]
        L.wl_fill_normal_bf16.argtypes = [u64, i64, vp]
        L.wl_fill_uniform_f32.argtypes = [u64, i64, flt, flt, vp]
        L.wl_fill_uniform_int.argtypes = [u64, i64, i32, i32, vp]
        L.wl_permutation.argtypes = [u64, i32, vp]
        L.wl_kv_amax.restype = dbl
        L.wl_kv_amax.argtypes = [u64, ctypes.c_int, vp, ctypes.c_int, ctypes.c_int]
        L.wl_fill_kv_cache.argtypes = [u64, ctypes.c_int, vp, vp, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, dbl, vp]
        L.wl_fill_khat_cache.argtypes = [u64, ctypes.c_int, vp, vp, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
        L.wl_bf16_rne.restype = ctypes.c_uint16
        L.wl_bf16_rne.argtypes = [flt]
        L.wl_fp8_e4m3_rne.restype = ctypes.c_uint8
        L.wl_fp8_e4m3_rne.argtypes = [dbl]
        L.wl_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def key(seed: int, tensor: int) -> int:
    return lib().wl_stream_key(seed & 0xFFFFFFFFFFFFFFFF, tensor)


def normal_f32(seed: int, tensor: int, shape, bf16_exact=False) -> np.ndarray:
    a = np.empty(shape, np.float32)
    lib().wl_fill_normal_f32(key(seed, tensor), a.size, _p(a), int(bf16_exact))
    return a


def normal_bf16(seed: int, tensor: int, shape) -> np.ndarray:
    a = np.empty(shape, np.uint16)
    lib().wl_fill_normal_bf16(key(seed, tensor), a.size, _p(a))
    return a


def uniform_f32(seed: int, tensor: int, shape, lo=0.0, hi=1.0) -> np.ndarray:
    a = np.empty(shape, np.float32)
    lib().wl_fill_uniform_f32(key(seed, tensor), a.size, lo, hi, _p(a))
    return a


def uniform_int(seed: int, tensor: int, n: int, lo: int, hi: int) -> np.ndarray:
    a = np.empty(n, np.int32)
    lib().wl_fill_uniform_int(key(seed, tensor), n, lo, hi, _p(a))
    return a


def permutation(seed: int, tensor: int, n: int) -> np.ndarray:
    a = np.empty(n, np.int32)
    lib().wl_permutation(key(seed, tensor), n, _p(a))
    return a


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    """All inputs of one QSA call plus its geometry.

    kind is "decode" (``qsa_decode``: rows = requests, q_per_req positions
    each) or "prefill" (``qsa_prefill``: one request, n_q consecutive
    queries).  For both, ``row_req``/``row_len`` describe the indexer rows
    (base positions for decode, every query for prefill).
    """
    kind: str
    seed: int
    geom: dict
    batch: int                 # requests (page-table rows)
    q_per_req: int
    ctx_lens: np.ndarray       # decode: L0 per request; prefill: [first_pos + n_q]
    stored_lens: np.ndarray    # tokens present in the cache per request
    max_ctx: int
    page_table: np.ndarray     # [batch, max_pages] int32
    num_pages: int
    k_cache: np.ndarray        # [P, 64, Hkv, D] uint16 (bf16) or uint8 (fp8)
    v_cache: np.ndarray
    khat: np.ndarray           # [P, 16, 8, 64] f32
    q_idx: np.ndarray          # [rows, 8, 64] f32
    w_idx: np.ndarray          # [rows, 8] f32
    q: np.ndarray              # decode [B, Q, Hq, D]; prefill [n_q, Hq, D] uint16
    row_req: np.ndarray        # [rows] int32
    row_len: np.ndarray        # [rows] int32
    first_pos: int = 0
    n_q: int = 0
    req: int = 0
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def n_rows(self) -> int:
        return int(self.row_len.shape[0])

    @property
    def gstride(self) -> int:
        return self.max_ctx // RATIO


def geometry(num_q_heads=16, num_kv_heads=2, topk_groups=512, kv_dtype="bf16",
             sm_scale=0.0, k_scale=1.0, v_scale=1.0, indexer="per_head") -> dict:
    hi, hk, di = INDEXER[indexer]
    return dict(num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=HEAD_DIM,
                page_size=PAGE, compress_ratio=RATIO, idx_heads=hi, idx_dim=di,
                topk_groups=topk_groups, kv_dtype=0 if kv_dtype == "bf16" else 1,
                sm_scale=float(sm_scale), k_scale=float(k_scale), v_scale=float(v_scale),
                idx_key_heads=hk)


def _paged_pool(seed: int, stored: np.ndarray, random_pages: bool, max_pages: int | None = None):
    pages = [(int(L) + PAGE - 1) // PAGE for L in stored]
    total = max(1, sum(pages))
    mp = max_pages if max_pages is not None else max(1, max(pages))
    perm = permutation(seed, T_PAGES, total) if random_pages else np.arange(total, dtype=np.int32)
    pt = np.zeros((len(stored), mp), np.int32)
    off = 0
    for b, n in enumerate(pages):
        pt[b, :n] = perm[off:off + n]
        off += n
    return pt, total


def _caches(seed, geom, stored, pt, num_pages, idx_bf16_exact):
    L = lib()
    B = len(stored)
    Hkv, D = geom["num_kv_heads"], geom["head_dim"]
    stored32 = np.ascontiguousarray(stored, np.int32)
    fp8 = geom["kv_dtype"] == 1
    caches = []
    for tid in (T_K, T_V):
        kk = key(seed, tid)
        if fp8:
            # per-tensor scale amax/448, held as fp32: the same fp32 value is
            # used to encode the codes here and to decode them downstream
            amax = L.wl_kv_amax(kk, B, _p(stored32), Hkv, D)
            scale = float(np.float32(amax / 448.0)) if amax > 0 else 1.0
            c = np.zeros((num_pages, PAGE, Hkv, D), np.uint8)
        else:
            scale = 1.0
            c = np.zeros((num_pages, PAGE, Hkv, D), np.uint16)
        L.wl_fill_kv_cache(kk, B, _p(stored32), _p(pt), pt.shape[1], PAGE, Hkv, D,
                           geom["kv_dtype"], scale, _p(c))
        caches.append((c, scale))
    (kc, ks), (vc, vs) = caches
    geom = dict(geom, k_scale=ks, v_scale=vs)
    gpp = PAGE // RATIO
    hk, di = geom["idx_key_heads"], geom["idx_dim"]
    khat = np.zeros((num_pages, gpp, hk, di), np.float32)
    n_groups = np.ascontiguousarray(stored32 // RATIO, np.int32)
    L.wl_fill_khat_cache(key(seed, T_KHAT), B, _p(n_groups), _p(pt), pt.shape[1], gpp, hk, di,
                         int(idx_bf16_exact), _p(khat))
    return geom, kc, vc, khat


def decode_workload(seed: int, ctx_lens, q_per_req=1, num_q_heads=16, num_kv_heads=2,
                    topk_groups=512, kv_dtype="bf16", random_pages=True, sm_scale=0.0,
                    max_ctx: int | None = None, note="", indexer="per_head") -> Workload:
    """Decode step: request b has L0 = ctx_lens[b] (base position), its
    cache holds L0 + q_per_req - 1 tokens (the draft positions' KV is
    already written)."""
    ctx = np.ascontiguousarray(np.asarray(ctx_lens, np.int32))
    B = len(ctx)
    stored = ctx + (q_per_req - 1)
    geom = geometry(num_q_heads, num_kv_heads, topk_groups, kv_dtype, sm_scale,
                    indexer=indexer)
    hi, di = geom["idx_heads"], geom["idx_dim"]
    mc = int(max_ctx) if max_ctx is not None else int(stored.max())
    mc = max(RATIO, ((mc + RATIO - 1) // RATIO) * RATIO)
    pt, P = _paged_pool(seed, stored, random_pages, max_pages=(mc + PAGE - 1) // PAGE)
    geom, kc, vc, khat = _caches(seed, geom, stored, pt, P, idx_bf16_exact=False)
    q_idx = normal_f32(seed, T_QIDX, (B, hi, di))
    w_idx = uniform_f32(seed, T_WIDX, (B, hi))
    q = normal_bf16(seed, T_Q, (B, q_per_req, num_q_heads, HEAD_DIM))
    return Workload("decode", seed, geom, B, q_per_req, ctx, stored, mc, pt, P, kc, vc, khat,
                    q_idx, w_idx, q, np.arange(B, dtype=np.int32), ctx.copy(), note=note)


def prefill_workload(seed: int, first_pos: int, n_q: int, num_q_heads=16, num_kv_heads=2,
                     topk_groups=512, kv_dtype="bf16", random_pages=True, sm_scale=0.0,
                     idx_bf16_exact=True, note="", indexer="per_head") -> Workload:
    """Chunked prefill of one request: queries at positions first_pos ..
    first_pos + n_q - 1 over a cache holding first_pos + n_q tokens."""
    total = first_pos + n_q
    stored = np.array([total], np.int32)
    geom = geometry(num_q_heads, num_kv_heads, topk_groups, kv_dtype, sm_scale,
                    indexer=indexer)
    hi, di = geom["idx_heads"], geom["idx_dim"]
    mc = ((total + RATIO - 1) // RATIO) * RATIO
    pt, P = _paged_pool(seed, stored, random_pages, max_pages=(mc + PAGE - 1) // PAGE)
    geom, kc, vc, khat = _caches(seed, geom, stored, pt, P, idx_bf16_exact=idx_bf16_exact)
    q_idx = normal_f32(seed, T_QIDX, (n_q, hi, di), bf16_exact=idx_bf16_exact)
    w_idx = uniform_f32(seed, T_WIDX, (n_q, hi))
    q = normal_bf16(seed, T_Q, (n_q, num_q_heads, HEAD_DIM))
    row_len = np.arange(first_pos + 1, first_pos + n_q + 1, dtype=np.int32)
    return Workload("prefill", seed, geom, 1, 1, np.array([total], np.int32), stored, mc, pt, P,
                    kc, vc, khat, q_idx, w_idx, q, np.zeros(n_q, np.int32), row_len,
                    first_pos=first_pos, n_q=n_q, req=0, note=note)


def to_device(wl: Workload, device) -> dict:
    """Copies of a workload's arrays as torch tensors on `device`, keyed by
    the names the binding's callers use (marshalling only: the bf16 query
    bit patterns travel as int16)."""
    import torch

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    return dict(k=t(wl.k_cache), v=t(wl.v_cache), khat=t(wl.khat), pt=t(wl.page_table),
                q_idx=t(wl.q_idx), w_idx=t(wl.w_idx), q=t(wl.q.view(np.int16)),
                ctx=t(wl.ctx_lens), row_req=t(wl.row_req), row_len=t(wl.row_len))


CONFIG_SEED = 0x51A0


def config(i: int, tail: int = 1, instance: int = 0) -> Workload:
    """The five workloads of the QSA layer step (1-based index).

    1  decode, 1 request, L = 8,192 + tail (tail 1..3), BF16 KV,
       identity pages, K = 512 groups, Hq 16 / Hkv 2.
    2  decode, 8 requests, L ~ U{32,768 .. 65,536}, FP8 KV, random pages,
       K = 512.
    3  decode, 8 requests at L = 262,144 (65,536 groups, empty current
       block), FP8 KV, random pages, K = 2,048.
    4  prefill of one request: 4,096 queries at positions 28,672 .. 32,767
       over a 32,768-token cache, BF16 KV, random pages, K = 512,
       bf16-exact indexer inputs.
    5  decode with shared selection, 4 requests, L0 = 131,072 + r0
       (r0 = 1, 2, 3, 1), 3 positions (base + 2 drafts), Hq 24 / Hkv 2,
       FP8 KV, random pages, K = 1,024.

    instance > 0 gives further independent input sets of the same workload
    (other seeds), for timing loops that rotate over several.
    """
    seed = CONFIG_SEED + i + 1000 * instance
    if i == 1:
        return decode_workload(seed, [8192 + tail], kv_dtype="bf16", random_pages=False,
                               topk_groups=512, note=f"cfg1 L=8192+{tail}")
    if i == 2:
        lens = uniform_int(seed, T_LENS, 8, 32768, 65536)
        return decode_workload(seed, lens, kv_dtype="fp8", topk_groups=512,
                               max_ctx=65536, note="cfg2 B8 L~U[32K,64K]")
    if i == 3:
        return decode_workload(seed, [262144] * 8, kv_dtype="fp8", topk_groups=2048,
                               note="cfg3 B8 L=262144")
    if i == 4:
        return prefill_workload(seed, 28672, 4096, kv_dtype="bf16", topk_groups=512,
                                note="cfg4 prefill 4096q @28672")
    if i == 5:
        lens = [131072 + 1 + (b % 3) for b in range(4)]
        return decode_workload(seed, lens, q_per_req=3, num_q_heads=24, num_kv_heads=2,
                               kv_dtype="fp8", topk_groups=1024, note="cfg5 B4 MTP3")
    raise ValueError(i)
