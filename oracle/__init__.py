"""CPU oracle of the QSA layer step — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it and
shares no code with it.

The arithmetic lives in ``qsa_oracle.c`` (plain loops, binary64).  This
module compiles it, marshals numpy arrays, and composes the four steps in
the order the method is described (indexer score -> exact top-K ->
expansion -> sparse attention), following the "Qwen3.8-27B QSA - BF16 source
weights" model card ("QSA in brief") and the TensorRT-LLM
"QSASparseAttentionConfig" reference (exact top-K, token-level indices,
selection sharing across MTP draft positions).

Parity status: the indexer score follows an ASSUMED form (the pages print
no indexer formula); its pins check the code against that form only.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_oracle.c")
_LIB = os.path.join(_HERE, "libqsa_oracle.so")

PAGE = 64
RATIO = 4


def build() -> str:
    """Compile qsa_oracle.c (C11, -O2, no fast-math, OpenMP)."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                    "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        i32, vp, dbl = ctypes.c_int, ctypes.c_void_p, ctypes.c_double
        L.qo_fp8_e4m3.restype = dbl
        L.qo_fp8_e4m3.argtypes = [ctypes.c_uint8]
        L.qo_bf16.restype = dbl
        L.qo_bf16.argtypes = [ctypes.c_uint16]
        L.qo_round_bf16.restype = ctypes.c_float
        L.qo_round_bf16.argtypes = [ctypes.c_float]
        L.qo_scores.argtypes = [i32, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, i32, i32,
                                i32, i32, vp]
        L.qo_topk.restype = i32
        L.qo_topk.argtypes = [i32, vp, i32, vp, i32, vp]
        L.qo_expand.restype = i32
        L.qo_expand.argtypes = [i32, vp, i32, i32, i32, i32, vp]
        L.qo_attend.argtypes = [i32, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, dbl, dbl, dbl,
                                vp, i32, i32, vp, vp]
        L.qo_num_threads.restype = i32
        L.qo_fp8_e4m3_encode.restype = ctypes.c_uint8
        L.qo_fp8_e4m3_encode.argtypes = [dbl]
        L.qo_append.argtypes = [i32, vp, vp, i32, i32, i32, i32, dbl, dbl, vp, vp, vp, i32, i32,
                                i32, vp, vp, vp, vp, i32, i32, i32, i32]
        _lib = L
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(lib().qo_num_threads())


# --- element formats ------------------------------------------------------

def fp8_e4m3_value(code: int) -> float:
    return float(lib().qo_fp8_e4m3(int(code)))


def fp8_e4m3_encode(x: float) -> int:
    """Nearest E4M3FN code, ties to the even mantissa, saturating at 448."""
    return int(lib().qo_fp8_e4m3_encode(float(x)))


def bf16_value(bits: int) -> float:
    return float(lib().qo_bf16(int(bits)))


def round_bf16(x: float) -> float:
    return float(lib().qo_round_bf16(float(x)))


# --- step 1: indexer scores -----------------------------------------------

def scores(row_req, row_len, q_idx, w_idx, khat, page_table, num_pages, gstride,
           round_bf16_inputs=False) -> np.ndarray:
    """[n_rows, gstride] float32 scores; -inf past each row's complete groups."""
    row_req = _c(row_req, np.int32)
    row_len = _c(row_len, np.int32)
    q_idx = _c(q_idx, np.float32)
    w_idx = _c(w_idx, np.float32)
    khat = _c(khat, np.float32)
    page_table = _c(page_table, np.int32)
    n, Hi, Di = q_idx.shape
    Hk = khat.shape[2]  # key heads of k̂: Hi (per-head form) or 1 (multi-query form)
    assert khat.shape[3] == Di and Hk >= 1 and Hi % Hk == 0
    out = np.empty((n, gstride), np.float32)
    lib().qo_scores(n, _p(row_req), _p(row_len), Hi, Hk, Di, PAGE, RATIO, _p(q_idx), _p(w_idx),
                    _p(khat), _p(page_table), page_table.shape[1], int(num_pages),
                    int(bool(round_bf16_inputs)), int(gstride), _p(out))
    return out


# --- step 2: exact top-K ----------------------------------------------------

def topk(score_rows, row_G, K) -> np.ndarray:
    """[n_rows, K] int32 ascending group ids, -1 padded."""
    s = _c(score_rows, np.float32)
    G = _c(row_G, np.int32)
    out = np.empty((s.shape[0], K), np.int32)
    nan = lib().qo_topk(s.shape[0], _p(G), int(K), _p(s), s.shape[1], _p(out))
    if nan:
        raise ValueError(f"{nan} NaN indexer scores among candidates")
    return out


# --- step 3: expansion ------------------------------------------------------

def token_width(K: int, q_per_req: int = 1) -> int:
    """4K tokens of selected groups + up to 3 + (q_per_req - 1) tail tokens."""
    return RATIO * K + (RATIO - 1) + (q_per_req - 1)


def expand(groups, tail_begin: int, tail_end: int, width: int) -> np.ndarray:
    g = _c(groups, np.int32)
    out = np.empty(width, np.int32)
    n = lib().qo_expand(g.shape[0], _p(g), RATIO, int(tail_begin), int(tail_end), width, _p(out))
    if n < 0:
        raise ValueError("token list exceeds its width")
    return out


def position_tokens(groups, L0: int, j: int, width: int) -> np.ndarray:
    """Tokens of query position j (L_j = L0 + j) sharing the base selection
    S0 = groups: expand(S0), the groups completed since the base position
    and the current partial block, i.e. expand(S0) + [4*floor(L0/4), L0+j)."""
    return expand(groups, RATIO * (L0 // RATIO), L0 + j, width)


# --- step 4: attention ------------------------------------------------------

def attend(geom: dict, row_req, tokens, q, k_cache, v_cache, page_table, num_pages) -> np.ndarray:
    """[n_rows, Hq, D] float64 attention outputs over explicit token lists."""
    row_req = _c(row_req, np.int32)
    tokens = _c(tokens, np.int32)
    q = _c(q, np.uint16)
    page_table = _c(page_table, np.int32)
    kc = np.ascontiguousarray(k_cache)
    vc = np.ascontiguousarray(v_cache)
    n, width = tokens.shape
    Hq, D = geom["num_q_heads"], geom["head_dim"]
    assert q.shape == (n, Hq, D)
    sm = geom["sm_scale"] if geom["sm_scale"] > 0 else 1.0 / math.sqrt(D)
    out = np.empty((n, Hq, D), np.float64)
    lib().qo_attend(n, _p(row_req), _p(tokens), width, Hq, geom["num_kv_heads"], D, PAGE,
                    geom["kv_dtype"], _p(kc), _p(vc), float(np.float32(geom["k_scale"])),
                    float(np.float32(geom["v_scale"])), float(np.float32(sm)), _p(page_table),
                    page_table.shape[1], int(num_pages), _p(q), _p(out))
    return out


# --- composed layer step -----------------------------------------------------

def decode(wl, rows=None) -> dict:
    """Oracle of ``qsa_decode`` on a decode workload.

    S0 = top-K of the base position of each request; position j attends to
    position_tokens(S0, L0, j).  `rows` restricts the computation to a
    subset of requests (outputs for the others are left NaN).
    """
    g = wl.geom
    K = g["topk_groups"]
    B, Q = wl.batch, wl.q_per_req
    sel = np.arange(B) if rows is None else np.asarray(rows)
    s = scores(wl.row_req[sel], wl.row_len[sel], wl.q_idx[sel], wl.w_idx[sel], wl.khat,
               wl.page_table, wl.num_pages, wl.gstride)
    G = np.where((wl.row_len[sel] >= 0) & (wl.row_len[sel] <= wl.max_ctx - (Q - 1)),
                 wl.row_len[sel] // RATIO, 0).astype(np.int32)
    grp = topk(s, G, K)
    W = token_width(K, Q)
    toks = np.full((len(sel), Q, W), -1, np.int32)
    for i, b in enumerate(sel):
        L0 = int(wl.row_len[b])
        if G[i] == 0 and not (0 <= L0 <= wl.max_ctx - (Q - 1)):
            continue
        for j in range(Q):
            toks[i, j] = position_tokens(grp[i], L0, j, W)
    out = attend(g, np.repeat(wl.row_req[sel], Q), toks.reshape(-1, W),
                 wl.q[sel].reshape(-1, g["num_q_heads"], g["head_dim"]), wl.k_cache, wl.v_cache,
                 wl.page_table, wl.num_pages)
    return dict(rows=sel, scores=s, groups=grp, tokens=toks,
                out=out.reshape(len(sel), Q, g["num_q_heads"], g["head_dim"]))


def prefill(wl, rows=None) -> dict:
    """Oracle of ``qsa_prefill``: every query p (L = p + 1) selects its own
    top-K of the groups complete at p, over bf16-rounded indexer inputs."""
    g = wl.geom
    K = g["topk_groups"]
    sel = np.arange(wl.n_q) if rows is None else np.asarray(rows)
    gstride = (wl.first_pos + wl.n_q) // RATIO
    s = scores(wl.row_req[sel], wl.row_len[sel], wl.q_idx[sel], wl.w_idx[sel], wl.khat,
               wl.page_table, wl.num_pages, gstride, round_bf16_inputs=True)
    G = (wl.row_len[sel] // RATIO).astype(np.int32)
    grp = topk(s, G, K)
    W = token_width(K, 1)
    toks = np.stack([position_tokens(grp[i], int(wl.row_len[p]), 0, W) for i, p in enumerate(sel)])
    out = attend(g, wl.row_req[sel], toks, wl.q[sel], wl.k_cache, wl.v_cache, wl.page_table,
                 wl.num_pages)
    return dict(rows=sel, scores=s, groups=grp, tokens=toks, out=out)


def dense(geom, req: int, L: int, q_rows, k_cache, v_cache, page_table, num_pages) -> np.ndarray:
    """Dense causal attention of query rows at length L (all tokens [0, L))."""
    q_rows = np.asarray(q_rows)
    toks = np.tile(np.arange(L, dtype=np.int32), (q_rows.shape[0], 1))
    return attend(geom, np.full(q_rows.shape[0], req, np.int32), toks, q_rows, k_cache, v_cache,
                  page_table, num_pages)


# --- cache append (the "prefill writes" of the KV and k-hat caches) --------

def append_khat_slots(n_tokens: int) -> int:
    """k-hat slots per request of an append: groups completed by n_tokens
    new tokens, at most floor((n_tokens + 3) / 4)."""
    return (n_tokens + RATIO - 1) // RATIO


def append(geom: dict, k_cache, v_cache, khat, page_table, num_pages: int, req_rows, start_pos,
           k_new, v_new, khat_new=None):
    """Write the new tokens' K/V (bf16 [n_req, n, Hkv, D]) and the
    completed groups' k-hat into copies of the caches; returns
    (k_cache, v_cache, khat).  See qo_append."""
    L = lib()
    kc, vc, kh = k_cache.copy(), v_cache.copy(), khat.copy()
    pt = _c(page_table, np.int32)
    rr, sp = _c(req_rows, np.int32), _c(start_pos, np.int32)
    kn, vn = _c(k_new, np.uint16), _c(v_new, np.uint16)
    n_req, n_tok = kn.shape[0], kn.shape[1]
    slots = append_khat_slots(n_tok)
    if khat_new is not None:
        khn = _c(khat_new, np.float32)
        assert khn.shape[:2] == (n_req, slots)
        khp = _p(khn)
    else:
        khp = None
    # the geometry carries the scales as binary32 values
    ks, vs = float(np.float32(geom["k_scale"])), float(np.float32(geom["v_scale"]))
    L.qo_append(n_req, _p(rr), _p(sp), n_tok, geom["num_kv_heads"], geom["head_dim"],
                geom["kv_dtype"], ks, vs, _p(kn), _p(vn), khp, slots,
                kh.shape[2], kh.shape[3], _p(kc), _p(vc), _p(kh), _p(pt), pt.shape[1],
                int(num_pages), PAGE, RATIO)
    return kc, vc, kh
