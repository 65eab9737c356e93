"""Python binding of libqsa — one Qwen Sparse Attention (QSA) layer step on
AMD Instinct MI355X (gfx950).

Thin ctypes marshalling over the C ABI in ``include/qsa.h``: every step of
the layer step runs in the HIP kernels of ``libqsa.so``.  PyTorch supplies
device memory (inputs, outputs, workspace) and the current stream; nothing
here computes.  If the library is missing the calls raise: there is no
other execution path.

Functions take the geometry as a dict with the fields of ``qsa_geometry``
and CUDA/HIP tensors in the layouts of the header (non-contiguous tensors
are made contiguous).
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["QSAError", "load", "validate", "token_width", "index_topk_workspace_size",
           "decode_workspace_size", "prefill_workspace_size", "qsa_index_score",
           "qsa_index_score_prefill", "qsa_index_topk", "qsa_decode", "qsa_decode_noalloc",
           "qsa_prefill", "noalloc_scratch_bytes", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqsa.so")

STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported geometry", -3: "workspace",
          -4: "HIP error", -5: "needs more than the static scratch of qsa_decode_noalloc"}


class QSAError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({code})")
        self.code = code


class Geometry(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("compress_ratio", ctypes.c_int32), ("idx_heads", ctypes.c_int32),
                ("idx_dim", ctypes.c_int32), ("topk_groups", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("idx_key_heads", ctypes.c_int32)]


class PagedCache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("khat", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32),
                ("num_pages", ctypes.c_int32)]


_lib = None


def load():
    """Load libqsa.so (built by ``learned_sparse_attention_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m learned_sparse_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        G = ctypes.POINTER(Geometry)
        C = ctypes.POINTER(PagedCache)
        L.qsa_status_string.restype = ctypes.c_char_p
        L.qsa_status_string.argtypes = [ctypes.c_int]
        L.qsa_validate.restype = ctypes.c_int
        L.qsa_validate.argtypes = [G]
        L.qsa_token_width.restype = i32
        L.qsa_token_width.argtypes = [G, i32]
        for n, args in (("qsa_index_topk_workspace_size", [G, i32, i32]),
                        ("qsa_decode_workspace_size", [G, i32, i32, i32]),
                        ("qsa_prefill_workspace_size", [G, i32, i32])):
            f = getattr(L, n)
            f.restype = sz
            f.argtypes = args
        L.qsa_index_score.restype = ctypes.c_int
        L.qsa_index_score.argtypes = [G, C, i32, i32, vp, vp, vp, vp, vp, vp]
        L.qsa_index_score_prefill.restype = ctypes.c_int
        L.qsa_index_score_prefill.argtypes = [G, C, i32, i32, i32, vp, vp, vp, vp]
        L.qsa_index_topk.restype = ctypes.c_int
        L.qsa_index_topk.argtypes = [G, C, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.qsa_decode.restype = ctypes.c_int
        L.qsa_decode.argtypes = [G, C, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.qsa_decode_noalloc.restype = ctypes.c_int
        L.qsa_decode_noalloc.argtypes = [G, C, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.qsa_noalloc_scratch_bytes.restype = sz
        L.qsa_noalloc_scratch_bytes.argtypes = []
        L.qsa_prefill.restype = ctypes.c_int
        L.qsa_prefill.argtypes = [G, C, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.qsa_append_khat_slots.restype = i32
        L.qsa_append_khat_slots.argtypes = [i32]
        L.qsa_append_kv.restype = ctypes.c_int
        L.qsa_append_kv.argtypes = [G, vp, vp, vp, vp, i32, i32, i32, vp, vp, i32, vp, vp, vp, vp]
        _lib = L
    return _lib


def _geom(g: dict) -> Geometry:
    g = dict(g)
    g.setdefault("idx_key_heads", g["idx_heads"])  # per-head form unless stated
    return Geometry(*(int(g[f]) if t is ctypes.c_int32 else float(g[f])
                      for f, t in Geometry._fields_))


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _c(t):
    return None if t is None else t.contiguous()


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(fn: str, code: int):
    if code != 0:
        raise QSAError(fn, code)


def _cache(k, v, khat, page_table, num_pages=None) -> tuple[PagedCache, list]:
    keep = [_c(k), _c(v), _c(khat), _c(page_table)]
    k_, v_, kh_, pt_ = keep
    npg = int(num_pages if num_pages is not None else kh_.shape[0])
    c = PagedCache(None if k_ is None else k_.data_ptr(), None if v_ is None else v_.data_ptr(),
                   kh_.data_ptr(), pt_.data_ptr(), int(pt_.shape[1]), npg)
    return c, keep


def _workspace(nbytes: int, device, workspace=None):
    import torch
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace, workspace.numel() * workspace.element_size()
    # 256-byte aligned (torch's caching allocator returns 512-byte aligned blocks)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, nbytes


def validate(geom: dict) -> int:
    return load().qsa_validate(ctypes.byref(_geom(geom)))


def token_width(geom: dict, q_per_req: int = 1) -> int:
    return load().qsa_token_width(ctypes.byref(_geom(geom)), q_per_req)


def index_topk_workspace_size(geom: dict, n_rows: int, max_ctx: int) -> int:
    return load().qsa_index_topk_workspace_size(ctypes.byref(_geom(geom)), n_rows, max_ctx)


def decode_workspace_size(geom: dict, batch: int, q_per_req: int, max_ctx: int) -> int:
    return load().qsa_decode_workspace_size(ctypes.byref(_geom(geom)), batch, q_per_req, max_ctx)


def prefill_workspace_size(geom: dict, n_q: int, max_ctx: int) -> int:
    return load().qsa_prefill_workspace_size(ctypes.byref(_geom(geom)), n_q, max_ctx)


def qsa_index_score(geom, khat, page_table, row_req, row_len, q_idx, w_idx, max_ctx,
                    out_scores=None, num_pages=None):
    """Indexer scores only (fp32 GEMV).  row_req may be None (row r uses
    page-table row r).  Returns out_scores [n_rows, max_ctx // 4]."""
    import torch
    dev = q_idx.device
    n = int(row_len.shape[0])
    if out_scores is None:
        out_scores = torch.empty((n, max_ctx // 4), dtype=torch.float32, device=dev)
    g = _geom(geom)
    c, keep = _cache(None, None, khat, page_table, num_pages)
    args = [_c(row_req), _c(row_len), _c(q_idx), _c(w_idx)]
    code = load().qsa_index_score(ctypes.byref(g), ctypes.byref(c), n, int(max_ctx),
                                  *(_ptr(t) for t in args), _ptr(out_scores), _stream(dev))
    _check("qsa_index_score", code)
    return out_scores


def qsa_index_score_prefill(geom, khat, page_table, req, first_pos, q_idx, w_idx,
                            out_scores=None, num_pages=None):
    """Indexer scores of a prefill chunk on the matrix cores (bf16 operands,
    fp32 sums).  Query i has L = first_pos + i + 1.  Returns out_scores
    [n_q, (first_pos + n_q) // 4]."""
    import torch
    dev = q_idx.device
    n = int(q_idx.shape[0])
    if out_scores is None:
        out_scores = torch.empty((n, (first_pos + n) // 4), dtype=torch.float32, device=dev)
    g = _geom(geom)
    c, keep = _cache(None, None, khat, page_table, num_pages)
    code = load().qsa_index_score_prefill(ctypes.byref(g), ctypes.byref(c), int(req),
                                          int(first_pos), n, _ptr(_c(q_idx)), _ptr(_c(w_idx)),
                                          _ptr(out_scores), _stream(dev))
    _check("qsa_index_score_prefill", code)
    return out_scores


def qsa_index_topk(geom, khat, page_table, row_req, row_len, q_idx, w_idx, max_ctx,
                   out_groups=None, out_scores=None, want_scores=False, workspace=None,
                   num_pages=None):
    """Indexer scores + exact top-K (fp32).  Returns (groups, scores|None)."""
    import torch
    dev = q_idx.device
    n = int(row_len.shape[0])
    K = int(geom["topk_groups"])
    if out_groups is None:
        out_groups = torch.empty((n, K), dtype=torch.int32, device=dev)
    if out_scores is None and want_scores:
        out_scores = torch.empty((n, max_ctx // 4), dtype=torch.float32, device=dev)
    g = _geom(geom)
    c, keep = _cache(None, None, khat, page_table, num_pages)
    args = [_c(row_req), _c(row_len), _c(q_idx), _c(w_idx)]
    ws, wsb = _workspace(index_topk_workspace_size(geom, n, max_ctx), dev, workspace)
    code = load().qsa_index_topk(ctypes.byref(g), ctypes.byref(c), n, int(max_ctx),
                                 *(_ptr(t) for t in args), _ptr(out_groups), _ptr(out_scores),
                                 _ptr(ws), wsb, _stream(dev))
    _check("qsa_index_topk", code)
    return out_groups, out_scores


def qsa_decode(geom, k_cache, v_cache, khat, page_table, ctx_lens, q_idx, w_idx, q, max_ctx,
               q_per_req=1, out=None, want_groups=False, want_tokens=False, want_scores=False,
               workspace=None, num_pages=None):
    """One decode step.  q: [B, q_per_req, Hq, D] bf16 (or its int16/uint16
    bit pattern).  Returns dict(out, groups, tokens, scores)."""
    import torch
    dev = q.device
    B = int(ctx_lens.shape[0])
    Hq, D = int(geom["num_q_heads"]), int(geom["head_dim"])
    K = int(geom["topk_groups"])
    if out is None:
        out = torch.empty((B, q_per_req, Hq, D), dtype=torch.float32, device=dev)
    groups = torch.empty((B, K), dtype=torch.int32, device=dev) if want_groups else None
    W = token_width(geom, q_per_req)
    tokens = torch.empty((B, q_per_req, W), dtype=torch.int32, device=dev) if want_tokens else None
    scores = (torch.empty((B, max_ctx // 4), dtype=torch.float32, device=dev)
              if want_scores else None)
    g = _geom(geom)
    c, keep = _cache(k_cache, v_cache, khat, page_table, num_pages)
    args = [_c(ctx_lens), _c(q_idx), _c(w_idx), _c(q)]
    ws, wsb = _workspace(decode_workspace_size(geom, B, q_per_req, max_ctx), dev, workspace)
    code = load().qsa_decode(ctypes.byref(g), ctypes.byref(c), B, int(q_per_req), int(max_ctx),
                             *(_ptr(t) for t in args), _ptr(out), _ptr(groups), _ptr(tokens),
                             _ptr(scores), _ptr(ws), wsb, _stream(dev))
    _check("qsa_decode", code)
    return dict(out=out, groups=groups, tokens=tokens, scores=scores)


def noalloc_scratch_bytes() -> int:
    return int(load().qsa_noalloc_scratch_bytes())


def qsa_decode_noalloc(geom, k_cache, v_cache, khat, page_table, ctx_lens, q_idx, w_idx, q,
                       max_ctx, q_per_req=1, out=None, groups=None, tokens=None, scores=None,
                       num_pages=None):
    """qsa_decode without a workspace: the library's static device scratch
    stands in for it.  Every output is caller-supplied (None skips the
    optional lists); the call itself allocates nothing on the device."""
    g = _geom(geom)
    c, keep = _cache(k_cache, v_cache, khat, page_table, num_pages)
    args = [_c(ctx_lens), _c(q_idx), _c(w_idx), _c(q)]
    code = load().qsa_decode_noalloc(ctypes.byref(g), ctypes.byref(c), int(ctx_lens.shape[0]),
                                     int(q_per_req), int(max_ctx), *(_ptr(t) for t in args),
                                     _ptr(out), _ptr(groups), _ptr(tokens), _ptr(scores),
                                     _stream(q.device))
    _check("qsa_decode_noalloc", code)
    return dict(out=out, groups=groups, tokens=tokens, scores=scores)


def qsa_prefill(geom, k_cache, v_cache, khat, page_table, req, first_pos, q_idx, w_idx, q,
                out=None, want_groups=False, want_tokens=False, want_scores=False,
                workspace=None, num_pages=None):
    """Chunked prefill of one request: q [n_q, Hq, D] bf16 bits."""
    import torch
    dev = q.device
    n_q = int(q.shape[0])
    Hq, D = int(geom["num_q_heads"]), int(geom["head_dim"])
    K = int(geom["topk_groups"])
    total = int(first_pos) + n_q
    if out is None:
        out = torch.empty((n_q, Hq, D), dtype=torch.float32, device=dev)
    groups = torch.empty((n_q, K), dtype=torch.int32, device=dev) if want_groups else None
    tokens = (torch.empty((n_q, token_width(geom, 1)), dtype=torch.int32, device=dev)
              if want_tokens else None)
    scores = (torch.empty((n_q, total // 4), dtype=torch.float32, device=dev)
              if want_scores else None)
    g = _geom(geom)
    c, keep = _cache(k_cache, v_cache, khat, page_table, num_pages)
    args = [_c(q_idx), _c(w_idx), _c(q)]
    ws, wsb = _workspace(prefill_workspace_size(geom, n_q, total), dev, workspace)
    code = load().qsa_prefill(ctypes.byref(g), ctypes.byref(c), int(req), int(first_pos), n_q,
                              *(_ptr(t) for t in args), _ptr(out), _ptr(groups), _ptr(tokens),
                              _ptr(scores), _ptr(ws), wsb, _stream(dev))
    _check("qsa_prefill", code)
    return dict(out=out, groups=groups, tokens=tokens, scores=scores)


def append_khat_slots(n_tokens: int) -> int:
    return int(load().qsa_append_khat_slots(int(n_tokens)))


def qsa_append_kv(geom, k_cache, v_cache, khat_cache, page_table, req_rows, start_pos, k_new,
                  v_new, khat_new=None, num_pages=None):
    """Cache append, in place: the new tokens' K/V (bf16 bit patterns
    [n_req, n_tokens, Hkv, D]) are stored in the cache format at positions
    start_pos[r] + i of page-table row req_rows[r]; khat_new (optional,
    [n_req, append_khat_slots(n_tokens), 8, 64] f32) fills the groups those
    tokens complete.  The caches must be contiguous device tensors."""
    for t in (k_cache, v_cache, khat_cache, page_table):
        if t is not None and not t.is_contiguous():
            raise ValueError("caches and page table must be contiguous (written in place)")
    dev = k_new.device
    n_req, n_tok = int(k_new.shape[0]), int(k_new.shape[1])
    npg = int(num_pages if num_pages is not None else k_cache.shape[0])
    g = _geom(geom)
    ins = [_c(req_rows), _c(start_pos), _c(k_new), _c(v_new), _c(khat_new)]
    code = load().qsa_append_kv(ctypes.byref(g), _ptr(k_cache), _ptr(v_cache), _ptr(khat_cache),
                                _ptr(page_table), int(page_table.shape[1]), npg, n_req,
                                _ptr(ins[0]), _ptr(ins[1]), n_tok, _ptr(ins[2]), _ptr(ins[3]),
                                _ptr(ins[4]), _stream(dev))
    _check("qsa_append_kv", code)
