"""Helpers of the GPU parity tests: move a seeded workload to the device,
run the HIP library through its binding, and compare with the oracle."""
from __future__ import annotations

import numpy as np

import oracle
import workload

TIE_REL = 1e-6          # top-K: members may differ only within 1e-6 of the K-th score
ATOL = {0: 2e-3, 1: 2e-2}  # attention max-abs, BF16 KV / FP8 KV


to_dev = workload.to_device


def run_decode(wl, dev_inputs, **kw):
    import learned_sparse_attention_amd as qsa
    d = dev_inputs
    return qsa.qsa_decode(wl.geom, d["k"], d["v"], d["khat"], d["pt"], d["ctx"], d["q_idx"],
                          d["w_idx"], d["q"], wl.max_ctx, q_per_req=wl.q_per_req,
                          want_groups=True, want_tokens=True, want_scores=True,
                          num_pages=wl.num_pages, **kw)


def run_prefill(wl, dev_inputs, **kw):
    import learned_sparse_attention_amd as qsa
    d = dev_inputs
    return qsa.qsa_prefill(wl.geom, d["k"], d["v"], d["khat"], d["pt"], wl.req, wl.first_pos,
                           d["q_idx"], d["w_idx"], d["q"], want_groups=True, want_tokens=True,
                           want_scores=True, num_pages=wl.num_pages, **kw)


def score_bound(wl, rows=None, gstride=None, round_bf16=False) -> np.ndarray:
    """Magnitude sum_h |w_h| sum_d |q_hd k_ghd| of each score (the oracle
    run on absolute values): fp32 accumulation error is a small multiple of
    2^-24 times this."""
    sel = np.arange(wl.n_rows) if rows is None else np.asarray(rows)
    gs = wl.gstride if gstride is None else gstride
    return oracle.scores(wl.row_req[sel], wl.row_len[sel], np.abs(wl.q_idx[sel]),
                         np.abs(wl.w_idx[sel]), np.abs(wl.khat), wl.page_table, wl.num_pages, gs,
                         round_bf16_inputs=round_bf16)


def score_bound_matmul(wl, rows, gstride, chunk=1024) -> np.ndarray:
    """The same magnitude as score_bound, sum_h |w_h| sum_d |q_hd k_ghd|,
    for many rows at once: per-head binary64 matrix products (numpy) of the
    absolute values, with k̂ gathered in logical group order through the
    page table (groups on out-of-range pages get 0; their scores are -inf).
    Rounding the inputs to bf16 changes a magnitude by under 2^-8
    relative, which the factor 1.01 covers."""
    rows = np.asarray(rows)
    Hi, Di = wl.q_idx.shape[1:]
    Hk = wl.khat.shape[2]
    gpp = wl.khat.shape[1]
    out = np.zeros((len(rows), gstride))
    for req in np.unique(wl.row_req[rows]):
        idx = np.flatnonzero(wl.row_req[rows] == req)
        npg = min(wl.page_table.shape[1], (gstride + gpp - 1) // gpp)
        pages = wl.page_table[req, :npg]
        ok = (pages >= 0) & (pages < wl.num_pages)
        kabs = np.zeros((npg, gpp, Hk, Di))
        kabs[ok] = np.abs(wl.khat[pages[ok]])
        kabs = kabs.reshape(npg * gpp, Hk, Di)[:gstride]
        for c0 in range(0, len(idx), chunk):
            sel = idx[c0:c0 + chunk]
            q = np.abs(wl.q_idx[rows[sel]].astype(np.float64))
            w = np.abs(wl.w_idx[rows[sel]].astype(np.float64))
            acc = np.zeros((len(sel), kabs.shape[0]))
            for h in range(Hi):
                acc += w[:, h:h + 1] * (q[:, h, :] @ kabs[:, h * Hk // Hi, :].T)
            out[sel, :kabs.shape[0]] = acc
    return 1.01 * out


def check_scores(gpu_scores: np.ndarray, ora_scores: np.ndarray, G: np.ndarray,
                 bound: np.ndarray):
    """fp32 scores within fp32 accumulation error of the binary64 oracle on
    candidates (|err| <= 80 * 2^-24 * magnitude: 64 products per head, 8
    heads); -inf past each row's complete groups."""
    for r in range(gpu_scores.shape[0]):
        g = int(G[r])
        a, b = gpu_scores[r, :g].astype(np.float64), ora_scores[r, :g].astype(np.float64)
        tol = 80 * 2.0 ** -24 * bound[r, :g].astype(np.float64) + 1e-30
        with np.errstate(invalid="ignore"):  # -inf - -inf on out-of-range pages
            bad = np.flatnonzero(~((a == b) | (np.abs(a - b) <= tol)))
        assert bad.size == 0, f"row {r}: score mismatch at {bad[:5]} gpu={a[bad[:5]]} ora={b[bad[:5]]}"
        assert np.all(np.isneginf(gpu_scores[r, g:])), f"row {r}: masked columns not -inf"


def check_topk(gpu_groups: np.ndarray, gpu_scores: np.ndarray, ora_groups: np.ndarray,
               ora_scores: np.ndarray, G: np.ndarray, K: int):
    """Top-K parity: (1) the GPU selection is exactly the top-K of the
    GPU's own fp32 scores (bit-exact, lowest-index ties); (2) against the
    oracle's selection it differs only in groups whose oracle score lies
    within 1e-6 relative of the oracle's K-th score."""
    exact = oracle.topk(gpu_scores, G, K)
    assert np.array_equal(gpu_groups, exact), "selection is not the exact top-K of its scores"
    for r in range(gpu_groups.shape[0]):
        a = set(gpu_groups[r][gpu_groups[r] >= 0].tolist())
        b = set(ora_groups[r][ora_groups[r] >= 0].tolist())
        if a == b:
            continue
        g = int(G[r])
        s = ora_scores[r, :g].astype(np.float64)
        kth = np.sort(s)[::-1][K - 1]
        for x in a ^ b:
            assert abs(s[x] - kth) <= TIE_REL * abs(kth), (
                f"row {r}: group {x} (score {s[x]}) differs outside the tie window of {kth}")


def check_tokens(gpu_tokens: np.ndarray, groups: np.ndarray, L0: np.ndarray, W: int,
                 max_ctx: int, Q: int):
    for b in range(gpu_tokens.shape[0]):
        for j in range(gpu_tokens.shape[1]):
            L = int(L0[b])
            if not (0 <= L <= max_ctx - (Q - 1)):
                assert np.all(gpu_tokens[b, j] == -1)
                continue
            want = oracle.position_tokens(groups[b], L, j, W)
            assert np.array_equal(gpu_tokens[b, j], want), f"token list of ({b},{j})"


def check_attention(gpu_out: np.ndarray, ora_out: np.ndarray, kv_dtype: int):
    err = np.abs(gpu_out.astype(np.float64) - ora_out)
    tol = ATOL[kv_dtype]
    worst = float(err.max()) if err.size else 0.0
    assert np.all(np.isfinite(gpu_out)), "non-finite attention output"
    assert worst <= tol, f"attention max-abs {worst:.3e} > {tol}"
    return worst
