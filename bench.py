"""Benchmark of the QSA layer step on one MI355X.

A step is one ``qsa_decode`` call (indexer scoring -> exact top-K ->
expansion -> paged sparse GQA attention) on the headline workload: decode
of 8 requests at 262,144 tokens each (65,536 C4 groups), FP8 E4M3 paged KV
(page 64, random page table), Hq 16 / Hkv 2, head dim 256, K = 2,048 groups.
Inputs are seeded and synthetic and resident in HBM before timing.

Prints one JSON line: layer-steps/s, the roofline position of the dominant
kernel (the indexer GEMV, HBM-bound) measured with HIP events on the stream
it runs on, the prefill indexer scoring on the matrix cores against the BF16
MFMA peak (the long-prefill chunk), the cache append of that chunk against
the HBM peak, the multi-query indexer form (decode at the Flash-Next shape
and prefill scoring), and the CPU oracle timed on this host as a reported
baseline.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense BF16 MFMA (no sparsity)
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense FP32 MFMA (context for the prefill scoring)

CONFIG_NAMES = {
    1: "decode B1, L=8,193, BF16 KV, identity pages, K=512 groups",
    2: "decode B8, L~U[32K,64K], FP8 KV, random pages, K=512 groups",
    3: "decode B8, L=262,144 (65,536 groups), FP8 E4M3 KV, random pages, K=2,048 groups",
    5: "decode B4 x 3 positions (base + 2 drafts), L0=131,072+r, Hq24/Hkv2, FP8 KV, K=1,024",
}


# short names of the workloads, used for the profile summaries
WORKLOAD_SLUG = {
    1: "decode_b1_l8193_bf16_k512",
    2: "decode_b8_l32k-64k_fp8_k512",
    3: "decode_b8_l262144_fp8_k2048",
    5: "mtp_b4x3_l131073_fp8_k1024",
}


def algorithmic_bytes(wl) -> dict:
    """Bytes a step must move at minimum: the k̂ of every complete group, the
    K/V rows of every selected token, indexer/attention queries, outputs
    and page-table entries read."""
    g = wl.geom
    esize = 1 if g["kv_dtype"] == 1 else 2
    kv_row = 2 * g["num_kv_heads"] * g["head_dim"] * esize  # K + V of one token
    Q = wl.q_per_req
    khat = scores = pt = pt_score = kv = 0
    hk = g.get("idx_key_heads", g["idx_heads"])
    group_bytes = hk * g["idx_dim"] * 4             # fp32 k̂ of one group (2 KiB or 512 B)
    for L in wl.ctx_lens.tolist():
        G = L // 4
        khat += G * group_bytes                   # the k̂ of every complete group
        scores += G * 4                           # one fp32 score written per group
        pt_score += (G + 15) // 16 * 4            # page ids read by the indexer
        pt += (L + Q - 1 + 63) // 64 * 4          # page ids of the request
        sel = 4 * min(g["topk_groups"], G) + (L + Q - 1 - 4 * G)
        kv += sel * kv_row                        # K and V rows of the selected tokens
    B = wl.batch
    idx_q = B * (g["idx_heads"] * g["idx_dim"] * 4 + g["idx_heads"] * 4)  # q_idx + w_idx
    attn_io = B * Q * g["num_q_heads"] * g["head_dim"] * (2 + 4)  # bf16 q in, fp32 out
    return dict(khat=khat, kv=kv, scores=scores, page_table=pt,
                step=khat + kv + pt + idx_q + attn_io,
                score_kernel=khat + scores + pt_score + idx_q)


def source_digest(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "learned_sparse_attention_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, digest: str, profiles_dir: str = None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    path = os.path.join(profiles_dir or os.path.join(ROOT, "profiles"),
                        f"{kernel}__{workload}.counters.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_digest") != digest:
        return None
    return d.get("hbm_bytes_per_launch")


COPY_BYTES = 1 << 30  # calibration copy: 1 GiB read, 1 GiB written


def calibrate_copy(dev) -> None:
    """Three launches of a plain elementwise copy (negation) of known size, so
    a counter run can scale FETCH_SIZE / WRITE_SIZE to bytes."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


def _read_counters(path: str) -> dict:
    """Mean counter value per kernel name from rocprofv3 counter_collection CSVs
    found under ``path``."""
    import csv
    import glob
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {path}")
    sums: dict = {}
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                key = (row["Kernel_Name"], row["Counter_Name"])
                v = sums.setdefault(key, [0.0, 0])
                v[0] += float(row["Counter_Value"])
                v[1] += 1
    return {k: v[0] / v[1] for k, v in sums.items()}


def write_counters(fetch_dir: str, write_dir: str, workload_name: str, commands: list,
                   out_dir: str = None) -> None:
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch) into HBM bytes per launch, each scaled by what the counter reads
    for the calibration copy; writes profiles/<kernel>__<workload>.counters.json
    for the indexer kernel and a text table for every kernel."""
    fetch, write = _read_counters(fetch_dir), _read_counters(write_dir)

    def mean(d, sub, counter):
        vals = [v for (k, c), v in d.items() if sub in k and c == counter]
        return sum(vals) / len(vals) if vals else None

    copy_f = mean(fetch, "neg_kernel", "FETCH_SIZE")
    copy_w = mean(write, "neg_kernel", "WRITE_SIZE")
    ff = COPY_BYTES / (copy_f * 1024.0)
    fw = COPY_BYTES / (copy_w * 1024.0)
    kernels = sorted({k for (k, c) in fetch} | {k for (k, c) in write})
    lines = [f"# HBM traffic per dispatch (rocprofv3 FETCH_SIZE, WRITE_SIZE), workload {workload_name}", "",
             "Commands:", *[f"    {c}" for c in commands], "",
             f"Calibration copy (1 GiB in, 1 GiB out): FETCH_SIZE {copy_f:.0f} KiB -> factor "
             f"{ff:.4f}; WRITE_SIZE {copy_w:.0f} KiB -> factor {fw:.4f}", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled HBM bytes |",
             "|---|---|---|---|"]
    for k in kernels:
        f_, w_ = mean(fetch, k, "FETCH_SIZE"), mean(write, k, "WRITE_SIZE")
        if f_ is None or w_ is None:
            continue
        tot = f_ * 1024.0 * ff + w_ * 1024.0 * fw
        short = k.replace("qsa::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
        lines.append(f"| {short[:90]} | {f_:.0f} | {w_:.0f} | {tot:.0f} |")
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"hbm_traffic__{workload_name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    sf = mean(fetch, "index_score_gemv_kernel", "FETCH_SIZE")
    sw = mean(write, "index_score_gemv_kernel", "WRITE_SIZE")
    rec = {"kernel": "index_score_gemv_kernel", "workload": workload_name,
           "source_digest": source_digest("index_score.hip", "qsa_device.h"),
           "fetch_kib": sf, "write_kib": sw, "copy_fetch_kib": copy_f, "copy_write_kib": copy_w,
           "fetch_factor": ff, "write_factor": fw,
           "hbm_bytes_per_launch": sf * 1024.0 * ff + sw * 1024.0 * fw, "commands": commands}
    with open(os.path.join(out_dir, f"index_score_gemv__{workload_name}.counters.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_BUSY_CYCLES",
                 "GRBM_GUI_ACTIVE")
PREFILL_SLUG = "prefill_q4096_p28672_g8192"
N_XCC, N_SIMD = 8, 1024


def write_mfma_counters(pmc_dir: str, commands: list, out_dir: str = None) -> None:
    """Turn one rocprofv3 --pmc run of the four MFMA_COUNTERS into matrix-core
    utilisation per matrix-core kernel.  rocprofv3 reports GRBM_GUI_ACTIVE
    summed over the 8 XCDs (it reads 8x the kernel's cycles), so the per-XCD
    busy time is that sum / 8; utilisation = MFMA busy cycles summed over all
    SIMDs / (per-XCD GPU-active cycles x 1,024 SIMDs), and flops = MOPS x 512.
    Writes a text table and profiles/index_score_mfma__<workload>.counters.json."""
    import csv
    import glob
    d = _read_counters(pmc_dir)
    kernels = sorted({k for (k, c) in d if c == "SQ_VALU_MFMA_BUSY_CYCLES"})
    # mean dispatch duration (ns) per kernel, to check the XCD reading: the
    # per-XCD cycles over it must come out near the shader clock
    durs: dict = {}
    for fn in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                durs.setdefault(row["Kernel_Name"], {})[row["Dispatch_Id"]] = (
                    int(row["End_Timestamp"]) - int(row["Start_Timestamp"]))
    lines = [f"# Matrix-core utilisation per dispatch (rocprofv3 --pmc), prefill chunk of 4,096 "
             f"queries at positions 28,672..32,767 (8,192 groups)", "",
             "Command:", *[f"    {c}" for c in commands], "",
             "util = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1,024 SIMDs); "
             "GFLOP = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / 1e9", "",
             "GRBM_GUI_ACTIVE is read as the sum over the 8 XCDs: an eighth of it over the "
             "dispatch's duration (the 'GHz implied' column) comes out at the shader clock for "
             "the long dispatches; short ones carry the counter window's own overhead.  Each "
             "16x16x32 BF16 MFMA counts 32 MOPs and 16 busy cycles, so the utilisation is the "
             "issued flops over the peak at the clock the kernel actually ran at.", "",
             "| kernel | us | GRBM_GUI_ACTIVE (sum of 8 XCDs) | GHz implied | SQ_BUSY_CYCLES | "
             "MFMA_MOPS_BF16 | MFMA_BUSY_CYCLES | GFLOP | MFMA util |",
             "|---|---|---|---|---|---|---|---|---|"]
    recs = {}
    for k in kernels:
        grbm = d.get((k, "GRBM_GUI_ACTIVE"))
        busy = d[(k, "SQ_VALU_MFMA_BUSY_CYCLES")]
        mops = d.get((k, "SQ_INSTS_VALU_MFMA_MOPS_BF16"), 0.0)
        if not grbm or not busy:
            continue
        util = busy / (grbm / N_XCC * N_SIMD)
        short = k.replace("qsa::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
        dk = durs.get(k, {})
        us = sum(dk.values()) / len(dk) / 1e3 if dk else float("nan")
        lines.append(f"| {short[:70]} | {us:.1f} | {grbm:.0f} | {grbm / N_XCC / us / 1e3:.2f} | "
                     f"{d.get((k, 'SQ_BUSY_CYCLES'), 0):.0f} | {mops:.0f} | {busy:.0f} | "
                     f"{mops * 512 / 1e9:.2f} | {100 * util:.1f}% |")
        if "index_score_mfma_kernel" in short:
            recs[short.split("<", 1)[1].rsplit(">", 1)[0].strip()] = {
                "mfma_util": util, "flops_per_launch": mops * 512, "us_per_launch": us,
                "grbm_gui_active_sum": grbm, "mfma_busy_cycles": busy}
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"mfma_util__{PREFILL_SLUG}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    rec = {"kernel": "index_score_mfma_kernel", "workload": PREFILL_SLUG,
           "source_digest": source_digest("index_score_prefill.hip", "qsa_device.h"),
           "forms": recs, "commands": commands}
    with open(os.path.join(out_dir, f"index_score_mfma__{PREFILL_SLUG}.counters.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def write_trace(trace_dir: str, commands: list, out_dir: str = None) -> str:
    """Turn a rocprofv3 --kernel-trace --stats run of this script into the
    kernel-time table of profiles/qsa_decode__<workload>.kernel_trace.md
    (durations in microseconds, per kernel: calls, mean, min, max, share)."""
    import csv
    import glob
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    rows = []
    for fn in files:
        with open(fn, newline="") as f:
            rows += list(csv.DictReader(f))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = ["# Kernel trace: bench.py (decode B8 at 262,144 tokens, FP8 E4M3 KV, K = 2,048 groups; "
             "prefill chunk of 4,096 queries; cache append; multi-query indexer legs)", "",
             "Command (from the repository root, on one MI355X):", "",
             *[f"    {c}" for c in commands], "",
             "rocprofv3 kernel statistics (durations in microseconds).  bench.py times the decode "
             "step (one `qsa_decode`: index_score_gemv_kernel, topk_extract_kernel, "
             "topk_finish_kernel, attn_decode_kernel, combine_kernel), the indexer GEMV alone, "
             "the prefill scoring alone and whole `qsa_prefill` steps on the 4,096-query chunk "
             "(index_score_mfma_kernel, topk_row_kernel, attn_prefill_kernel; BF16 and FP8 K/V), "
             "the cache append, and the multi-query indexer legs "
             "(`Form<4, 1, 128>` is the shared-key form, `Form<8, 8, 64>` the per-head form).", "",
             "| kernel | calls | average | min | max | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("qsa::(anonymous namespace)::", "").replace("void ", "")
        name = name.split("(")[0]
        lines.append(f"| {name[:110]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{100 * float(r['TotalDurationNs']) / total:.1f}% |")
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    path = os.path.join(out_dir, f"qsa_decode__{WORKLOAD_SLUG[3]}.kernel_trace.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def measured_mfma_util(form: str, profiles_dir: str = None):
    """Matrix-core utilisation of index_score_mfma_kernel<form> from the
    committed counter summary, if it was taken on the current kernel source;
    else None."""
    path = os.path.join(profiles_dir or os.path.join(ROOT, "profiles"),
                        f"index_score_mfma__{PREFILL_SLUG}.counters.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_digest") != source_digest("index_score_prefill.hip", "qsa_device.h"):
        return None
    return d.get("forms", {}).get(form, {}).get("mfma_util")


def prefill_scoring(dev, steps: int, warmup: int) -> dict:
    """The long-prefill chunk (4,096 queries at positions 28,672 .. 32,767 of
    one request, 8,192 groups): the matrix-core indexer scoring alone, timed
    with events on the stream it runs on, against the dense BF16 MFMA peak;
    and the whole qsa_prefill step (scoring, top-K, attention) for context."""
    import numpy as np
    import torch
    import learned_sparse_attention_amd as qsa
    import workload
    wl = workload.config(4)
    d = workload.to_device(wl, dev)
    g = wl.geom
    gstride = (wl.first_pos + wl.n_q) // 4
    sc = torch.empty((wl.n_q, gstride), dtype=torch.float32, device=dev)

    def score():
        qsa.qsa_index_score_prefill(g, d["khat"], d["pt"], wl.req, wl.first_pos, d["q_idx"],
                                    d["w_idx"], out_scores=sc, num_pages=wl.num_pages)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(warmup):
        score()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        score()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    visible = int((wl.row_len.astype(np.int64) // 4).sum()) * 2 * 8 * 64
    dense = wl.n_q * gstride * 2 * 8 * 64
    out = torch.empty((wl.n_q, g["num_q_heads"], g["head_dim"]), dtype=torch.float32, device=dev)
    ws = torch.empty(qsa.prefill_workspace_size(g, wl.n_q, wl.first_pos + wl.n_q),
                     dtype=torch.uint8, device=dev)

    def step():
        qsa.qsa_prefill(g, d["k"], d["v"], d["khat"], d["pt"], wl.req, wl.first_pos, d["q_idx"],
                        d["w_idx"], d["q"], out=out, workspace=ws, num_pages=wl.num_pages)

    step()
    torch.cuda.synchronize()
    n_step = max(1, steps // 10)
    e0.record()
    for _ in range(n_step):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / n_step
    del d, sc, out, ws
    # the same chunk with FP8 E4M3 K/V
    wf = workload.prefill_workload(workload.CONFIG_SEED + 4, 28672, 4096, kv_dtype="fp8",
                                   topk_groups=512)
    df = workload.to_device(wf, dev)
    outf = torch.empty((wf.n_q, 16, 256), dtype=torch.float32, device=dev)
    wsf = torch.empty(qsa.prefill_workspace_size(wf.geom, wf.n_q, wf.first_pos + wf.n_q),
                      dtype=torch.uint8, device=dev)

    def step_fp8():
        qsa.qsa_prefill(wf.geom, df["k"], df["v"], df["khat"], df["pt"], wf.req, wf.first_pos,
                        df["q_idx"], df["w_idx"], df["q"], out=outf, workspace=wsf,
                        num_pages=wf.num_pages)

    step_fp8()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n_step):
        step_fp8()
    e1.record()
    torch.cuda.synchronize()
    ms_step_fp8 = e0.elapsed_time(e1) / n_step
    del df, outf, wsf
    tflops = visible / (ms * 1e-3) / 1e12
    return {"workload": "prefill chunk of 4,096 queries at positions 28,672..32,767, "
                        "8,192 groups, 8 heads x 64, BF16 KV, K=512 groups",
            "kernel": "index_score_mfma_kernel", "bound": "mfma", "achieved": tflops,
            "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tflops / BF16_PEAK_TFLOPS,
            "frac_vs_fp32_mfma_peak": tflops / FP32_MFMA_PEAK_TFLOPS,
            "flops_per_launch": visible, "dense_tile_flops": dense, "ms_per_launch": ms,
            "score_bytes_written": wl.n_q * gstride * 4,
            "mfma_util_counters": measured_mfma_util("Form<8, 8, 64>"),
            "prefill_step_ms": ms_step, "prefill_step_fp8_ms": ms_step_fp8}


def mqa_indexer(dev, steps: int, warmup: int) -> dict:
    """The multi-query indexer form (4 heads x 128 sharing one key head):
    the decode step at the Flash-Next attention shape (B8 at 262,144 tokens,
    Hq 24 / Hkv 2, FP8 KV, K = 2,048 groups) with its GEMV against the HBM
    peak, and the long-prefill chunk's matrix-core scoring against the BF16
    peak."""
    import numpy as np
    import torch
    import learned_sparse_attention_amd as qsa
    import workload

    def timed(fn, n):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    wl = workload.decode_workload(0x51A6, [262144] * 8, num_q_heads=24, num_kv_heads=2,
                                  kv_dtype="fp8", topk_groups=2048, indexer="mqa")
    d = workload.to_device(wl, dev)
    g = wl.geom
    out = torch.empty((8, 1, 24, 256), dtype=torch.float32, device=dev)
    ws = torch.empty(qsa.decode_workspace_size(g, 8, 1, wl.max_ctx), dtype=torch.uint8,
                     device=dev)
    sc = torch.empty((8, wl.max_ctx // 4), dtype=torch.float32, device=dev)
    ms_step = timed(lambda: qsa.qsa_decode(g, d["k"], d["v"], d["khat"], d["pt"], d["ctx"],
                                           d["q_idx"], d["w_idx"], d["q"], wl.max_ctx, out=out,
                                           workspace=ws, num_pages=wl.num_pages), steps)
    ms_gemv = timed(lambda: qsa.qsa_index_score(g, d["khat"], d["pt"], None, d["ctx"],
                                                d["q_idx"], d["w_idx"], wl.max_ctx,
                                                out_scores=sc, num_pages=wl.num_pages), steps)
    ab = algorithmic_bytes(wl)
    del d, out, ws, sc
    pw = workload.prefill_workload(0x51A7, 28672, 4096, kv_dtype="bf16", topk_groups=512,
                                   indexer="mqa")
    pd = workload.to_device(pw, dev)
    gstride = (pw.first_pos + pw.n_q) // 4
    psc = torch.empty((pw.n_q, gstride), dtype=torch.float32, device=dev)
    ms_pf = timed(lambda: qsa.qsa_index_score_prefill(pw.geom, pd["khat"], pd["pt"], pw.req,
                                                      pw.first_pos, pd["q_idx"], pd["w_idx"],
                                                      out_scores=psc, num_pages=pw.num_pages),
                  max(5, steps // 2))
    visible = int((pw.row_len.astype(np.int64) // 4).sum()) * 2 * 4 * 128
    gemv_gbs = ab["score_kernel"] / (ms_gemv * 1e-3) / 1e9
    step_gbs = ab["step"] / (ms_step * 1e-3) / 1e9
    tflops = visible / (ms_pf * 1e-3) / 1e12
    return {"indexer": "4 query heads x 128 dims sharing one key head (512 B of k-hat/group)",
            "decode": {"workload": "decode B8, L=262,144, Hq 24 / Hkv 2, FP8 E4M3 KV, "
                                   "K=2,048 groups",
                       "layer_steps_per_s": 1e3 / ms_step, "ms_per_step": ms_step,
                       "step_bytes": ab["step"], "step_frac": step_gbs / HBM_PEAK_GBS,
                       "gemv_kernel": "index_score_gemv_mqa_kernel",
                       "gemv_ms": ms_gemv, "gemv_bytes": ab["score_kernel"],
                       "gemv_achieved": gemv_gbs, "gemv_frac": gemv_gbs / HBM_PEAK_GBS,
                       "unit": "GB/s", "peak": HBM_PEAK_GBS},
            "prefill_scoring": {"workload": "prefill chunk of 4,096 queries at positions "
                                            "28,672..32,767, 8,192 groups",
                                "kernel": "index_score_mfma_kernel<SharedKeyForm>",
                                "achieved": tflops, "peak": BF16_PEAK_TFLOPS,
                                "unit": "TFLOP/s", "frac": tflops / BF16_PEAK_TFLOPS,
                                "flops_per_launch": visible, "ms_per_launch": ms_pf,
                                "mfma_util_counters": measured_mfma_util("Form<4, 1, 128>")}}


def kv_append(dev, steps: int, warmup: int) -> dict:
    """The cache append of the long-prefill chunk: 4,096 new tokens' K and V
    (bf16, 2 KV heads x 256) written into an FP8 E4M3 paged cache at
    positions 28,672 .. 32,767, and the k-hat of the 1,024 groups they
    complete.  A streaming copy: HBM bytes read + written per call."""
    import numpy as np
    import torch
    import learned_sparse_attention_amd as qsa
    import workload
    n, start, hkv, dim = 4096, 28672, 2, 256
    P = (start + n) // 64
    g = workload.geometry(kv_dtype="fp8", k_scale=0.02, v_scale=0.02)
    perm = workload.permutation(0x5A, 1, P)
    pt = torch.from_numpy(perm.reshape(1, P).astype(np.int32)).to(dev)
    kc = torch.zeros((P, 64, hkv, dim), dtype=torch.uint8, device=dev)
    vc = torch.zeros_like(kc)
    kh = torch.zeros((P, 16, 8, 64), dtype=torch.float32, device=dev)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    kn = t(workload.normal_bf16(0x5A, 2, (1, n, hkv, dim)).view(np.int16))
    vn = t(workload.normal_bf16(0x5A, 3, (1, n, hkv, dim)).view(np.int16))
    slots = qsa.append_khat_slots(n)
    khn = t(workload.normal_f32(0x5A, 4, (1, slots, 8, 64)))
    rows, sp = t(np.zeros(1, np.int32)), t(np.array([start], np.int32))

    def call():
        qsa.qsa_append_kv(g, kc, vc, kh, pt, rows, sp, kn, vn, khn, num_pages=P)

    # One call issued from Python takes longer on the host than the kernel
    # takes on the GPU, so back-to-back calls would time the host.  The
    # calls are captured in a HIP graph instead and the replays timed; the
    # cache after the replays must equal the cache after an eager call.
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ref = [kc.clone(), vc.clone(), kh.clone()]
    n_in_graph = max(1, min(steps, 50))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(n_in_graph):
            call()
    replays = max(1, steps // n_in_graph)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (replays * n_in_graph)
    for a, b in zip(ref, (kc, vc, kh)):
        if not torch.equal(a.view(torch.uint8), b.view(torch.uint8)):
            raise RuntimeError("kv_append: the cache after graph replays differs from eager")
    groups = (start + n) // 4 - start // 4
    nbytes = 2 * n * hkv * dim * (2 + 1) + groups * 8 * 64 * 4 * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "append of 4,096 tokens (positions 28,672..32,767) into an FP8 E4M3 "
                        "paged cache, 2 KV heads x 256, plus 1,024 k-hat groups",
            "kernel": "append_kernel", "bound": "hbm",
            "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
            "bytes_per_call": nbytes, "ms_per_call": ms,
            "timing": f"{replays} replays of a HIP graph of {n_in_graph} calls"}


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s: float = 15.0) -> dict:
    """The oracle, unchanged, on this host: whole-batch decode passes over
    all requests of the workload for about budget_s seconds.  The oracle
    spreads its indexer scoring and top-K over rows (one thread per
    request) and its attention over (request, position, head) triples;
    attention is nearly all of its time at this workload (fp64 over 8,192
    selected tokens per head), so `cores` counts the threads that phase
    runs on."""
    import oracle
    threads = oracle.num_threads()
    oracle.decode(wl)  # warm: page in the caches and the library
    passes, t_total = 0, 0.0
    while t_total < budget_s and passes < 1000:
        t0 = time.perf_counter()
        oracle.decode(wl)
        t_total += time.perf_counter() - t0
        passes += 1
    B, Q, Hq = wl.batch, wl.q_per_req, wl.geom["num_q_heads"]
    return {"value": passes / t_total, "unit": "layer-steps/s",
            "cores": min(threads, B * Q * Hq), "kind": "oracle",
            "threads_attention": min(threads, B * Q * Hq),
            "threads_scoring_topk": min(threads, B),
            "omp_threads": threads, "cpu_model": cpu_model(),
            "sample": f"{passes} whole-batch decode passes ({B} requests each, {t_total:.1f} s "
                      f"after one untimed pass); attention, nearly all of the time, runs one "
                      f"thread per (request, head), scoring and top-K one per request"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--input-sets", type=int, default=0,
                    help="independent input sets the timed loops rotate over (default: 1 for "
                         "config 3, whose 3 GiB exceed the 256 MB MALL; 3 for the smaller ones)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill-scoring measurement")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also launch a 1 GiB copy kernel (for counter runs)")
    ap.add_argument("--write-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: summarise two rocprofv3 --pmc runs into profiles/")
    ap.add_argument("--write-mfma-counters", metavar="PMC_DIR",
                    help="no GPU: summarise a rocprofv3 --pmc run of the matrix-core counters "
                         "into profiles/")
    ap.add_argument("--write-trace", metavar="TRACE_DIR",
                    help="no GPU: summarise a rocprofv3 --kernel-trace --stats run into profiles/")
    ap.add_argument("--counter-commands", nargs="*", default=[],
                    help="the commands that made the counter runs (recorded with them)")
    args = ap.parse_args()
    if args.write_trace:
        print(write_trace(args.write_trace, args.counter_commands))
        return 0
    if args.write_mfma_counters:
        write_mfma_counters(args.write_mfma_counters, args.counter_commands)
        return 0
    if args.write_counters:
        write_counters(*args.write_counters, WORKLOAD_SLUG[args.config], args.counter_commands)
        return 0
    if args.gpus != 1:
        print("bench.py: the QSA layer step runs on one GPU (it is not sharded); "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import learned_sparse_attention_amd as qsa
    import workload

    dev = torch.device("cuda:0")
    # Workloads smaller than the MALL are timed over several independent
    # input sets in turn, so that a step does not find the previous step's
    # data in the cache.
    n_sets = args.input_sets if args.input_sets > 0 else (1 if args.config == 3 else 3)
    t0 = time.perf_counter()
    wls = [workload.config(args.config, instance=k) for k in range(n_sets)]
    t_gen = time.perf_counter() - t0
    # A collector pass inside a timed loop (the binding allocates small host
    # objects per call) would stall the launches for milliseconds: collect
    # now and keep the collector off until the GPU legs are done.
    gc.collect()
    gc.disable()
    devs = [workload.to_device(w, dev) for w in wls]
    wl, d = wls[0], devs[0]
    g = wl.geom
    B, Q = wl.batch, wl.q_per_req
    out = torch.empty((B, Q, g["num_q_heads"], g["head_dim"]), dtype=torch.float32, device=dev)
    ws = torch.empty(max(qsa.decode_workspace_size(g, B, Q, w.max_ctx) for w in wls),
                     dtype=torch.uint8, device=dev)
    turn = [0]

    def step():
        k = turn[0] % n_sets
        turn[0] += 1
        w, dk = wls[k], devs[k]
        qsa.qsa_decode(g, dk["k"], dk["v"], dk["khat"], dk["pt"], dk["ctx"], dk["q_idx"],
                       dk["w_idx"], dk["q"], w.max_ctx, q_per_req=Q, out=out, workspace=ws,
                       num_pages=w.num_pages)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    # the spread of single steps, from an event pair around each step of a
    # second loop (the timed region above carries no per-step events)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for a, b in ev:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    per_step_us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)

    def pct(p):
        return per_step_us[min(len(per_step_us) - 1, int(p * len(per_step_us)))]

    # dominant kernel alone: the indexer GEMV (one launch per call), timed
    # with events on the current stream, which is the stream it runs on
    scs = [torch.empty((B, w.max_ctx // 4), dtype=torch.float32, device=dev) for w in wls]

    def score():
        k = turn[0] % n_sets
        turn[0] += 1
        w, dk = wls[k], devs[k]
        qsa.qsa_index_score(g, dk["khat"], dk["pt"], None, dk["ctx"], dk["q_idx"], dk["w_idx"],
                            w.max_ctx - (Q - 1), out_scores=scs[k], num_pages=w.num_pages)

    for _ in range(args.warmup):
        score()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        score()
    e1.record()
    torch.cuda.synchronize()
    ms_score = e0.elapsed_time(e1) / args.steps

    # algorithmic bytes: the mean over the input sets (their lengths differ
    # for config 2)
    abs_ = [algorithmic_bytes(w) for w in wls]
    ab = {key: sum(a[key] for a in abs_) / n_sets for key in abs_[0]}
    score_gbs = ab["score_kernel"] / (ms_score * 1e-3) / 1e9
    step_gbs = ab["step"] / (ms_step * 1e-3) / 1e9
    wname = WORKLOAD_SLUG[args.config]
    digest = source_digest("index_score.hip", "qsa_device.h")
    traffic = measured_traffic("index_score_gemv", wname, digest)

    result = {
        "metric": "QSA decode layer-steps/sec (B8, 256K ctx) + achieved HBM GB/s vs peak",
        "value": 1000.0 / ms_step,
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded SplitMix64/Box-Muller; N(0,1) KV quantised to FP8 E4M3 "
                "with per-tensor scale, N(0,1) q and k̂, U(0,1) w)",
        "config": {"workload": CONFIG_NAMES[args.config], "batch": B, "q_per_req": Q,
                   "ctx_lens": [int(x) for x in wl.ctx_lens[:8]], "topk_groups": g["topk_groups"],
                   "num_q_heads": g["num_q_heads"], "num_kv_heads": g["num_kv_heads"],
                   "head_dim": g["head_dim"], "kv": "fp8_e4m3" if g["kv_dtype"] else "bf16",
                   "seed": wl.seed, "input_sets": n_sets},
        "roofline": {"kernel": "index_score_gemv_kernel", "bound": "hbm",
                     "achieved": score_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": score_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": ab["score_kernel"],
                     "ms_per_launch": ms_score},
        "step_roofline": {"bound": "hbm", "algorithmic_bytes": ab["step"],
                          "achieved": step_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": step_gbs / HBM_PEAK_GBS},
        "step_us": {"p10": pct(0.10), "p50": pct(0.50), "p90": pct(0.90)},
        "gen_seconds": round(t_gen, 1),
    }
    if not args.no_prefill:
        result["prefill_scoring"] = prefill_scoring(dev, max(5, args.steps // 2), 3)
        result["kv_append"] = kv_append(dev, max(20, args.steps), 5)
        result["mqa_indexer"] = mqa_indexer(dev, max(10, args.steps // 2), 3)
    if args.calibrate_copy:
        calibrate_copy(dev)
    gc.enable()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
