"""Host logic of bench.py, on the CPU: the algorithmic byte count of the
headline decode step, and the summaries that turn rocprofv3 counter CSVs
into per-launch HBM bytes and matrix-core utilisation (with the source
digest that retires them once a kernel changes)."""
import csv
import json
import os
from types import SimpleNamespace

import numpy as np

import bench

HEADER = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write_csv(path, rows):
    """rows: (dispatch id, kernel name, counter, value, start ns, end ns)"""
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HEADER)
        for i, (d, k, c, v, t0, t1) in enumerate(rows):
            w.writerow([i, d, "Agent 1", 1, 1, 1, 1024, 1, k, 256, 0, 0, 8, 0, 16, c, v, t0, t1])


def test_headline_algorithmic_bytes():
    # decode B8 at 262,144 tokens, FP8 KV, 2 KV heads x 256, 16 query heads,
    # K = 2,048 groups, 8 x 64 indexer: 65,536 groups per request
    geom = dict(kv_dtype=1, num_kv_heads=2, head_dim=256, idx_heads=8, idx_dim=64,
                topk_groups=2048, num_q_heads=16)
    wl = SimpleNamespace(geom=geom, ctx_lens=np.full(8, 262144), q_per_req=1, batch=8)
    ab = bench.algorithmic_bytes(wl)
    khat = 8 * 65536 * 2048                  # 2 KiB of fp32 k̂ per group
    scores = 8 * 65536 * 4
    score_pages = 8 * 4096 * 4               # one page id per 16 groups
    idx_q = 8 * (8 * 64 * 4 + 8 * 4)         # q_idx and w_idx
    assert ab["score_kernel"] == khat + scores + score_pages + idx_q == 1_075_986_688
    kv = 8 * (4 * 2048) * (2 * 2 * 256)      # 8,192 selected tokens (no partial block), K + V
    pages = 8 * 4096 * 4                     # 262,144 / 64 page ids per request
    attn_io = 8 * 16 * 256 * (2 + 4)         # bf16 q in, fp32 out
    assert ab["step"] == khat + kv + pages + idx_q + attn_io == 1_141_195_008


def test_hbm_counter_summary_and_digest(tmp_path):
    gemv = "qsa::(anonymous namespace)::index_score_gemv_kernel(float const*, int const*)"
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(int)"
    fetch = [(1, copy, "FETCH_SIZE", 524288.0, 0, 10), (2, gemv, "FETCH_SIZE", 100.0, 20, 30),
             (3, gemv, "FETCH_SIZE", 300.0, 40, 50)]
    write = [(1, copy, "WRITE_SIZE", 1048576.0, 0, 10), (2, gemv, "WRITE_SIZE", 10.0, 20, 30),
             (3, gemv, "WRITE_SIZE", 30.0, 40, 50)]
    _write_csv(str(tmp_path / "f" / "x_counter_collection.csv"), fetch)
    _write_csv(str(tmp_path / "w" / "x_counter_collection.csv"), write)
    out = tmp_path / "profiles"
    bench.write_counters(str(tmp_path / "f"), str(tmp_path / "w"), "wl", ["cmd"], out_dir=str(out))
    rec = json.loads((out / "index_score_gemv__wl.counters.json").read_text())
    # the copy reads 1 GiB as 512 Ki KiB of FETCH_SIZE (factor 2) and writes
    # 1 GiB as 1 Mi KiB (factor 1); the GEMV's means are 200 and 20 KiB
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    assert rec["hbm_bytes_per_launch"] == 200 * 1024 * 2 + 20 * 1024
    digest = bench.source_digest("index_score.hip", "qsa_device.h")
    assert rec["source_digest"] == digest
    assert bench.measured_traffic("index_score_gemv", "wl", digest, str(out)) == 430080
    assert bench.measured_traffic("index_score_gemv", "wl", "0" * 16, str(out)) is None
    assert "| index_score_gemv_kernel | 200 | 20 | 430080 |" in (out / "hbm_traffic__wl.md").read_text()


def test_mfma_counter_summary_and_digest(tmp_path):
    k = ("void qsa::(anonymous namespace)::index_score_mfma_kernel<qsa::(anonymous namespace)::"
         "Form<8, 8, 64> >(float const*, int const*, int)")
    rows = []
    for d in (1, 2):  # two dispatches of 1 us each
        t0 = 1000 * d
        rows += [(d, k, "GRBM_GUI_ACTIVE", 8000.0, t0, t0 + 1000),
                 (d, k, "SQ_VALU_MFMA_BUSY_CYCLES", 256000.0 * d, t0, t0 + 1000),
                 (d, k, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1000.0, t0, t0 + 1000),
                 (d, k, "SQ_BUSY_CYCLES", 5000.0, t0, t0 + 1000)]
    _write_csv(str(tmp_path / "pmc" / "m_counter_collection.csv"), rows)
    out = tmp_path / "profiles"
    bench.write_mfma_counters(str(tmp_path / "pmc"), ["cmd"], out_dir=str(out))
    rec = json.loads((out / f"index_score_mfma__{bench.PREFILL_SLUG}.counters.json").read_text())
    form = rec["forms"]["Form<8, 8, 64>"]
    # GRBM_GUI_ACTIVE is the sum of 8 XCDs: 1,000 cycles each; the mean busy
    # count 384,000 over 1,000 cycles x 1,024 SIMDs is 37.5 %
    assert form["mfma_util"] == 384000.0 / (1000 * 1024)
    assert form["flops_per_launch"] == 1000.0 * 512
    assert rec["source_digest"] == bench.source_digest("index_score_prefill.hip", "qsa_device.h")
    assert bench.measured_mfma_util("Form<8, 8, 64>", str(out)) == form["mfma_util"]
    assert bench.measured_mfma_util("Form<4, 1, 128>", str(out)) is None
    rec["source_digest"] = "0" * 16
    (out / f"index_score_mfma__{bench.PREFILL_SLUG}.counters.json").write_text(json.dumps(rec))
    assert bench.measured_mfma_util("Form<8, 8, 64>", str(out)) is None
    md = (out / f"mfma_util__{bench.PREFILL_SLUG}.md").read_text()
    # 1,000 cycles per XCD in 1 us: the implied clock column reads 1.00 GHz
    assert "| index_score_mfma_kernel<Form<8, 8, 64> > | 1.0 | 8000 | 1.00 |" in md


def test_kernel_trace_summary(tmp_path):
    # a rocprofv3 kernel_stats.csv of two kernels -> the table in the
    # committed profile format, sorted by total time, shares summing to 100 %
    d = tmp_path / "trace" / "host"
    os.makedirs(d)
    with open(d / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                    "MaxNs", "StdDev"])
        w.writerow(["void qsa::(anonymous namespace)::combine_kernel(float const*, int)", 10,
                    50000, 5000, 20.0, 4000, 7000, 1.0])
        w.writerow(["qsa::(anonymous namespace)::index_score_gemv_kernel(float const*)", 2,
                    200000, 100000, 80.0, 99000, 101000, 1.0])
    path = bench.write_trace(str(tmp_path / "trace"), ["rocprofv3 ... -- python3 bench.py"],
                             out_dir=str(tmp_path / "profiles"))
    text = open(path).read()
    rows = [l for l in text.splitlines() if l.startswith("| ") and "calls" not in l]
    assert rows[0].startswith("| index_score_gemv_kernel | 2 | 100.00 | 99.00 | 101.00 | 80.0% |")
    assert rows[1].startswith("| combine_kernel | 10 | 5.00 | 4.00 | 7.00 | 20.0% |")
    assert "rocprofv3 ... -- python3 bench.py" in text
