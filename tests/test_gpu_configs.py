"""GPU parity on the five seeded workloads at their full sizes, in the
launch configuration bench.py times (qsa_decode / qsa_prefill with their
default splits): scores, exact top-K (tie window 1e-6 of the K-th score),
token lists (bit-exact) and attention on the GPU's own selection.  The
decode workloads are checked on every request.  The long-prefill chunk is
checked in test_gpu_prefill.py (test_prefill_long_chunk_every_row): scores,
top-K and attention on every one of its 4,096 query rows."""
import numpy as np
import pytest

import workload
from tests.test_gpu_parity import _decode_check

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("tail", [1, 2, 3])
def test_config_decode_b1_8192_plus_tail(gpu, tail):
    wl = workload.config(1, tail=tail)
    assert int(wl.ctx_lens[0]) == 8192 + tail
    _decode_check(wl, gpu)


def test_config_decode_b8_mixed_32k_64k_fp8(gpu):
    wl = workload.config(2)
    assert wl.batch == 8 and wl.geom["kv_dtype"] == 1
    assert np.all((wl.ctx_lens >= 32768) & (wl.ctx_lens <= 65536))
    _decode_check(wl, gpu)


def test_config_decode_b8_262144_fp8_k2048(gpu):
    wl = workload.config(3)
    assert wl.batch == 8 and np.all(wl.ctx_lens == 262144)
    assert wl.geom["topk_groups"] == 2048
    _decode_check(wl, gpu)


def test_config_mtp_b4_three_positions_hq24(gpu):
    wl = workload.config(5)
    assert wl.q_per_req == 3 and wl.geom["num_q_heads"] == 24 and wl.geom["num_kv_heads"] == 2
    _decode_check(wl, gpu)
