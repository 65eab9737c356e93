"""Pins of the oracle's cache append ("prefill writes" into the paged caches,
qsa-hisparse README, entry points; FP8 E4M3 KV of its offload contract):
the FP8 encoder against the format (exact codes round-trip, ties to the
even mantissa, saturation) and against torch's CPU float8_e4m3fn cast, and
the append against invariants (exactly the addressed slots change, values
within half a code step, k-hat slots, page-permutation invariance)."""
import math

import numpy as np
import pytest
import torch

import oracle
import workload

PAGE, RATIO, GPP = 64, 4, 16


def _e4m3(code):
    return oracle.fp8_e4m3_value(code)


def test_encode_round_trips_every_finite_code():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.fp8_e4m3_encode(_e4m3(c)) == c, hex(c)


def test_encode_ties_go_to_even_mantissa():
    # midpoints of adjacent positive codes (format values, not oracle output)
    for c in range(0x7E):
        lo, hi = _e4m3(c), _e4m3(c + 1)
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.fp8_e4m3_encode(mid) == even, hex(c)
        assert oracle.fp8_e4m3_encode(-mid) == 0x80 | even, hex(c)
        assert oracle.fp8_e4m3_encode(math.nextafter(mid, 0.0)) == c
        assert oracle.fp8_e4m3_encode(math.nextafter(mid, math.inf)) == c + 1


def test_encode_saturates_and_keeps_nan():
    for x in (448.0, 460.0, 464.0, 465.0, 1e6, math.inf):
        assert oracle.fp8_e4m3_encode(x) == 0x7E
        assert oracle.fp8_e4m3_encode(-x) == 0xFE
    assert oracle.fp8_e4m3_encode(math.nan) == 0x7F
    assert oracle.fp8_e4m3_encode(-0.0) == 0x80 and oracle.fp8_e4m3_encode(0.0) == 0x00


def test_encode_matches_torch_cast_in_range():
    # torch's CPU float32 -> float8_e4m3fn cast rounds to nearest even; it
    # turns magnitudes past 464 into NaN, where this reading saturates, so
    # the comparison stays inside [-464, 464]
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(-464, 464, 3000), rng.normal(0, 1, 3000),
                        rng.uniform(-0.03, 0.03, 3000), np.ldexp(rng.uniform(-1, 1, 1000), -9)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = np.array([oracle.fp8_e4m3_encode(float(v)) for v in x], np.uint8)
    assert np.array_equal(ref, mine)


def _random_append(seed, geom, n_req, n_tokens, start, pages_per_req=40):
    """Caches filled with a recognisable background, a random page table
    and random new bf16 rows."""
    rng = np.random.default_rng(seed)
    Hkv, D = geom["num_kv_heads"], geom["head_dim"]
    P = n_req * pages_per_req + 3
    fp8 = geom["kv_dtype"] == 1
    dt = np.uint8 if fp8 else np.uint16
    kc = rng.integers(0, 0x7E if fp8 else 0x3F00, (P, PAGE, Hkv, D)).astype(dt)
    vc = rng.integers(0, 0x7E if fp8 else 0x3F00, (P, PAGE, Hkv, D)).astype(dt)
    kh = rng.normal(size=(P, GPP, 8, 64)).astype(np.float32)
    pt = rng.permutation(P)[:n_req * pages_per_req].reshape(n_req, pages_per_req).astype(np.int32)
    k_new = workload.normal_bf16(seed, 1, (n_req, n_tokens, Hkv, D))
    v_new = workload.normal_bf16(seed, 2, (n_req, n_tokens, Hkv, D))
    kh_new = rng.normal(size=(n_req, oracle.append_khat_slots(n_tokens), 8, 64)).astype(np.float32)
    return kc, vc, kh, pt, P, np.asarray(start, np.int32), k_new, v_new, kh_new


def _slot_of(pt, r, t):
    return pt[r, t // PAGE], t % PAGE


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_append_writes_exactly_the_addressed_slots(kv):
    geom = workload.geometry(kv_dtype=kv, k_scale=0.37 if kv == "fp8" else 1.0,
                             v_scale=0.05 if kv == "fp8" else 1.0)
    start = [5, 64 * 3 + 62, 1000]
    kc, vc, kh, pt, P, sp, kn, vn, khn = _random_append(4, geom, 3, 7, start)
    pt[2, 1000 // PAGE] = P + 9   # an out-of-range page: its tokens are skipped
    kc2, vc2, kh2 = oracle.append(geom, kc, vc, kh, pt, P, np.arange(3), sp, kn, vn, khn)
    written = np.zeros(kc.shape[:2], bool)
    for r in range(3):
        for i in range(7):
            t = int(sp[r]) + i
            p, s = _slot_of(pt, r, t)
            if not (0 <= p < P):
                continue
            written[p, s] = True
            for cache, new, scale in ((kc2, kn, geom["k_scale"]), (vc2, vn, geom["v_scale"])):
                x = np.array([oracle.bf16_value(int(b)) for b in new[r, i].ravel()])
                got = cache[p, s].ravel()
                if kv == "bf16":
                    assert np.array_equal(got, new[r, i].ravel())  # scale 1: the bits themselves
                    continue
                q = (x / scale).astype(np.float32).astype(np.float64)
                dec = np.array([_e4m3(int(c)) for c in got])
                # within half the spacing of adjacent E4M3 values around q
                step = np.where(np.abs(q) < 2.0 ** -6, 2.0 ** -9,
                                2.0 ** (np.floor(np.log2(np.maximum(np.abs(q), 2.0 ** -6))) - 3))
                assert np.all(np.abs(dec - np.clip(q, -448, 448)) <= step / 2)
    assert np.array_equal(kc2[~written], kc[~written]) and np.array_equal(vc2[~written], vc[~written])


def test_append_khat_slots_follow_group_completion():
    geom = workload.geometry(kv_dtype="bf16")
    # start 6, 8 tokens (6..13): groups 1 and 2 complete (last tokens 7 and
    # 11); group 3 ends at 15 > 13.  Two slots: groups 1, 2.
    kc, vc, kh, pt, P, sp, kn, vn, khn = _random_append(5, geom, 1, 8, [6])
    assert oracle.append_khat_slots(8) == 2
    _, _, kh2 = oracle.append(geom, kc, vc, kh, pt, P, [0], sp, kn, vn, khn)
    for j in range(2):
        g = 6 // RATIO + j
        p, s = pt[0, g // GPP], g % GPP
        if 4 * g + 3 < 6 + 8:
            assert np.array_equal(kh2[p, s], khn[0, j]), j
        else:
            assert np.array_equal(kh2[p, s], kh[p, s]), j
    changed = np.any(kh2 != kh, axis=(2, 3))
    assert int(changed.sum()) == 2
    # start 4 (aligned), 5 tokens (4..8): only group 1 (last token 7)
    kc, vc, kh, pt, P, sp, kn, vn, khn = _random_append(8, geom, 1, 5, [4])
    _, _, kh2 = oracle.append(geom, kc, vc, kh, pt, P, [0], sp, kn, vn, khn)
    changed = np.argwhere(np.any(kh2 != kh, axis=(2, 3)))
    assert changed.tolist() == [[pt[0, 0], 1]]
    assert np.array_equal(kh2[pt[0, 0], 1], khn[0, 0])


def test_append_is_invariant_under_page_permutation():
    geom = workload.geometry(kv_dtype="fp8", k_scale=0.2, v_scale=0.3)
    kc, vc, kh, pt, P, sp, kn, vn, khn = _random_append(6, geom, 2, 70, [100, 3])
    a = oracle.append(geom, kc, vc, kh, pt, P, [0, 1], sp, kn, vn, khn)
    perm = np.random.default_rng(7).permutation(P)   # physical page p -> perm[p]
    inv = np.argsort(perm)
    b = oracle.append(geom, kc[inv], vc[inv], kh[inv], perm[pt].astype(np.int32), P, [0, 1], sp,
                      kn, vn, khn)
    for x, y in zip(a, b):
        assert np.array_equal(x, y[perm])
