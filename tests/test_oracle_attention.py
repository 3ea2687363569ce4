"""Pins of the oracle's decode attention: brute force on tiny inputs, closed
forms, invariants, split-K equivalence and the pages' byte counts."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import kvq_oracle as orc
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute_dequant(codes, scales, group):
    """Scalar dequantization with Fractions, independent of the oracle."""
    out = []
    for i, c in enumerate(codes.tolist()):
        out.append(float(Fraction(int(c)) * Fraction(float(scales[i // group]))))
    return out


def _brute_attend(q, keys, vals, sm_scale):
    """Scalar softmax attention with math.exp / math.fsum for one query row."""
    z = [sm_scale * math.fsum(float(a) * float(b) for a, b in zip(q, k)) for k in keys]
    mx = max(z)
    e = [math.exp(t - mx) for t in z]
    den = math.fsum(e)
    d = len(vals[0])
    return [math.fsum(e[p] * vals[p][i] for p in range(len(vals))) / den for i in range(d)]


def _filled_cache(seed, B, max_ctx, Hkv, d, g, lens, kdt="int8", vdt="int8", k_scale=1.0):
    cache = orc.Cache(B, max_ctx, Hkv, d, g, kdt, vdt)
    k = wl.uniform_rows(seed, (B, max_ctx, Hkv, d), k_scale)
    v = wl.uniform_rows(seed + 1, (B, max_ctx, Hkv, d))
    cache.append(k, v, np.zeros(B, dtype=np.int64))
    return cache, k, v


@pytest.mark.parametrize("case", [
    dict(B=2, Hq=4, Hkv=2, d=16, g=8, lens=[7, 3], W=0),
    dict(B=1, Hq=6, Hkv=3, d=8, g=8, lens=[8], W=3),
    dict(B=2, Hq=4, Hkv=1, d=16, g=16, lens=[5, 8], W=6),
    dict(B=1, Hq=2, Hkv=2, d=8, g=4, lens=[6], W=0, kdt="fp32", vdt="int8"),
    dict(B=1, Hq=4, Hkv=2, d=8, g=4, lens=[6], W=2, kdt="int8", vdt="fp32"),
])
def test_attend_matches_bruteforce(case):
    B, Hq, Hkv, d, g, W = case["B"], case["Hq"], case["Hkv"], case["d"], case["g"], case["W"]
    lens = np.array(case["lens"])
    kdt, vdt = case.get("kdt", "int8"), case.get("vdt", "int8")
    cache, _, _ = _filled_cache(11, B, 8, Hkv, d, g, lens, kdt, vdt, k_scale=2.0)
    q = wl.uniform_rows(12, (B, Hq, d))
    sm = 1.0 / math.sqrt(d)
    got = orc.attend(q, cache, lens, W, sm)
    G = Hq // Hkv
    for b in range(B):
        L = int(lens[b])
        lo = L - W if (W and L > W) else 0
        for h in range(Hq):
            hk = h // G

            def row(s, p):
                if cache.dtypes[s] == "int8":
                    return _brute_dequant(cache.data[s][b, p, hk], cache.scales[s][b, p, hk], g)
                return [float(x) for x in cache.data[s][b, p, hk]]
            keys = [row("k", p) for p in range(lo, L)]
            vals = [row("v", p) for p in range(lo, L)]
            want = _brute_attend(q[b, h].astype(np.float64), keys, vals, sm)
            np.testing.assert_allclose(got[b, h], want, rtol=0, atol=1e-12)


def test_single_position_returns_that_value_row():
    cache, _, _ = _filled_cache(21, 1, 4, 2, 64, 64, [1])
    q = wl.uniform_rows(22, (1, 8, 64), 3.0)
    out = orc.attend(q, cache, np.array([1]), 0, 0.125)
    for h in range(8):
        np.testing.assert_array_equal(out[0, h], cache.values("v", 0, 0, 1, h // 4)[0])


def test_constant_values_return_that_row():
    cache, _, _ = _filled_cache(23, 1, 32, 1, 64, 64, [32])
    row = cache.data["v"][0, 0, 0].copy()
    cache.data["v"][0, :, 0] = row
    cache.scales["v"][0, :, 0] = cache.scales["v"][0, 0, 0]
    q = wl.uniform_rows(24, (1, 4, 64), 2.0)
    out = orc.attend(q, cache, np.array([32]), 0, 0.125)
    want = cache.values("v", 0, 0, 1, 0)[0]
    np.testing.assert_allclose(out[0], np.broadcast_to(want, (4, 64)), rtol=1e-15, atol=1e-15)


def test_zero_query_gives_mean_of_values():
    cache, _, _ = _filled_cache(25, 1, 40, 2, 32, 32, [40])
    q = np.zeros((1, 4, 32), dtype=np.float16)
    for W, lo in ((0, 0), (9, 31)):
        out = orc.attend(q, cache, np.array([40]), W, 0.2)
        for h in range(4):
            want = cache.values("v", 0, lo, 40, h // 2).mean(axis=0)
            np.testing.assert_allclose(out[0, h], want, rtol=1e-13, atol=1e-14)


def test_window_semantics():
    cache, _, _ = _filled_cache(26, 1, 64, 1, 16, 16, [64])
    q = wl.uniform_rows(27, (1, 2, 16))
    L = np.array([50])
    full = orc.attend(q, cache, L, 0, 0.25)
    np.testing.assert_array_equal(orc.attend(q, cache, L, 50, 0.25), full)
    np.testing.assert_array_equal(orc.attend(q, cache, L, 1000, 0.25), full)
    # window 10 == attention over exactly the last 10 positions
    w10 = orc.attend(q, cache, L, 10, 0.25)
    K = cache.values("k", 0, 40, 50, 0)
    V = cache.values("v", 0, 40, 50, 0)
    want = _brute_attend(q[0, 0].astype(np.float64), K.tolist(), V.tolist(), 0.25)
    np.testing.assert_allclose(w10[0, 0], want, atol=1e-12)
    # window 1 returns the newest value row
    np.testing.assert_array_equal(orc.attend(q, cache, L, 1, 0.25)[0, 1], cache.values("v", 0, 49, 50, 0)[0])


def test_permutation_invariance():
    cache, _, _ = _filled_cache(28, 1, 24, 1, 32, 32, [24])
    q = wl.uniform_rows(29, (1, 3, 32))
    out = orc.attend(q, cache, np.array([24]), 0, 0.2)
    perm = np.random.default_rng(3).permutation(24)
    for s in ("k", "v"):
        cache.data[s][0] = cache.data[s][0][perm]
        cache.scales[s][0] = cache.scales[s][0][perm]
    out2 = orc.attend(q, cache, np.array([24]), 0, 0.2)
    np.testing.assert_allclose(out, out2, rtol=1e-13, atol=1e-14)


def test_gqa_equals_replicated_mha():
    cache, _, _ = _filled_cache(30, 1, 16, 2, 16, 8, [16])
    q = wl.uniform_rows(31, (1, 6, 16))
    gqa = orc.attend(q, cache, np.array([16]), 0, 0.3)
    mha = orc.Cache(1, 16, 6, 16, 8)
    for s in ("k", "v"):
        mha.data[s][:] = np.repeat(cache.data[s], 3, axis=2)
        mha.scales[s][:] = np.repeat(cache.scales[s], 3, axis=2)
    np.testing.assert_allclose(orc.attend(q, mha, np.array([16]), 0, 0.3), gqa, rtol=1e-13, atol=1e-14)


def test_fp32_store_is_plain_attention_over_fp16_values():
    """Strata PR 2698: the fp32 store runs plain attention on the values."""
    cache, k, v = _filled_cache(32, 1, 20, 1, 16, 16, [20], "fp32", "fp32")
    q = wl.uniform_rows(33, (1, 2, 16))
    out = orc.attend(q, cache, np.array([20]), 0, 0.25)
    want = orc.attend_one(q[0].astype(np.float64), k[0, :, 0].astype(np.float64),
                          v[0, :, 0].astype(np.float64), 0.25)
    np.testing.assert_array_equal(out[0], want)


@pytest.mark.parametrize("bounds", [[0, 200], [0, 1, 200], [0, 64, 128, 192, 200],
                                    [0, 0, 50, 50, 199, 200], [0, 7, 13, 100, 101, 200]])
def test_split_partials_combine_to_single_pass(bounds):
    """genie releases v1.3.0: split-K equals the single-block result."""
    cache, _, _ = _filled_cache(34, 1, 200, 1, 64, 64, [200], k_scale=3.0)
    q = wl.uniform_rows(35, (1, 4, 64))
    K = cache.values("k", 0, 0, 200, 0)
    V = cache.values("v", 0, 0, 200, 0)
    m, l, O = orc.split_partials(q[0], K, V, 0.125, bounds)
    got = orc.combine_partials(m, l, O)
    want = orc.attend_one(q[0].astype(np.float64), K, V, 0.125)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_empty_context_gives_zero_row():
    cache, _, _ = _filled_cache(36, 2, 8, 1, 16, 16, [0, 4])
    q = wl.uniform_rows(37, (2, 2, 16))
    out = orc.attend(q, cache, np.array([0, 4]), 0, 0.25)
    assert not out[0].any() and out[1].any()
    m, l, O = orc.split_partials(q[0], np.zeros((0, 16)), np.zeros((0, 16)), 0.25, [0, 0, 0])
    assert not orc.combine_partials(m, l, O).any()


def test_poison_outside_range_does_not_reach_output():
    cache, _, _ = _filled_cache(38, 1, 32, 1, 16, 16, [20], "fp32", "fp32")
    q = wl.uniform_rows(39, (1, 2, 16))
    ref = orc.attend(q, cache, np.array([20]), 8, 0.25)
    cache.data["k"][0, :12] = np.nan
    cache.data["v"][0, 20:] = np.nan
    out = orc.attend(q, cache, np.array([20]), 8, 0.25)
    np.testing.assert_array_equal(out, ref)


def test_page_byte_counts():
    g = json.load(open(os.path.join(GOLDEN, "page_byte_counts.json")))
    c = g["cell"]
    i8 = orc.cell_bytes(c["n_kv_heads_derived"], c["head_dim"], c["group"], "int8")
    f32 = orc.cell_bytes(c["n_kv_heads_derived"], c["head_dim"], c["group"], "fp32")
    assert i8 == c["int8_bytes"] and f32 == c["fp32_bytes"]
    assert round(f32 / i8, 1) == c["ratio_printed"]
    p = g["pool"]
    sh = p["shape_external"]
    body16, _ = orc.pool_bytes(sh["n_layers"], sh["ctx"], sh["n_kv_heads"], sh["head_dim"], "fp16")
    body8, sc4 = orc.pool_bytes(sh["n_layers"], sh["ctx"], sh["n_kv_heads"], sh["head_dim"], "int8", 4)
    assert body16 == p["fp16_mib"] * 2 ** 20
    assert body8 == p["int8_body_mib"] * 2 ** 20
    assert sc4 == p["scales_mib"] * 2 ** 20


def test_peaked_softmax_returns_argmax_row():
    """Scores spread by thousands: every weight but the top one underflows to
    exactly 0, so the output is the value row of the best-scoring key."""
    cache, _, _ = _filled_cache(40, 1, 48, 1, 32, 32, [48], k_scale=4.0)
    q = wl.uniform_rows(41, (1, 2, 32), 8.0)
    sm = 400.0
    out = orc.attend(q, cache, np.array([48]), 0, sm)
    K = cache.values("k", 0, 0, 48, 0)
    V = cache.values("v", 0, 0, 48, 0)
    for h in range(2):
        z = sm * (q[0, h].astype(np.float64) @ K.T)
        top = np.sort(z)[-2:]
        assert top[1] - top[0] > 800
        np.testing.assert_array_equal(out[0, h], V[int(np.argmax(z))])
