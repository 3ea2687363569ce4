"""Pins of the oracle's chunk attention (several consecutive query tokens per
sequence, causal inside the chunk): scalar brute force on tiny inputs, the
reduction of each token to single-token decode attention, causality under
perturbation, the window's limits and a constructed closed form.

Strata PR 2698, "What it does": the prompt chunk and the verify windows read
the same int8 cache, dequantized on the fly."""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import kvq_oracle as orc
import workloads as wl


def _brute_row(cache, s, b, p, hk, g):
    if cache.dtypes[s] == "int8":
        codes, scales = cache.data[s][b, p, hk], cache.scales[s][b, p, hk]
        return [float(Fraction(int(c)) * Fraction(float(scales[i // g]))) for i, c in enumerate(codes.tolist())]
    return [float(x) for x in cache.data[s][b, p, hk]]


def _brute_token(q_row, keys, vals, sm):
    z = [sm * math.fsum(float(a) * float(b) for a, b in zip(q_row, k)) for k in keys]
    mx = max(z)
    e = [math.exp(t - mx) for t in z]
    den = math.fsum(e)
    return [math.fsum(e[p] * vals[p][i] for p in range(len(vals))) / den for i in range(len(vals[0]))]


def _cache(seed, B, max_ctx, Hkv, d, g, kdt="int8", vdt="int8"):
    cache = orc.Cache(B, max_ctx, Hkv, d, g, kdt, vdt)
    k = wl.uniform_rows(seed, (B, max_ctx, Hkv, d), 2.0)
    v = wl.uniform_rows(seed + 1, (B, max_ctx, Hkv, d))
    cache.append(k, v, np.zeros(B, dtype=np.int64))
    return cache


@pytest.mark.parametrize("case", [
    dict(B=2, T=3, Hq=4, Hkv=2, d=16, g=8, start=[4, 0], W=0),
    dict(B=1, T=4, Hq=6, Hkv=3, d=8, g=8, start=[5], W=3),
    dict(B=2, T=2, Hq=4, Hkv=1, d=16, g=16, start=[6, 2], W=5),
    dict(B=1, T=3, Hq=2, Hkv=2, d=8, g=4, start=[2], W=0, kdt="fp32", vdt="int8"),
    dict(B=1, T=3, Hq=4, Hkv=2, d=8, g=4, start=[3], W=2, kdt="int8", vdt="fp32"),
])
def test_chunk_matches_bruteforce(case):
    """Every (sequence, token, head) against scalar softmax over the keys
    lo <= p <= start + t, with the rows dequantized by exact rationals."""
    B, T, Hq, Hkv, d, g, W = (case[k] for k in ("B", "T", "Hq", "Hkv", "d", "g", "W"))
    start = np.array(case["start"])
    cache = _cache(31, B, 10, Hkv, d, g, case.get("kdt", "int8"), case.get("vdt", "int8"))
    q = wl.uniform_rows(32, (B, T, Hq, d))
    sm = 1.0 / math.sqrt(d)
    got = orc.attend_chunk(q, cache, start, W, sm)
    G = Hq // Hkv
    for b in range(B):
        for t in range(T):
            P = int(start[b]) + t
            lo = P + 1 - W if (W and P + 1 > W) else 0
            for h in range(Hq):
                keys = [_brute_row(cache, "k", b, p, h // G, g) for p in range(lo, P + 1)]
                vals = [_brute_row(cache, "v", b, p, h // G, g) for p in range(lo, P + 1)]
                want = _brute_token(q[b, t, h].astype(np.float64), keys, vals, sm)
                np.testing.assert_allclose(got[b, t, h], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("W", [0, 7, 40])
def test_each_token_is_decode_attention_at_its_own_position(W):
    """Token t of the chunk equals single-token decode attention (the pinned
    decode oracle, written separately) at context start + t + 1, for every t:
    the first, the interior and the last token of the chunk."""
    B, T, Hq, Hkv, d, g = 2, 6, 8, 2, 32, 16
    cache = _cache(41, B, 64, Hkv, d, g)
    start = np.array([20, 57])
    q = wl.uniform_rows(42, (B, T, Hq, d))
    got = orc.attend_chunk(q, cache, start, W, 0.2)
    for t in range(T):
        want = orc.attend(q[:, t], cache, start + t + 1, W, 0.2)
        np.testing.assert_allclose(got[:, t], want, rtol=0, atol=1e-13)


def test_causal_keys_after_a_token_do_not_reach_it():
    """Overwriting the cache at position start + k changes tokens t >= k and
    leaves tokens t < k bit-identical."""
    B, T, Hq, Hkv, d, g = 1, 8, 4, 2, 32, 32
    cache = _cache(51, B, 40, Hkv, d, g)
    start = np.array([30])
    q = wl.uniform_rows(52, (B, T, Hq, d))
    before = orc.attend_chunk(q, cache, start, 0, 0.3)
    k = 5
    cache.append(wl.uniform_rows(53, (B, 1, Hkv, d), 3.0), wl.uniform_rows(54, (B, 1, Hkv, d), 3.0),
                 start + k)
    after = orc.attend_chunk(q, cache, start, 0, 0.3)
    np.testing.assert_array_equal(after[0, :k], before[0, :k])
    assert np.all(np.abs(after[0, k:] - before[0, k:]).max(axis=(1, 2)) > 1e-6)


def test_window_covering_everything_is_no_window_and_window_one_is_own_row():
    B, T, Hq, Hkv, d, g = 1, 5, 4, 2, 16, 16
    cache = _cache(61, B, 30, Hkv, d, g)
    start = np.array([20])
    q = wl.uniform_rows(62, (B, T, Hq, d))
    np.testing.assert_array_equal(orc.attend_chunk(q, cache, start, 25, 0.25),
                                  orc.attend_chunk(q, cache, start, 0, 0.25))
    # W = 1: each token attends only to its own position -> its value row
    out = orc.attend_chunk(q, cache, start, 1, 0.25)
    for t in range(T):
        for h in range(Hq):
            np.testing.assert_array_equal(out[0, t, h], cache.values("v", 0, 20 + t, 21 + t, h // 2)[0])


def test_zero_query_is_the_mean_of_the_attended_rows():
    """q = 0: equal weights, so token t's output is the mean of the value rows
    lo..start+t (a closed form that does not go through the softmax code)."""
    B, T, Hq, Hkv, d, g = 1, 4, 2, 1, 8, 8
    cache = _cache(71, B, 16, Hkv, d, g)
    start = np.array([9])
    q = np.zeros((B, T, Hq, d), dtype=np.float16)
    out = orc.attend_chunk(q, cache, start, 6, 1.0)
    for t in range(T):
        P = 9 + t
        rows = [_brute_row(cache, "v", 0, p, 0, g) for p in range(P + 1 - 6, P + 1)]
        want = [math.fsum(r[i] for r in rows) / len(rows) for i in range(d)]
        for h in range(Hq):
            np.testing.assert_allclose(out[0, t, h], want, rtol=0, atol=1e-14)
