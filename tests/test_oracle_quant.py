"""Pins of the oracle's quantization against what the pages and arithmetic fix.

Nothing here re-types the oracle's formula: the scale is checked against exact
rational rounding over every fp16 value, the codes against a brute-force
nearest-code search, and both against invariants and a constructed tie case.
"""
import bisect
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import kvq_oracle as orc
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# All non-negative finite fp16 values, in increasing order of value.
_POS_BITS = np.arange(0, 0x7C00, dtype=np.uint16)
_POS_F16 = _POS_BITS.view(np.float16)
_POS_FRAC = [Fraction(float(v)) for v in _POS_F16]


def _round_to_f16_exact(fr: Fraction) -> np.float16:
    """Nearest non-negative fp16 to the rational fr, ties to even bit pattern."""
    i = bisect.bisect_left(_POS_FRAC, fr)
    if i < len(_POS_FRAC) and _POS_FRAC[i] == fr:
        return _POS_F16[i]
    lo, hi = i - 1, i
    dl, dh = fr - _POS_FRAC[lo], _POS_FRAC[hi] - fr
    if dl < dh:
        return _POS_F16[lo]
    if dh < dl:
        return _POS_F16[hi]
    return _POS_F16[lo] if _POS_BITS[lo] % 2 == 0 else _POS_F16[hi]


def _brute_codes(xs, s):
    """For each x, the integer c in [-127, 127] minimising |x - c*s| exactly,
    ties to even c; all zero when s == 0."""
    sF = Fraction(float(s))
    out = []
    for x in xs:
        xF = Fraction(float(x))
        if sF == 0:
            out.append(0)
            continue
        best, bestd = None, None
        for c in range(-127, 128):
            dd = abs(xF - c * sF)
            if bestd is None or dd < bestd or (dd == bestd and c % 2 == 0):
                best, bestd = c, dd
        out.append(best)
    return out


def test_scale_exhaustive_all_fp16_absmax():
    """Every non-negative finite fp16 absmax: the oracle's scale is the exact
    nearest fp16 to absmax/127 (Strata PR 2698: scale = group absmax / 127)."""
    got = orc.scale_from_absmax(_POS_F16)
    want = np.array([_round_to_f16_exact(f / 127) for f in _POS_FRAC], dtype=np.float16)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_scale_via_fp32_division_is_exact_for_fp16_inputs():
    """Reading r1: dividing in fp32 (correctly rounded) and rounding the result
    to fp16 gives the same scale as the exact quotient, for every fp16 absmax.
    This is the arithmetic a device kernel can use."""
    via32 = (_POS_F16.astype(np.float32) / np.float32(127.0)).astype(np.float16)
    assert np.array_equal(via32.view(np.uint16), orc.scale_from_absmax(_POS_F16).view(np.uint16))


def test_tie_case_golden():
    g = json.load(open(os.path.join(GOLDEN, "tie_case.json")))
    x = np.array([g["group"]], dtype=np.float16)
    c, s = orc.quantize_rows(x, len(g["group"]))
    assert float(s[0, 0]) == g["scale"]
    assert hex(int(s.view(np.uint16)[0, 0])) == g["scale_bits"]
    assert c[0].tolist() == g["codes"]
    assert _brute_codes(x[0], s[0, 0]) == g["codes"]


@pytest.mark.parametrize("seed", range(6))
def test_codes_match_bruteforce(seed):
    rng = np.random.default_rng(seed)
    scale = [1.0, 1e-2, 3.0, 1e-5, 40.0, 1.0][seed]
    x = (rng.standard_normal((6, 16)) * scale).astype(np.float16)
    if seed == 5:  # outlier element dominating the group
        x[:, 3] *= np.float16(20)
    for g in (16, 8):
        c, s = orc.quantize_rows(x, g)
        for r in range(x.shape[0]):
            for j in range(16 // g):
                blk = x[r, j * g:(j + 1) * g]
                assert c[r, j * g:(j + 1) * g].tolist() == _brute_codes(blk, s[r, j]), (r, j)
                a = Fraction(float(np.abs(blk.astype(np.float64)).max()))
                assert s[r, j] == _round_to_f16_exact(a / 127)


def test_code_rounding_fp32_division_equals_exact_rne():
    """Reading r3: rint(fp32(x) / fp32(s)) equals exact round-half-even of x/s
    for fp16 x and s in the range quantization produces (s = fp16(a/127),
    |x| <= a). Checked on random pairs plus every exact tie of a scale grid."""
    rng = np.random.default_rng(7)
    a = np.abs(rng.standard_normal(200_000).astype(np.float32) * np.float32(4)).astype(np.float16)
    a = a[a > np.float16(0.01)]
    s = orc.scale_from_absmax(a)
    x = (rng.uniform(-1, 1, a.shape).astype(np.float32) * a.astype(np.float32)).astype(np.float16)
    # add exact half-way points k/2 * s for a few scales
    ks = np.arange(-253, 254, 2) / 2.0
    grid = np.array([2.0 ** -e * (8 + m) / 8 for e in range(3, 14) for m in range(8)])
    s_all = np.concatenate([s[:400], grid.astype(np.float16)])
    n_s = s_all.size
    s_t = np.repeat(s_all, ks.size)
    x_t = (np.tile(ks, n_s) * s_t.astype(np.float64)).astype(np.float16)
    keep = x_t.astype(np.float64) == np.tile(ks, n_s) * s_t.astype(np.float64)
    xs = np.concatenate([x, x_t[keep]])
    ss = np.concatenate([s, s_t[keep]])
    via32 = np.clip(np.rint(xs.astype(np.float32) / ss.astype(np.float32)), -127, 127)
    exact = np.clip(np.rint(xs.astype(np.float64) / ss.astype(np.float64)), -127, 127)
    assert keep.sum() > 10_000, keep.sum()
    assert np.array_equal(via32, exact)
    # spot-check the float64 rint against Fractions on the ties
    for xv, sv in list(zip(x_t[keep], s_t[keep]))[:300]:
        q = Fraction(float(xv)) / Fraction(float(sv))
        assert q.denominator in (1, 2)
        assert _brute_codes([xv], sv)[0] == int(np.clip(np.rint(float(q)), -127, 127))


def _normal_groups(seed, shape, scale=1.0):
    return wl.uniform_rows(seed, shape, scale)


@pytest.mark.parametrize("g", [64, 256])
def test_invariants_code_range_and_error(g):
    x = _normal_groups(101, (64, 4, 256))
    c, s = orc.quantize_rows(x, g)
    xg = x.astype(np.float64).reshape(64, 4, 256 // g, g)
    cg = c.astype(np.int64).reshape(xg.shape)
    sg = s.astype(np.float64)[..., None]
    assert np.abs(cg).max() <= 127
    # 127 is reached at the absmax element of every group with a normal scale
    amax = np.abs(xg).max(axis=-1)
    assert (amax >= 7.7515e-3).all()
    at = np.take_along_axis(np.abs(cg), np.abs(xg).argmax(axis=-1)[..., None], -1)[..., 0]
    assert (at == 127).all()
    # per-element error at most half a scale step
    assert (np.abs(xg - cg * sg) <= sg / 2).all()


def test_per_position_scale_is_max_of_group_scales():
    x = _normal_groups(102, (32, 2, 256))
    _, s64 = orc.quantize_rows(x, 64)
    _, s256 = orc.quantize_rows(x, 256)
    assert np.array_equal(s256[..., 0], s64.max(axis=-1))


@pytest.mark.parametrize("k", [-3, -1, 1, 4])
def test_power_of_two_scaling(k):
    x = _normal_groups(104, (8, 2, 128))
    c0, s0 = orc.quantize_rows(x, 64)
    xk = (x.astype(np.float64) * 2.0 ** k).astype(np.float16)
    assert np.array_equal(xk.astype(np.float64), x.astype(np.float64) * 2.0 ** k)
    ck, sk = orc.quantize_rows(xk, 64)
    assert np.array_equal(c0, ck)
    assert np.array_equal(sk.astype(np.float64), s0.astype(np.float64) * 2.0 ** k)


def test_zero_row_after_large_row_gets_zero_scale():
    """Regression for the uninitialised row maximum of the genie conversion
    kernel (v0.1.0-alpha.12 'Path I series' #64): each row starts afresh."""
    x = np.zeros((2, 1, 64), dtype=np.float16)
    x[0] = np.float16(1000.0)
    c, s = orc.quantize_rows(x, 64)
    assert float(s[1, 0, 0]) == 0.0 and not c[1].any()
    assert (c[0] == 127).all()


def test_each_kv_head_gets_its_own_scale():
    """Regression for rows=1 instead of rows=n_kv_heads (genie v0.1.0-alpha.11
    '--int8-kv triage'): heads of different magnitude keep separate scales."""
    x = _normal_groups(105, (4, 3, 64))
    x[:, 1] = (x[:, 1].astype(np.float32) * 100).astype(np.float16)
    _, s = orc.quantize_rows(x, 64)
    ratio = s[:, 1, 0].astype(np.float64) / s[:, 0, 0].astype(np.float64)
    assert (ratio > 10).all()
    # the small head still uses its full code range
    c, _ = orc.quantize_rows(x, 64)
    assert (np.abs(c[:, 0]).max(axis=-1) == 127).all()


def test_tiny_and_subnormal_groups():
    """Reading r5: absmax <= ~3.755e-6 gives scale 0 and zero codes; subnormal
    scales engage the clamp, which the brute-force search (limited to
    [-127, 127]) agrees with."""
    for a in (0.0, 3.0e-6, 3.7e-6):
        x = np.array([[a, -a / 2, a / 4, 0.0]], dtype=np.float16)
        c, s = orc.quantize_rows(x, 4)
        assert float(s[0, 0]) == 0.0 and not c.any()
    for a in (4e-6, 1e-5, 6e-5, 5e-4, 7e-3):
        rng = np.random.default_rng(int(a * 1e7))
        x = np.concatenate([[a], rng.uniform(-a, a, 15)]).astype(np.float16)[None]
        c, s = orc.quantize_rows(x, 16)
        assert float(s[0, 0]) > 0
        assert c[0].tolist() == _brute_codes(x[0], s[0, 0])


def test_dequantize_is_exact_product():
    x = _normal_groups(106, (3, 2, 128))
    c, s = orc.quantize_rows(x, 64)
    xh = orc.dequantize_rows(c, s, 64)
    for idx in [(0, 0, 0), (1, 1, 77), (2, 0, 127), (2, 1, 64)]:
        j = idx[-1] // 64
        want = Fraction(int(c[idx])) * Fraction(float(s[idx[:-1] + (j,)]))
        assert Fraction(xh[idx]) == want


def test_cache_append_places_rows_and_leaves_others():
    cache = orc.Cache(2, 16, 2, 64, 64)
    k = _normal_groups(107, (2, 3, 2, 64))
    v = _normal_groups(108, (2, 3, 2, 64))
    cache.append(k, v, np.array([5, 0]))
    c, s = orc.quantize_rows(k[0], 64)
    assert np.array_equal(cache.data["k"][0, 5:8], c)
    assert np.array_equal(cache.scales["k"][0, 5:8].view(np.uint16), s.view(np.uint16))
    assert not cache.data["k"][0, :5].any() and not cache.data["k"][0, 8:].any()
    mixed = orc.Cache(1, 8, 2, 64, 64, k_dtype="fp32", v_dtype="int8")
    mixed.append(k[:1], v[:1], np.array([2]))
    assert np.array_equal(mixed.data["k"][0, 2:5], k[0].astype(np.float32))
    assert mixed.scales["k"] is None
