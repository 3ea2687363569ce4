"""Pins of the oracle's 4-bit stores: the Walsh-Hadamard rotation over 256
values and the Q4_0 block quantizer, and attention over rotated stores.

Strata PR 2698, "Not in this PR": q4_0 (both stores) and k8v4 (V only) use a
Hadamard rotation over head_dim 256 with Q4_0 blocks; K is rotated with the
queries, V is rotated and the output rotated back. The pins check the
rotation against scipy's Hadamard matrix and its float32 error bound, the
quantizer against exact rational arithmetic and closed-form blocks, and the
attention against scalar brute force in the unrotated basis."""
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

from oracle import kvq_oracle as orc
import workloads as wl

H256 = scipy.linalg.hadamard(256).astype(np.float64)


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_is_sylvester_matrix(n):
    np.testing.assert_array_equal(orc.hadamard(n), scipy.linalg.hadamard(n).astype(np.float64))


def test_exact_rotation_is_orthonormal_and_its_own_inverse():
    x = wl.uniform_rows(3, (5, 256), 2.0).astype(np.float64)
    y = orc.rotate_exact(x)
    np.testing.assert_allclose(y, x @ H256.T / 16.0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    np.testing.assert_allclose(orc.rotate_exact(y), x, rtol=0, atol=1e-13)


def test_float32_rotation_of_basis_vectors_is_exact():
    """A single nonzero input goes through every butterfly without rounding:
    the output is that column of H times the value / 16, exactly."""
    for i in range(256):
        e = np.zeros(256, dtype=np.float16)
        e[i] = 0.75
        got = orc.rotate_f32(e).astype(np.float64)
        np.testing.assert_array_equal(got, H256[:, i] * 0.75 / 16.0)


@pytest.mark.parametrize("scale", [1.0, 30.0, 1e-3])
def test_float32_rotation_within_summation_bound(scale):
    """Each output is a sum of 256 terms formed by a depth-8 addition tree in
    float32, so |error| <= 8 u sum|x| / 16 (u = 2^-24, first order)."""
    x = wl.uniform_rows(5, (64, 256), scale)
    want = x.astype(np.float64) @ H256.T / 16.0
    got = orc.rotate_f32(x).astype(np.float64)
    bound = 8 * 2.0 ** -24 * np.abs(x.astype(np.float64)).sum(axis=1, keepdims=True) / 16.0 * 1.001
    assert np.all(np.abs(got - want) <= bound)
    assert got.dtype == np.float64 and orc.rotate_f32(x).dtype == np.float32


def test_q4_integer_block_is_represented_exactly():
    """A block whose largest magnitude is a leading -8 has d = 1: integer values
    in [-8, 7] get codes value + 8 and dequantize exactly."""
    vals = np.array([-8] + [((j * 5) % 16) - 8 for j in range(1, 32)], dtype=np.float32)
    codes, d = orc.quantize_q4_0(vals)
    assert d.tolist() == [1.0]
    np.testing.assert_array_equal(codes, (vals + 8).astype(np.uint8))
    np.testing.assert_array_equal(orc.dequantize_q4_0(codes, d), vals.astype(np.float64))


def test_q4_halves_round_up():
    """Q4_0 adds 8.5 and truncates: with d = 1, k + 0.5 becomes k + 1 (round
    half up, not half to even)."""
    vals = np.zeros(32, dtype=np.float32)
    vals[0] = -8.0
    vals[1:6] = [2.5, -3.5, 0.5, -0.5, 6.5]
    codes, d = orc.quantize_q4_0(vals)
    assert d.tolist() == [1.0]
    assert codes[1:6].tolist() == [11, 5, 9, 8, 15]
    np.testing.assert_array_equal(orc.dequantize_q4_0(codes, d)[1:6], [3.0, -3.0, 1.0, 0.0, 7.0])


def test_q4_extreme_maps_to_code_zero_and_opposite_extreme_clamps():
    """d = m / -8 sends the extreme m itself to code 0; a value -m would need
    code 16 and clamps to 15 (error exactly |d|)."""
    vals = np.zeros(32, dtype=np.float32)
    vals[4], vals[9] = 3.0, -3.0
    codes, d = orc.quantize_q4_0(vals)
    assert d.tolist() == [-0.375]
    assert codes[4] == 0 and codes[9] == 15 and codes[0] == 8
    deq = orc.dequantize_q4_0(codes, d)
    assert deq[4] == 3.0 and deq[9] == -2.625


def test_q4_ties_take_the_first_extreme():
    for first, second in ((3.0, -3.0), (-3.0, 3.0)):
        vals = np.zeros(32, dtype=np.float32)
        vals[2], vals[7] = first, second
        codes, d = orc.quantize_q4_0(vals)
        assert float(d[0]) == first / -8.0
        assert codes[2] == 0 and codes[7] == 15


def test_q4_zero_block():
    codes, d = orc.quantize_q4_0(np.zeros(64, dtype=np.float32))
    assert np.all(codes == 8) and np.all(d == 0)
    assert np.all(orc.dequantize_q4_0(codes, d) == 0)


def test_q4_codes_against_exact_rationals():
    """Against exact arithmetic: code = min(15, floor(y / d + 8.5)) with d = the
    float32 m / -8 (exact, a power-of-two division), wherever y / d + 8.5 is not
    within 1e-5 of an integer (where float32 rounding may decide)."""
    y = orc.rotate_f32(wl.uniform_rows(9, (40, 256), 3.0))
    codes, dh = orc.quantize_q4_0(y)
    checked = 0
    for r in range(y.shape[0]):
        for blk in range(8):
            seg = [Fraction(float(v)) for v in y[r, 32 * blk:32 * blk + 32]]
            m = max(seg, key=abs)
            m = next(v for v in seg if abs(v) == abs(m))  # first of the largest magnitude
            d = m / -8
            for j, v in enumerate(seg):
                t = v / d + Fraction(17, 2)
                if abs(t - round(t)) < Fraction(1, 100000):
                    continue
                assert codes[r, 32 * blk + j] == min(15, math.floor(t))
                checked += 1
            assert float(dh[r, blk]) == float(np.float16(np.float32(float(d))))
    assert checked > 9000


def test_q4_reconstruction_error_bound():
    """Every value is within half a step of its dequantized value, except a
    clamped opposite extreme (within one step); steps are the stored fp16 d,
    plus the error of rounding d to fp16 (at most 8 |d - d16|)."""
    y = orc.rotate_f32(wl.uniform_rows(11, (50, 256), 5.0))
    codes, d16 = orc.quantize_q4_0(y)
    deq = orc.dequantize_q4_0(codes, d16)
    yb = y.astype(np.float64).reshape(50, 8, 32)
    db = np.abs(d16.astype(np.float64))[..., None]
    m = np.take_along_axis(yb, np.argmax(np.abs(yb), axis=-1)[..., None], axis=-1)
    d32 = np.abs(m / 8.0)
    err = np.abs(deq.reshape(50, 8, 32) - yb)
    slack = 8 * np.abs(d32 - db) + 1e-6 * db
    clamped = codes.reshape(50, 8, 32) == 15
    lim = np.where(clamped, db + slack, 0.5 * db + slack)
    assert np.all(err <= lim + 1e-12)
    assert np.all(codes <= 15)
    # the first extreme of each block gets code 0
    first = np.argmax(np.abs(yb), axis=-1)
    assert np.all(np.take_along_axis(codes.reshape(50, 8, 32), first[..., None], axis=-1) == 0)


def test_q4_nibble_layout():
    """Byte j of a 32-value block holds value j in its low nibble and value
    j + 16 in its high nibble."""
    codes = np.array([j % 16 for j in range(16)] + [15 - j for j in range(16)], dtype=np.uint8)
    second = np.array([15 - j for j in range(16)] + [j for j in range(16)], dtype=np.uint8)
    packed = orc.pack_q4(np.concatenate([codes, second]))
    assert packed.shape == (32,)
    assert packed[:4].tolist() == [0xF0, 0xE1, 0xD2, 0xC3]
    assert packed[15] == 0x0F
    assert packed[16:18].tolist() == [0x0F, 0x1E]
    assert packed[31] == 0xF0


def test_cache_rows_rotate_back_to_the_inputs_within_the_quantization_error():
    """Rotated back, a 4-bit store's rows are the appended fp16 rows up to the
    block rounding error (the rotation preserves the 2-norm), and they are not
    close without the rotation back."""
    B, ctx, Hkv, d = 1, 12, 2, 256
    cache = orc.Cache(B, ctx, Hkv, d, 64, "q4", "q4")
    k = wl.uniform_rows(21, (B, ctx, Hkv, d), 2.0)
    v = wl.uniform_rows(22, (B, ctx, Hkv, d))
    cache.append(k, v, np.zeros(B, dtype=np.int64))
    for s, x in (("k", k), ("v", v)):
        for h in range(Hkv):
            rows = cache.values(s, 0, 0, ctx, h)
            back = orc.rotate_exact(rows)
            d16 = np.abs(cache.scales[s][0, :, h].astype(np.float64))
            # a value with code 15 may be clamped (error <= |d|), the others are
            # within |d| / 2; each widened by 1% for the fp16 rounding of d
            n15 = (cache.data[s][0, :, h].reshape(ctx, 8, 32) == 15).sum(axis=2)
            bound = np.sqrt((n15 * (1.01 * d16) ** 2 + (32 - n15) * (0.505 * d16) ** 2).sum(axis=1)) + 1e-4
            err = np.linalg.norm(back - x[0, :, h].astype(np.float64), axis=1)
            assert np.all(err <= bound)
            assert np.all(np.linalg.norm(rows - x[0, :, h].astype(np.float64), axis=1) > 4 * bound)


def _brute_rows(cache, s, b, lo, hi, h):
    """Rows in the unrotated basis via scipy's H and scalar fsums."""
    if cache.dtypes[s] == "q4":
        out = []
        for p in range(lo, hi):
            c = cache.data[s][b, p, h].astype(np.int64) - 8
            dd = cache.scales[s][b, p, h].astype(np.float64)
            rot = [float(c[i]) * float(dd[i // 32]) for i in range(256)]
            out.append([math.fsum(H256[i, j] * rot[j] for j in range(256)) / 16.0 for i in range(256)])
        return out
    g = cache.group
    return [[float(c) * float(cache.scales[s][b, p, h][i // g]) for i, c in enumerate(cache.data[s][b, p, h])]
            for p in range(lo, hi)]


@pytest.mark.parametrize("kdt,vdt", [("q4", "q4"), ("int8", "q4"), ("q4", "int8")])
def test_attention_over_rotated_stores_matches_bruteforce(kdt, vdt):
    """Decode attention with rotated stores equals scalar attention of the
    original queries over the stores' rows rotated back (the rotation is
    orthogonal, so q.k is basis-free and the output lands in the original
    basis)."""
    B, ctx, Hq, Hkv, d = 1, 7, 4, 2, 256
    cache = orc.Cache(B, ctx, Hkv, d, 64, kdt, vdt)
    cache.append(wl.uniform_rows(31, (B, ctx, Hkv, d), 2.0), wl.uniform_rows(32, (B, ctx, Hkv, d)),
                 np.zeros(B, dtype=np.int64))
    q = wl.uniform_rows(33, (B, Hq, d))
    sm = 1.0 / 16.0
    L = 6
    got = orc.attend(q, cache, np.array([L]), 0, sm)
    for h in range(Hq):
        K = _brute_rows(cache, "k", 0, 0, L, h // 2)
        V = _brute_rows(cache, "v", 0, 0, L, h // 2)
        z = [sm * math.fsum(float(a) * b for a, b in zip(q[0, h], kr)) for kr in K]
        mx = max(z)
        e = [math.exp(t - mx) for t in z]
        den = math.fsum(e)
        want = [math.fsum(e[p] * V[p][i] for p in range(L)) / den for i in range(d)]
        np.testing.assert_allclose(got[0, h], want, rtol=0, atol=1e-12)


def test_chunk_attention_over_rotated_stores_is_decode_attention_per_token():
    B, ctx, T, Hq, Hkv, d = 1, 20, 3, 4, 1, 256
    cache = orc.Cache(B, ctx, Hkv, d, 64, "int8", "q4")
    cache.append(wl.uniform_rows(41, (B, ctx, Hkv, d), 2.0), wl.uniform_rows(42, (B, ctx, Hkv, d)),
                 np.zeros(B, dtype=np.int64))
    q = wl.uniform_rows(43, (B, T, Hq, d))
    start = np.array([9])
    got = orc.attend_chunk(q, cache, start, 5, 0.1)
    for t in range(T):
        np.testing.assert_allclose(got[:, t], orc.attend(q[:, t], cache, start + t + 1, 5, 0.1), rtol=0, atol=1e-13)


def test_q4_store_needs_head_dim_256_and_cell_bytes():
    with pytest.raises(ValueError):
        orc.Cache(1, 4, 1, 128, 64, "q4", "q4")
    # 128 bytes of codes + 8 fp16 scales per kv head: 4.5 bits per value
    assert orc.cell_bytes(1, 256, 64, "q4") == 144
    assert orc.cell_bytes(2, 256, 64, "q4") * 8 == 2 * 256 * 4.5
