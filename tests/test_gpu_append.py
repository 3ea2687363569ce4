"""kv_quant_append on the GPU against the CPU oracle: codes and fp16 scales
bit-exact, fp32 stores exact, nothing written outside the target rows."""
import json
import os

import numpy as np
import pytest

import workloads as wl
from oracle import kvq_oracle as orc

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _setup():
    import kvq_setup
    return kvq_setup


def _check_rows(lay, cache, w, b, positions, k_rows, v_rows):
    ks = _setup()
    for s, rows in (("k", k_rows), ("v", v_rows)):
        dt = w.k_dtype if s == "k" else w.v_dtype
        for h in range(w.n_kv_heads):
            got = ks.rows_of(lay, cache[s], b, positions, h)
            if dt == "int8":
                want_c, want_s = orc.quantize_rows(rows[:, h], w.scale_group)
                np.testing.assert_array_equal(got, want_c, err_msg=f"{w.name} {s} codes h={h}")
                gs = ks.scales_of(lay, cache[s + "_scales"], b, positions, h)
                np.testing.assert_array_equal(gs.view(np.uint16), want_s.view(np.uint16),
                                              err_msg=f"{w.name} {s} scales h={h}")
            else:
                np.testing.assert_array_equal(got, rows[:, h].astype(np.float32))


@pytest.mark.parametrize("name", ["tiny", "gemma"])
def test_append_full_cache_bit_exact(name):
    ks = _setup()
    w = wl.WORKLOADS[name]
    L = w.contexts[-1]
    lens = np.full(w.batch, L, dtype=np.int32)
    print(f"[append] {name} L={L}", flush=True)
    lay, cache = ks.fill_cache(w, lens, block=1000, fill=0x55)
    pos = np.arange(L)
    _check_rows(lay, cache, w, 0, pos, wl.kv_rows(w, "k", 0, 0, L), wl.kv_rows(w, "v", 0, 0, L))
    # slot tail [head_dim, slot_dim) and positions >= L keep the canary
    if w.slot_dim > w.head_dim:
        for h in range(w.n_kv_heads):
            full = ks.rows_of(lay, cache["k"], 0, pos[::97], h, width=w.slot_dim)
            assert (full[:, w.head_dim:] == 0x55).all()
    if L < w.max_ctx:
        tail = ks.rows_of(lay, cache["v"], 0, np.arange(L, w.max_ctx), 0)
        assert (tail == 0x55).all()


def test_append_long_context_outlier_channels_sampled():
    """Long workload (K with 1 % outlier channels x20), group-64 scales, full
    131072 positions appended; 4096 sampled positions compared bit-exactly."""
    ks = _setup()
    w = wl.WORKLOADS["long"]
    L = w.contexts[-1]
    print("[append] long full size", flush=True)
    lay, cache = ks.fill_cache(w, np.array([L], dtype=np.int32))
    rng = np.random.default_rng(5)
    pos = np.unique(np.concatenate([rng.integers(0, L, 4096), [0, L - 1]]))
    k_all = wl.kv_rows(w, "k", 0, 0, L)
    v_all = wl.kv_rows(w, "v", 0, 0, L)
    _check_rows(lay, cache, w, 0, pos, k_all[pos], v_all[pos])


def test_append_batched_ragged_sampled():
    ks = _setup()
    w = wl.WORKLOADS["batched"]
    lens = wl.seq_lens(w)
    seqs = (int(np.argmin(lens)), int(np.argmax(lens)), 17)
    print(f"[append] batched {w.batch} seqs, sampled {seqs}", flush=True)
    lay, cache = ks.fill_cache(w, lens, seqs=seqs)
    rng = np.random.default_rng(6)
    for b in seqs:
        L = int(lens[b])
        pos = np.unique(rng.integers(0, L, 512))
        k = wl.kv_rows(w, "k", b, 0, L)[pos]
        v = wl.kv_rows(w, "v", b, 0, L)[pos]
        _check_rows(lay, cache, w, b, pos, k, v)


@pytest.mark.parametrize("name", ["mixed_k8v32", "mixed_k32v8"])
def test_append_chunk_mixed_stores(name):
    """Mixed stores: 30000 positions, then a 2048-token chunk at position 30000
    (one store int8 group-64, the other fp32 holding the fp16 values)."""
    ks = _setup()
    w = wl.WORKLOADS[name]
    print(f"[append] {name}", flush=True)
    lay, cache = ks.fill_cache(w, np.array([w.prefill]), fill=0x55)
    k = wl.kv_rows(w, "k", 0, w.prefill, w.append)
    v = wl.kv_rows(w, "v", 0, w.prefill, w.append)
    ks.append_rows(lay, cache, 0, w.prefill, k, v)
    _check_rows(lay, cache, w, 0, np.arange(w.prefill, w.prefill + w.append), k, v)
    # the positions after the chunk are untouched
    rest = np.arange(w.prefill + w.append, w.max_ctx)
    st = "k" if w.k_dtype == "int8" else "v"
    assert (ks.rows_of(lay, cache[st], 0, rest, 1) == 0x55).all()


def _append_host(rows, group, n_kv=1):
    """Quantize-append rows [n][n_kv][d] at positions 0..n-1 of a fresh cache."""
    import int8_quantized_kv_quant_amd as kvq
    ks = _setup()
    n, _, d = rows.shape
    lay = kvq.make_layout(n_kv, d, n, 1, scale_group=group)
    cache = kvq.alloc_cache(lay, 1)
    ks.append_rows(lay, cache, 0, 0, rows, rows)
    return lay, cache


def test_append_tie_case_golden():
    g = json.load(open(os.path.join(GOLDEN, "tie_case.json")))
    row = np.zeros((1, 1, 64), dtype=np.float16)
    row[0, 0, :len(g["group"])] = np.array(g["group"], dtype=np.float16)
    lay, cache = _append_host(row, 64)
    ks = _setup()
    codes = ks.rows_of(lay, cache["k"], 0, [0], 0)[0]
    assert codes[:len(g["codes"])].tolist() == g["codes"]
    sc = ks.scales_of(lay, cache["k_scales"], 0, [0], 0)
    assert hex(int(sc.view(np.uint16)[0, 0])) == g["scale_bits"]


@pytest.mark.parametrize("group,d", [(64, 256), (256, 256), (64, 128), (128, 128), (64, 64)])
def test_append_wide_dynamic_range(group, d):
    """Groups spanning 1e-7 .. 4e4 in magnitude (subnormal and zero scales,
    clamp engaged, large values), plus exact ties built on power-of-two scales."""
    rng = np.random.default_rng(group + d)
    n = 512
    mag = 10.0 ** rng.uniform(-7, 4.6, (n, 1, d // 64, 1))
    x = (rng.standard_normal((n, 1, d // 64, 64)) * mag).reshape(n, 1, d)
    x[::7] = 0.0                                   # all-zero rows
    x[3::11, :, :5] = 65504.0                      # fp16 max
    x[5::13] *= 1e-4                               # tiny groups
    x = np.clip(x, -65504, 65504).astype(np.float16)
    # exact half-way points: absmax 127/64 gives scale 1/64; k/128 lands on ties
    x[1, 0, :8] = np.array([1.984375, 0.0390625, 0.0546875, -0.0390625, -0.0546875, 0.0078125, 0, 0],
                           dtype=np.float16)
    lay, cache = _append_host(x, group)
    ks = _setup()
    got_c = ks.rows_of(lay, cache["k"], 0, np.arange(n), 0)
    got_s = ks.scales_of(lay, cache["k_scales"], 0, np.arange(n), 0)
    want_c, want_s = orc.quantize_rows(x[:, 0], group)
    np.testing.assert_array_equal(got_s.view(np.uint16), want_s.view(np.uint16))
    np.testing.assert_array_equal(got_c, want_c)


def test_append_zero_row_after_large_row_and_per_head_scales():
    """Regressions of genie v0.1.0-alpha.12 #64 (uninitialised row max) and
    v0.1.0-alpha.11 (rows=1 instead of one row per kv head)."""
    x = np.zeros((4, 3, 128), dtype=np.float16)
    x[0] = 1000.0
    x[2, 1] = wl.uniform_rows(3, (128,), 100.0)
    x[2, 0] = wl.uniform_rows(4, (128,), 0.01)
    x[3] = wl.uniform_rows(5, (3, 128))
    lay, cache = _append_host(x, 128, n_kv=3)
    ks = _setup()
    for h in range(3):
        got = ks.scales_of(lay, cache["k_scales"], 0, np.arange(4), h)
        _, want = orc.quantize_rows(x[:, h], 128)
        np.testing.assert_array_equal(got.view(np.uint16), want.view(np.uint16))
    assert float(ks.scales_of(lay, cache["k_scales"], 0, [1], 0)[0, 0]) == 0.0


def test_append_out_of_range_positions_are_not_written():
    import int8_quantized_kv_quant_amd as kvq
    lay = kvq.make_layout(2, 64, 16, 2, scale_group=64)
    cache = kvq.alloc_cache(lay, 2, fill=0x55)
    rows = wl.uniform_rows(9, (2, 4, 2, 64))
    kn = torch.from_numpy(rows).cuda()
    sp = torch.tensor([14, 3], dtype=torch.int32, device="cuda")   # seq 0: positions 14..17
    kvq.kv_quant_append(lay, cache["k"], cache["v"], cache["k_scales"], cache["v_scales"], kn, kn, sp, 2, 4)
    ks = _setup()
    for b, p0 in ((0, 14), (1, 3)):
        for h in range(2):
            ok = [p for p in range(p0, p0 + 4) if p < 16]
            want, _ = orc.quantize_rows(rows[b, :len(ok), h], 64)
            np.testing.assert_array_equal(ks.rows_of(lay, cache["k"], b, ok, h), want)
            others = [p for p in range(16) if p not in ok]
            assert (ks.rows_of(lay, cache["k"], b, others, h) == 0x55).all()


# Scales with at most three significant bits: absmax = 127 * s is an fp16
# value whose quotient by 127 is s exactly, and every (k + 1/2) * s with
# |k + 1/2| <= 126.5 is an fp16 value, so x / s lands exactly half-way between
# two codes. 6 * 2^-24 is a subnormal scale.
TIE_SCALES = (2.0 ** -6, 3 * 2.0 ** -8, 5 * 2.0 ** -9, 7 * 2.0 ** -9, 6 * 2.0 ** -24, 2.0 ** 4, 96.0)


def _tie_rows(d, group, n_kv, seed):
    """Rows [n][n_kv][d] whose groups each hold one +-127*s element and, for
    the rest, exact ties (k + 1/2) * s; together they take every tie value
    -126.5 .. 126.5 of every scale in TIE_SCALES."""
    rng = np.random.default_rng(seed)
    groups = []
    for s in TIE_SCALES:
        ties = (np.arange(-127, 127) + 0.5) * s
        rng.shuffle(ties)
        for i in range(0, len(ties), group - 1):
            part = ties[i:i + group - 1]
            g = np.concatenate([[127 * s * rng.choice([-1.0, 1.0])], part,
                                rng.choice(ties, group - 1 - len(part))])
            rng.shuffle(g)
            groups.append(g)
    per_row = n_kv * d // group
    while len(groups) % per_row:
        groups.append(groups[len(groups) % len(TIE_SCALES)])
    x = np.concatenate(groups).reshape(-1, n_kv, d)
    x16 = x.astype(np.float16)
    assert np.array_equal(x16.astype(np.float64), x), "tie values must be exact in fp16"
    return x16


def _assert_ties(x, group):
    """The oracle on the tie rows: every scale is one of TIE_SCALES, every
    non-max element sits exactly half-way, and its code is the even neighbour."""
    c, s = orc.quantize_rows(x, group)
    s64 = np.repeat(s.astype(np.float64), group, axis=-1)
    assert set(np.unique(s.astype(np.float64))) <= set(TIE_SCALES)
    q = x.astype(np.float64) / s64
    tie = np.abs(q) < 127
    assert np.all(q[tie] - np.floor(q[tie]) == 0.5)
    assert np.all(c[tie] % 2 == 0) and np.all(np.abs(c[tie] - q[tie]) == 0.5)
    return c, s


@pytest.mark.parametrize("group,d,v_dtype", [(64, 256, "int8"), (128, 128, "int8"), (256, 256, "int8"),
                                             (64, 64, "int8"), (256, 256, "q4")])
def test_append_every_exact_tie(group, d, v_dtype):
    """Every exact half-way quotient of several scales rounds to the even code,
    as in the oracle, through the append kernel (int8 stores, and the int8 K of
    a layout whose V is a 4-bit store)."""
    import int8_quantized_kv_quant_amd as kvq
    ks = _setup()
    x = _tie_rows(d, group, 2, seed=group + d)
    n = x.shape[0]
    lay = kvq.make_layout(2, d, n, 1, v_dtype=v_dtype, scale_group=group)
    cache = kvq.alloc_cache(lay, 1)
    v = np.ascontiguousarray(x[::-1])
    ks.append_rows(lay, cache, 0, 0, x, v)
    for s, rows in (("k", x), ("v", v)) if v_dtype == "int8" else (("k", x),):
        for h in range(2):
            want_c, want_s = _assert_ties(rows[:, h], group)
            np.testing.assert_array_equal(ks.rows_of(lay, cache[s], 0, np.arange(n), h), want_c,
                                          err_msg=f"{s} codes h={h}")
            got_s = ks.scales_of(lay, cache[s + "_scales"], 0, np.arange(n), h)
            np.testing.assert_array_equal(got_s.view(np.uint16), want_s.view(np.uint16))


@pytest.mark.parametrize("group,d", [(64, 128), (256, 256)])
def test_fused_step_every_exact_tie(group, d):
    """The fused decode step appends tie rows at L_b - 1 with the same codes."""
    import int8_quantized_kv_quant_amd as kvq
    ks = _setup()
    n_kv, n_q = 2, 8
    x = _tie_rows(d, group, n_kv, seed=7 * group + d)
    lens = np.array([1, 129, 700, 2049] * ((x.shape[0] + 3) // 4))[:x.shape[0]]
    batch = len(lens)
    lay = kvq.make_layout(n_kv, d, int(lens.max()), batch, scale_group=group)
    cache = kvq.alloc_cache(lay, batch)
    for b, L in enumerate(lens):
        if L > 1:
            rows = wl.uniform_rows(100 + b, (int(L) - 1, n_kv, d))
            ks.append_rows_device(lay, cache, b, 0, torch.from_numpy(rows).cuda(),
                                  torch.from_numpy(rows).cuda())
    k_new = torch.from_numpy(x).cuda()
    v_new = torch.from_numpy(np.ascontiguousarray(-x)).cuda()
    q = torch.from_numpy(wl.uniform_rows(3, (batch, n_q, d))).cuda()
    ld = torch.from_numpy(lens.astype(np.int32)).cuda()
    kvq.decode(lay, cache, q, ld, 0, new_kv=(k_new, v_new), n_cu=ks.n_cu())
    torch.cuda.synchronize()
    for s, rows in (("k", x), ("v", -x)):
        for h in range(n_kv):
            want_c, want_s = _assert_ties(rows[:, h], group)
            for b, L in enumerate(lens):
                got = ks.rows_of(lay, cache[s], b, [int(L) - 1], h)[0]
                np.testing.assert_array_equal(got, want_c[b], err_msg=f"{s} b={b} h={h}")
                got_s = ks.scales_of(lay, cache[s + "_scales"], b, [int(L) - 1], h)[0]
                np.testing.assert_array_equal(got_s.view(np.uint16), want_s[b].view(np.uint16))
