"""4-bit stores on the GPU against the CPU oracle (Strata PR 2698, "Not in this
PR": q4_0 and k8v4 with a Hadamard rotation over head_dim 256).

kv_quant_append into a q4 store: the packed Q4_0 bytes and the fp16 block
scales bit-exact with the oracle's rotation (fp32 butterflies) and quantizer,
including rows built to give exact ties, zero blocks and extreme magnitudes;
nothing written outside the target rows."""
import numpy as np
import pytest

import workloads as wl
from oracle import kvq_oracle as orc

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _setup():
    import kvq_setup
    return kvq_setup


def _want_q4(rows):
    """Oracle packed bytes and scale bits of fp16 rows [n][256]."""
    codes, scales = orc.quantize_q4_0(orc.rotate_f32(rows))
    return orc.pack_q4(codes), scales.view(np.uint16)


def _check(lay, cache, w, b, positions, k_rows, v_rows):
    ks = _setup()
    for s, rows, dt in (("k", k_rows, w.k_dtype), ("v", v_rows, w.v_dtype)):
        for h in range(w.n_kv_heads):
            if dt == "q4":
                got = ks.q4_rows_of(lay, cache[s], b, positions, h)
                gs = ks.scales_of(lay, cache[s + "_scales"], b, positions, h, n=w.head_dim // 32)
                want, want_s = _want_q4(rows[:, h])
                np.testing.assert_array_equal(got, want, err_msg=f"{w.name} {s} bytes h={h}")
                np.testing.assert_array_equal(gs.view(np.uint16), want_s, err_msg=f"{w.name} {s} scales h={h}")
            else:
                got = ks.rows_of(lay, cache[s], b, positions, h)
                want_c, want_s = orc.quantize_rows(rows[:, h], w.scale_group)
                np.testing.assert_array_equal(got, want_c, err_msg=f"{w.name} {s} codes h={h}")
                gs = ks.scales_of(lay, cache[s + "_scales"], b, positions, h)
                np.testing.assert_array_equal(gs.view(np.uint16), want_s.view(np.uint16))


@pytest.mark.parametrize("name", ["long_q4", "long_k8v4"])
@pytest.mark.parametrize("order", ["pos", "head"])
def test_q4_append_bit_exact(name, order):
    """3000 positions of the long-context rows (K with outlier channels),
    appended in ragged blocks, every position compared."""
    ks = _setup()
    w = wl.WORKLOADS[name].with_(max_ctx=4096)
    L = 3000
    print(f"[q4 append] {name} {order} L={L}", flush=True)
    lay = ks.layout_for(w, order)
    cache = kvq_alloc(lay, w)
    p = 0
    for n in (1, 7, 992, 1000, 1000):
        ks.append_rows(lay, cache, 0, p, wl.kv_rows(w, "k", 0, p, n), wl.kv_rows(w, "v", 0, p, n))
        p += n
    assert p == L
    pos = np.arange(L)
    _check(lay, cache, w, 0, pos, wl.kv_rows(w, "k", 0, 0, L), wl.kv_rows(w, "v", 0, 0, L))
    tail = ks.q4_rows_of(lay, cache["v"], 0, np.arange(L, w.max_ctx), 1)
    assert (tail == 0x5A).all()


def kvq_alloc(lay, w, fill=0x5A):
    import int8_quantized_kv_quant_amd as kvq
    return kvq.alloc_cache(lay, w.batch, fill=fill)


def _edge_rows():
    """fp16 rows [n][1][256] whose rotations hit the quantizer's edge cases."""
    H = orc.hadamard(256)
    rows = []
    # exact ties after the rotation: y = 8 e_i - 8 e_j (first of the pair wins)
    for i, j in ((0, 1), (1, 0), (5, 37), (31, 30), (200, 255)):
        y = np.zeros(256)
        y[i], y[j] = 8.0, -8.0
        rows.append(H @ y / 16.0)
    # a rotated row with equal magnitudes everywhere (x = 4 e_k)
    for k in (0, 77):
        x = np.zeros(256)
        x[k] = 4.0
        rows.append(x)
    rows.append(np.zeros(256))                           # all blocks zero: scale 0, codes 8
    big = np.full(256, 30000.0)
    big[::3] = -30000.0
    rows.append(big)                                     # large magnitudes (the fp16 scale stays finite)
    rows.append(np.full(256, 2.0 ** -24))                # fp16 subnormals
    half = np.zeros(256)
    half[:128] = wl.uniform_rows(7, (128,), 3.0)
    rows.append(half)                                    # half the input zero
    out = np.stack(rows).astype(np.float16)
    assert np.all(np.isfinite(out))
    return out[:, None, :]


@pytest.mark.parametrize("store", ["k", "v"])
def test_q4_append_edge_rows(store):
    ks = _setup()
    w = wl.WORKLOADS["long_q4"].with_(max_ctx=64, n_kv_heads=1, n_q_heads=8)
    lay = ks.layout_for(w)
    cache = kvq_alloc(lay, w)
    edge = _edge_rows()
    other = wl.uniform_rows(3, edge.shape)
    k_rows, v_rows = (edge, other) if store == "k" else (other, edge)
    print(f"[q4 append] edge rows in {store}", flush=True)
    ks.append_rows(lay, cache, 0, 3, k_rows, v_rows)
    _check(lay, cache, w, 0, np.arange(3, 3 + edge.shape[0]), k_rows, v_rows)
    # the first constructed tie (+8 at value 0, -8 at value 1): code 0 for the
    # first extreme, 15 (clamped) for the second, 8 for the zero value 16
    got = ks.q4_rows_of(lay, cache[store], 0, [3], 0)[0]
    assert got[0] == 0x80 and got[1] & 0x0F == 15
    # rows before and after are untouched
    assert (ks.q4_rows_of(lay, cache["k"], 0, [0, 1, 2, 3 + edge.shape[0]], 0) == 0x5A).all()


def test_q4_append_slot_tail_and_batch():
    """head_dim 256 in a 512-wide slot (the slot tail keeps its canary) over a
    batch of 3 sequences at different start positions."""
    ks = _setup()
    w = wl.WORKLOADS["long_k8v4"].with_(batch=3, max_ctx=300, slot_dim=512)
    lay = ks.layout_for(w, "head")
    cache = kvq_alloc(lay, w)
    import int8_quantized_kv_quant_amd as kvq
    starts = np.array([0, 100, 250], dtype=np.int32)
    n = 40
    k = wl.uniform_rows(11, (3, n, w.n_kv_heads, 256), 2.0)
    v = wl.uniform_rows(12, (3, n, w.n_kv_heads, 256))
    print("[q4 append] batch of 3, slot 512", flush=True)
    kvq.kv_quant_append(lay, cache["k"], cache["v"], cache["k_scales"], cache["v_scales"],
                        torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                        torch.from_numpy(starts).cuda(), 3, n)
    for b in range(3):
        pos = np.arange(starts[b], starts[b] + n)
        _check(lay, cache, w, b, pos, k[b], v[b])
        for h in range(w.n_kv_heads):
            base = (b * lay.s_seq + h * lay.s_head + pos * lay.s_pos) // 2
            idx = torch.as_tensor(base[:, None] + np.arange(128, 256)[None, :]).cuda()
            assert (cache["v"][idx] == 0x5A).all()
