"""4-bit stores on the GPU against the CPU oracle (Strata PR 2698, "Not in this
PR": q4_0 and k8v4 with a Hadamard rotation over head_dim 256).

kv_quant_append into a q4 store: the packed Q4_0 bytes and the fp16 block
scales bit-exact with the oracle's rotation (fp32 butterflies) and quantizer,
including rows built to give exact ties, zero blocks and extreme magnitudes;
nothing written outside the target rows.

Decode (kv_decode_attn_splitk + kv_decode_reduce, and the fused step
kv_append_decode_splitk) over q4_0 and k8v4 caches:
max abs error <= 2e-3 against the fp64 oracle (which rotates the query for a
q4 K store and rotates the output back for a q4 V store) over ragged lengths,
split counts, windows, GQA groups, both layout orders and the full 128K
context."""
import math

import numpy as np
import pytest

import workloads as wl
from oracle import kvq_oracle as orc

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _setup():
    import kvq_setup
    return kvq_setup


def _workload(name):
    """The 4-bit layouts by name; "long_k8v4_rowscale" is long_k8v4 with one int8
    key scale per row (scale group = head_dim) instead of one per 64 values."""
    if name == "long_k8v4_rowscale":
        return wl.WORKLOADS["long_k8v4"].with_(scale_group=256)
    return wl.WORKLOADS[name]


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


@pytest.mark.parametrize("name", ["long_q4", "long_k8v4", "long_k8v4_rowscale"])
@pytest.mark.parametrize("order", ["pos", "head"])
def test_q4_append_bit_exact(name, order):
    """3000 positions of the long-context rows (K with outlier channels),
    appended in ragged blocks, every position compared."""
    ks = _setup()
    w = _workload(name).with_(max_ctx=4096)
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


# ---- decode ---------------------------------------------------------------------------

TOL = 2e-3


def _oracle_seq(w, b, L, q_b, window, sm):
    """fp64 oracle output [n_q][d] of sequence b over positions [0, L)."""
    lo = max(0, L - window) if window else 0
    cache = orc.Cache(1, L, w.n_kv_heads, w.head_dim, w.scale_group, w.k_dtype, w.v_dtype)
    cache.append(wl.kv_rows(w, "k", b, lo, L - lo)[None], wl.kv_rows(w, "v", b, lo, L - lo)[None], [lo])
    return orc.attend(q_b[None], cache, [L], window, sm)[0]


def _run(w, lay, cache, q, lens, window, plan=None):
    import int8_quantized_kv_quant_amd as kvq
    qd = torch.from_numpy(q).cuda()
    ld = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    out = kvq.decode(lay, cache, qd, ld, window, 1.0 / math.sqrt(w.head_dim), plan=plan, n_cu=_setup().n_cu())
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name", ["long_q4", "long_k8v4", "long_k8v4_rowscale"])
@pytest.mark.parametrize("order", ["pos", "head"])
def test_q4_decode_ragged_lengths_and_split_sweep(name, order):
    """Lengths 0, 1, 33, 517, 1100 in one batch (tiles, a ragged tail, an
    empty context); every split size gives the oracle's result."""
    import int8_quantized_kv_quant_amd as kvq
    w = _workload(name).with_(batch=5, max_ctx=1100)
    lens = np.array([0, 1, 33, 517, 1100], dtype=np.int32)
    print(f"[q4 decode] {name} {order} lens {lens.tolist()}", flush=True)
    lay, cache = _setup().fill_cache(w, lens, order=order)
    q = wl.queries(w)
    want = [(_oracle_seq(w, b, int(lens[b]), q[b], 0, 1 / 16) if lens[b] else np.zeros((16, 256)))
            for b in range(w.batch)]
    outs = []
    for chunk in (32, 128, 512, 1120):
        n = -(-1100 // chunk)
        got = _run(w, lay, cache, q, lens, 0, plan=kvq.Plan(n, chunk, w.batch * 16 * n * 258 * 4))
        outs.append(got)
        for b in range(w.batch):
            e = np.abs(got[b] - want[b]).max()
            assert e <= TOL, (chunk, b, e)
        assert not got[0].any()  # empty context -> zero row
    assert np.abs(outs[0] - outs[-1]).max() <= 2 * TOL
    got = _run(w, lay, cache, q, lens, 0)  # the planner's plan
    for b in range(w.batch):
        assert np.abs(got[b] - want[b]).max() <= TOL


@pytest.mark.parametrize("name", ["long_q4", "long_k8v4"])
@pytest.mark.parametrize("window", [1, 300])
def test_q4_decode_sliding_window(name, window):
    w = wl.WORKLOADS[name].with_(batch=2, max_ctx=2000, window=window)
    lens = np.array([2000, 250], dtype=np.int32)
    print(f"[q4 decode] {name} window {window}", flush=True)
    lay, cache = _setup().fill_cache(w, lens)
    q = wl.queries(w)
    got = _run(w, lay, cache, q, lens, window)
    for b in range(2):
        want = _oracle_seq(w, b, int(lens[b]), q[b], window, 1 / 16)
        assert np.abs(got[b] - want).max() <= TOL


@pytest.mark.parametrize("name", ["long_q4", "long_k8v4"])
@pytest.mark.parametrize("n_q,n_kv", [(1, 1), (32, 2), (20, 1)])
def test_q4_decode_gqa_groups(name, n_q, n_kv):
    """GQA groups of 1, 16 and 20 query heads per kv head (20: two head
    blocks of 16 and 4)."""
    w = wl.WORKLOADS[name].with_(max_ctx=700, n_q_heads=n_q, n_kv_heads=n_kv)
    lens = np.array([700], dtype=np.int32)
    print(f"[q4 decode] {name} n_q={n_q} n_kv={n_kv}", flush=True)
    lay, cache = _setup().fill_cache(w, lens)
    q = wl.queries(w)
    got = _run(w, lay, cache, q, lens, 0)
    want = _oracle_seq(w, 0, 700, q[0], 0, 1 / 16)
    assert np.abs(got[0] - want).max() <= TOL


@pytest.mark.parametrize("name", ["long_q4", "long_k8v4"])
def test_q4_decode_long_context_128k(name):
    """The full 131072-position context (K with 1 % outlier channels x20),
    the planner's split plan, every query head against the oracle."""
    w = wl.WORKLOADS[name]
    L = w.contexts[-1]
    print(f"[q4 decode] {name} 131072", flush=True)
    lens = np.array([L], dtype=np.int32)
    lay, cache = _setup().fill_cache(w, lens)
    q = wl.queries(w)
    got = _run(w, lay, cache, q, lens, 0)
    want = _oracle_seq(w, 0, L, q[0], 0, 1 / 16)
    e = np.abs(got[0] - want).max()
    print(f"{name} 128K max abs err {e:.3g}", flush=True)
    assert e <= TOL


# ---- the fused step -------------------------------------------------------------------

def _fused_pair(w, lens, plan=None):
    """Positions [0, L_b - 1) filled, then the step at context L_b unfused
    (kv_quant_append, partials, reduce) and fused (kv_append_decode_splitk):
    (unfused out, fused out, unfused cache, fused cache)."""
    import int8_quantized_kv_quant_amd as kvq
    ks = _setup()
    upto = np.maximum(lens - 1, 0)
    lay, cache0 = ks.fill_cache(w, lens, upto=upto)
    kn = np.stack([wl.kv_rows(w, "k", b, max(int(lens[b]) - 1, 0), 1)[0] for b in range(w.batch)])
    vn = np.stack([wl.kv_rows(w, "v", b, max(int(lens[b]) - 1, 0), 1)[0] for b in range(w.batch)])
    k_new, v_new = torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda()
    q = torch.from_numpy(wl.queries(w)).cuda()
    ld = torch.from_numpy(lens.astype(np.int32)).cuda()
    sm = 1.0 / math.sqrt(w.head_dim)
    ca = {k: (None if t is None else t.clone()) for k, t in cache0.items()}
    start = torch.from_numpy((lens - 1).astype(np.int32)).cuda()
    kvq.kv_quant_append(lay, ca["k"], ca["v"], ca["k_scales"], ca["v_scales"], k_new, v_new, start, w.batch, 1)
    out_a = kvq.decode(lay, ca, q, ld, w.window, sm, plan=plan, n_cu=ks.n_cu())
    cb = {k: (None if t is None else t.clone()) for k, t in cache0.items()}
    out_b = kvq.decode(lay, cb, q, ld, w.window, sm, plan=plan, n_cu=ks.n_cu(), new_kv=(k_new, v_new))
    torch.cuda.synchronize()
    for name in ("k", "v", "k_scales", "v_scales"):
        x, y = ca[name], cb[name]
        if x.dtype == torch.float16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), f"{name} differs between the fused and the unfused step"
    return out_a.cpu().numpy().astype(np.float64), out_b.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name", ["long_q4", "long_k8v4", "long_k8v4_rowscale"])
@pytest.mark.parametrize("window", [0, 700])
def test_q4_fused_step_equals_append_then_decode(name, window):
    """The fused step leaves the cache bit-identical to kv_quant_append's and
    gives the oracle's output, on a batch of 3 with ragged contexts."""
    w = _workload(name).with_(batch=3, max_ctx=5000, window=window)
    lens = np.array([5000, 2, 1337], dtype=np.int64)
    print(f"[q4 fused] {name} window {window}", flush=True)
    out_a, out_b = _fused_pair(w, lens)
    q = wl.queries(w)
    for b in range(w.batch):
        want = _oracle_seq(w, b, int(lens[b]), q[b], window, 1 / 16)
        assert np.abs(out_b[b] - want).max() <= TOL, b
        assert np.abs(out_b[b] - out_a[b]).max() <= TOL, b


@pytest.mark.parametrize("name", ["long_q4", "long_k8v4"])
def test_q4_fused_new_row_alone_and_on_a_split_boundary(name):
    """L = 1 (the new row is the whole context), L - 1 on a split start (that
    split holds only the new row), L = 0 (nothing appended, zero output)."""
    import int8_quantized_kv_quant_amd as kvq
    w = wl.WORKLOADS[name].with_(batch=4, max_ctx=1024)
    lens = np.array([1, 257, 0, 513], dtype=np.int64)
    plan = kvq.Plan(4, 256, 4 * 16 * 4 * 258 * 4)  # splits start at 0, 256, 512, 768
    print(f"[q4 fused] {name} edges", flush=True)
    out_a, out_b = _fused_pair(w, lens, plan=plan)
    q = wl.queries(w)
    for b in (0, 1, 3):
        want = _oracle_seq(w, b, int(lens[b]), q[b], 0, 1 / 16)
        assert np.abs(out_b[b] - want).max() <= TOL, b
    assert not out_b[2].any()


# ---- short, peaked contexts at 16 query heads per kv head -------------------------------
# The chunk case q4_batch_g16 (two sequences of the long-context 4-bit layouts
# with x20 outlier K channels, 32 query / 2 kv heads, chunks of 33 tokens at
# positions 100 and 600) run token by token as decode queries: token t of
# sequence b is the query of a context of start_b + t + 1 positions, so the
# contexts are 101..133 and 601..633. Few keys and peaked softmax rows are
# where the rounding of scores is least averaged out.

_G16_STARTS = (100, 600)
_G16_TOKENS = 33


def _g16_workload(name):
    return wl.WORKLOADS[name].with_(batch=2, n_q_heads=32, max_ctx=1024)


def _g16_oracle(w, qs):
    """fp64 oracle outputs [t][b][32][256] at contexts start_b + t + 1."""
    out = np.zeros((_G16_TOKENS, 2, 32, 256))
    for b, s in enumerate(_G16_STARTS):
        for t in range(_G16_TOKENS):
            out[t, b] = _oracle_seq(w, b, s + t + 1, qs[b, t], 0, 1 / 16)
    return out


@pytest.mark.parametrize("name", ["long_q4", "long_k8v4"])
def test_q4_decode_short_peaked_contexts_g16(name):
    """kv_decode_attn_splitk + kv_decode_reduce at every context 101..133 and
    601..633, with the planner's plan and with 32-position splits, element by
    element within 2e-3 of the oracle."""
    import int8_quantized_kv_quant_amd as kvq
    w = _g16_workload(name)
    ends = np.array([s + _G16_TOKENS for s in _G16_STARTS])
    print(f"[q4 decode g16] {name} contexts 101..133, 601..633", flush=True)
    lay, cache = _setup().fill_cache(w, ends)
    qs = wl.chunk_queries(w, _G16_TOKENS)
    want = _g16_oracle(w, qs)
    worst = 0.0
    for plan in (None, kvq.Plan(20, 32, 2 * 32 * 20 * 258 * 4)):
        for t in range(_G16_TOKENS):
            lens = [s + t + 1 for s in _G16_STARTS]
            got = _run(w, lay, cache, np.ascontiguousarray(qs[:, t]), lens, 0, plan=plan)
            e = float(np.abs(got - want[t]).max())
            worst = max(worst, e)
            assert e <= TOL, (name, "planner" if plan is None else "32-position splits", lens, e)
    print(f"[q4 decode g16] {name} max abs err {worst:.3g}", flush=True)


@pytest.mark.parametrize("name", ["long_q4", "long_k8v4"])
def test_q4_fused_short_peaked_contexts_g16(name):
    """The fused step (kv_append_decode_splitk) token after token: each step
    appends the row at start_b + t and attends at context start_b + t + 1;
    every output within 2e-3 of the oracle, and the rows it appended equal the
    oracle's quantization."""
    import int8_quantized_kv_quant_amd as kvq
    ks = _setup()
    w = _g16_workload(name)
    print(f"[q4 fused g16] {name} contexts 101..133, 601..633", flush=True)
    lay, cache = ks.fill_cache(w, np.array(_G16_STARTS))
    qs = wl.chunk_queries(w, _G16_TOKENS)
    want = _g16_oracle(w, qs)
    worst = 0.0
    for t in range(_G16_TOKENS):
        lens = np.array([s + t + 1 for s in _G16_STARTS], dtype=np.int32)
        kn = np.stack([wl.kv_rows(w, "k", b, s + t, 1)[0] for b, s in enumerate(_G16_STARTS)])
        vn = np.stack([wl.kv_rows(w, "v", b, s + t, 1)[0] for b, s in enumerate(_G16_STARTS)])
        out = kvq.decode(lay, cache, torch.from_numpy(np.ascontiguousarray(qs[:, t])).cuda(),
                         torch.from_numpy(lens).cuda(), 0, 1 / 16, n_cu=ks.n_cu(),
                         new_kv=(torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda()))
        torch.cuda.synchronize()
        e = float(np.abs(out.cpu().numpy().astype(np.float64) - want[t]).max())
        worst = max(worst, e)
        assert e <= TOL, (name, lens.tolist(), e)
    print(f"[q4 fused g16] {name} max abs err {worst:.3g}", flush=True)
    for b, s in enumerate(_G16_STARTS):
        pos = np.arange(s, s + _G16_TOKENS)
        _check(lay, cache, w, b, pos, wl.kv_rows(w, "k", b, s, _G16_TOKENS), wl.kv_rows(w, "v", b, s, _G16_TOKENS))
