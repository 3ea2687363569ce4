"""The C-ABI library on the host: it loads, exports every function that
include/kvq.h declares, its planner keeps its stated properties, and every
argument error is returned before any device call (no GPU needed)."""
import ctypes
import math
import os
import re

import pytest

import int8_quantized_kv_quant_amd as kvq
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

needs_lib = pytest.mark.skipif(not os.path.exists(kvq.lib_path()), reason="libkvq.so not built")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^(?:const\s+)?(?:int|char\s*\*|const char\s*\*|void)\s*\*?\s*(\w+)\s*\(", src, re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared_functions()
    assert set(names) == set(kvq.EXPORTED_SYMBOLS), names


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(kvq.lib_path())
    for name in _declared_functions():
        assert hasattr(lib, name), name


@needs_lib
def test_status_strings_and_version():
    assert kvq.kvq_status_string(0) == "ok"
    for st in range(-8, 0):
        assert kvq.kvq_status_string(st) != "unknown status"
    assert kvq.kvq_status_string(-99) == "unknown status"
    assert kvq.kvq_version() > 0


def _layout(w: wl.Workload, order="pos"):
    return kvq.make_layout(w.n_kv_heads, w.head_dim, w.max_ctx, w.batch, slot_dim=w.slot_dim,
                           k_dtype=w.k_dtype, v_dtype=w.v_dtype, scale_group=w.scale_group, order=order)


@needs_lib
@pytest.mark.parametrize("name", sorted(wl.WORKLOADS))
@pytest.mark.parametrize("n_cu", [8, 256])
def test_plan_covers_the_context(name, n_cu):
    w = wl.WORKLOADS[name]
    lay = _layout(w)
    for L in (1, 63, 64, 100, w.max_ctx):
        p = kvq.kvq_plan(lay, w.batch, w.n_q_heads, L, w.window, n_cu)
        l_eff = min(L, w.window) if w.window else L
        assert p.chunk % 32 == 0 and p.chunk >= 32
        assert 1 <= p.n_splits <= 8192
        assert p.n_splits * p.chunk >= l_eff
        assert (p.n_splits - 1) * p.chunk < max(l_eff, 1)      # no split starts past the range
        assert p.ws_bytes == w.batch * w.n_q_heads * p.n_splits * (w.head_dim + 2) * 4
        if l_eff >= 128:
            assert p.chunk >= 128  # at least one 32-position tile per wavefront of a split
        if l_eff < 64:
            assert p.n_splits == 1  # genie v1.3.0: single block below 64 positions


@needs_lib
def test_plan_long_context_fills_the_chip():
    w = wl.WORKLOADS["long"]
    p = kvq.kvq_plan(_layout(w), 1, 16, 131072, 0, 256)
    assert (p.n_splits, p.chunk) == (128, 1024)  # 2 kv heads x 128 splits = one workgroup per CU


@needs_lib
def test_plan_ragged_batch_keeps_partials_small():
    w = wl.WORKLOADS["batched"]
    p = kvq.kvq_plan(_layout(w), 64, 32, 32768, 0, 256)
    kv_pos = 2 * (128 + 4)
    part = 4 * (128 + 2) * 4
    assert part / (p.chunk * kv_pos) <= 0.011


# ---------------------------------------------------------------- validation
FAKE = 0x10000  # never dereferenced: every call below fails validation first


def _base():
    return kvq.make_layout(2, 256, 1024, 1, scale_group=64)


def _append(lay, **kw):
    args = dict(k_store=FAKE, v_store=FAKE, k_scales=FAKE, v_scales=FAKE, k_new=FAKE, v_new=FAKE,
                start_pos=FAKE, batch=1, n_tok=1)
    args.update(kw)
    return kvq.load().kv_quant_append(ctypes.byref(lay.c()), args["k_store"], args["v_store"],
                                      args["k_scales"], args["v_scales"], args["k_new"], args["v_new"],
                                      args["start_pos"], args["batch"], args["n_tok"], None)


def _partial(lay, plan=None, **kw):
    plan = plan or kvq.Plan(4, 256, 1 * 16 * 4 * 258 * 4)
    args = dict(k_store=FAKE, v_store=FAKE, k_scales=FAKE, v_scales=FAKE, q=FAKE, batch=1, n_q=16,
                seq_lens=FAKE, window=0, sm=0.0625, ws=FAKE, ws_bytes=plan.ws_bytes)
    args.update(kw)
    return kvq.load().kv_decode_attn_splitk(
        ctypes.byref(lay.c()), args["k_store"], args["v_store"], args["k_scales"], args["v_scales"],
        args["q"], args["batch"], args["n_q"], args["seq_lens"], args["window"], args["sm"],
        ctypes.byref(plan.c()), args["ws"], args["ws_bytes"], None)


def _static(lay, plan=None, **kw):
    plan = plan or kvq.Plan(4, 256, 1 * 16 * 4 * 258 * 4)
    args = dict(k_store=FAKE, v_store=FAKE, k_scales=FAKE, v_scales=FAKE, q=FAKE, batch=1, n_q=16,
                seq_lens=FAKE, window=0, sm=0.0625, out=FAKE)
    args.update(kw)
    return kvq.load().kv_decode_attn_static(
        ctypes.byref(lay.c()), args["k_store"], args["v_store"], args["k_scales"], args["v_scales"],
        args["q"], args["batch"], args["n_q"], args["seq_lens"], args["window"], args["sm"],
        ctypes.byref(plan.c()), args["out"], None)


def _fused(lay, plan=None, **kw):
    plan = plan or kvq.Plan(4, 256, 1 * 16 * 4 * 258 * 4)
    args = dict(k_store=FAKE, v_store=FAKE, k_scales=FAKE, v_scales=FAKE, k_new=FAKE, v_new=FAKE, q=FAKE,
                batch=1, n_q=16, seq_lens=FAKE, window=0, sm=0.0625, ws=FAKE, ws_bytes=plan.ws_bytes)
    args.update(kw)
    return kvq.load().kv_append_decode_splitk(
        ctypes.byref(lay.c()), args["k_store"], args["v_store"], args["k_scales"], args["v_scales"],
        args["k_new"], args["v_new"], args["q"], args["batch"], args["n_q"], args["seq_lens"], args["window"],
        args["sm"], ctypes.byref(plan.c()), args["ws"], args["ws_bytes"], None)


def _one(lay, plan=None, **kw):
    plan = plan or kvq.Plan(4, 256, 1 * 16 * 4 * 258 * 4)
    args = dict(k_store=FAKE, v_store=FAKE, k_scales=FAKE, v_scales=FAKE, k_new=FAKE, v_new=FAKE, q=FAKE,
                batch=1, n_q=16, seq_lens=FAKE, window=0, sm=0.0625, ws=FAKE, ws_bytes=plan.ws_bytes, arrive=FAKE,
                out=FAKE)
    args.update(kw)
    return kvq.load().kv_decode_attn(
        ctypes.byref(lay.c()), args["k_store"], args["v_store"], args["k_scales"], args["v_scales"],
        args["k_new"], args["v_new"], args["q"], args["batch"], args["n_q"], args["seq_lens"], args["window"],
        args["sm"], ctypes.byref(plan.c()), args["ws"], args["ws_bytes"], args["arrive"], args["out"], None)


def _chunk(lay, plan=None, **kw):
    plan = plan or kvq.Plan(2, 256, 1 * 8 * 16 * 2 * 258 * 4)
    args = dict(k_store=FAKE, v_store=FAKE, k_scales=FAKE, v_scales=FAKE, q=FAKE, batch=1, n_tok=8, n_q=16,
                start=FAKE, window=0, sm=0.0625, ws=FAKE, ws_bytes=plan.ws_bytes, out=FAKE)
    args.update(kw)
    return kvq.load().kv_chunk_attn(
        ctypes.byref(lay.c()), args["k_store"], args["v_store"], args["k_scales"], args["v_scales"], args["q"],
        args["batch"], args["n_tok"], args["n_q"], args["start"], args["window"], args["sm"],
        ctypes.byref(plan.c()), args["ws"], args["ws_bytes"], args["out"], None)


def _reduce(lay, plan=None, **kw):
    plan = plan or kvq.Plan(4, 256, 1 * 16 * 4 * 258 * 4)
    args = dict(ws=FAKE, ws_bytes=plan.ws_bytes, seq_lens=FAKE, batch=1, n_q=16, window=0, out=FAKE)
    args.update(kw)
    return kvq.load().kv_decode_reduce(ctypes.byref(lay.c()), args["ws"], args["ws_bytes"], args["seq_lens"],
                                       args["batch"], args["n_q"], args["window"], ctypes.byref(plan.c()),
                                       args["out"], None)


def _with(lay, **kw):
    d = lay.__dict__.copy()
    d.update(kw)
    return kvq.Layout(**d)


NULL_, SHAPE, UNSUP, ALIGN, WS = -1, -2, -3, -4, -5


@needs_lib
def test_null_scale_pointer_is_refused_not_read_as_one():
    """genie v0.1.0-alpha.11 '--int8-kv triage': a null scale pointer became
    scale 1.0; here it is an error for every int8 store, in every entry point."""
    lay = _base()
    assert _append(lay, k_scales=None) == NULL_
    assert _append(lay, v_scales=None) == NULL_
    assert _partial(lay, k_scales=None) == NULL_
    assert _partial(lay, v_scales=None) == NULL_
    mixed = _with(lay, v_dtype=kvq.KVQ_STORE_FP32)   # k8v32: V has no scales
    assert _partial(mixed, v_scales=None, k_scales=None) == NULL_
    assert _fused(lay, k_scales=None) == NULL_
    assert _fused(lay, v_scales=None) == NULL_


@needs_lib
def test_static_entry_refuses_before_any_device_call():
    """kv_decode_attn_static validates like kv_decode_attn_splitk and refuses
    plans whose partials exceed the static scratch (KVQ_ERR_SCRATCH = -8)."""
    lay = _base()
    assert _static(lay, k_scales=None) == NULL_
    assert _static(lay, q=None) == NULL_
    assert _static(lay, out=None) == NULL_
    assert _static(lay, seq_lens=None) == NULL_
    assert _static(lay, out=FAKE + 2) == ALIGN
    assert _static(lay, n_q=15) == SHAPE
    assert _static(lay, window=-1) == SHAPE
    assert _static(lay, plan=kvq.Plan(2, 100, 0)) == SHAPE
    # 16 heads x 1017 splits x 258 floats x 4 B > 16 MiB; 1016 splits fit
    assert 16 * 1016 * 258 * 4 <= kvq.STATIC_SCRATCH_BYTES < 16 * 1017 * 258 * 4
    assert _static(lay, plan=kvq.Plan(1017, 128, 0)) == -8
    assert _static(lay, plan=kvq.Plan(1016, 128, 0), q=None) == NULL_
    assert _static(lay, batch=0) == 0
    assert kvq.kvq_status_string(-8) != "unknown status"


@needs_lib
def test_fused_append_refuses_what_either_part_refuses():
    lay = _base()
    assert _fused(lay, k_new=None) == NULL_
    assert _fused(lay, v_new=None) == NULL_
    assert _fused(lay, q=None) == NULL_
    assert _fused(lay, k_new=FAKE + 2) == ALIGN
    assert _fused(lay, v_new=FAKE + 8) == ALIGN
    assert _fused(lay, n_q=15) == SHAPE
    assert _fused(lay, window=-1) == SHAPE
    assert _fused(lay, ws=None) == WS
    assert _fused(lay, batch=0, plan=kvq.Plan(4, 256, 0), ws_bytes=0) == 0


@needs_lib
def test_one_call_step_refusals():
    """kv_decode_attn refuses what the partial or the reduce would, plus a
    missing output or arrival array and a half-given new token."""
    lay = _base()
    assert _one(lay, out=None) == NULL_
    assert _one(lay, arrive=None) == NULL_
    assert _one(lay, k_new=None) == NULL_
    assert _one(lay, v_new=None) == NULL_
    assert _one(lay, q=None) == NULL_
    assert _one(lay, out=FAKE + 8) == ALIGN
    assert _one(lay, arrive=FAKE + 2) == ALIGN
    assert _one(lay, k_new=FAKE + 2) == ALIGN
    assert _one(lay, n_q=15) == SHAPE
    assert _one(lay, window=-1) == SHAPE
    assert _one(lay, sm=float("nan")) == SHAPE
    assert _one(lay, ws=None) == WS
    assert _one(lay, ws_bytes=16) == WS
    assert _one(lay, plan=kvq.Plan(0, 256, 0)) == SHAPE
    assert _one(lay, batch=0, plan=kvq.Plan(4, 256, 0), ws_bytes=0) == 0
    assert _one(lay, batch=0, k_new=None, v_new=None, plan=kvq.Plan(4, 256, 0), ws_bytes=0) == 0


@needs_lib
def test_decode_launches():
    """kv_decode_attn: one launch for small int8 units and plans, two otherwise."""
    def n(w, plan=None, batch=None):
        lay = _layout(w)
        plan = plan or kvq.kvq_plan(lay, w.batch, w.n_q_heads, w.max_ctx, w.window, 256)
        return kvq.kvq_decode_launches(lay, w.batch if batch is None else batch, w.n_q_heads, plan)
    assert n(wl.WORKLOADS["tiny"]) == 1                               # 2 splits
    assert n(wl.WORKLOADS["gemma"]) == 1                              # 4 splits (four 2-head units)
    assert n(wl.WORKLOADS["long"]) == 2                               # 128 splits
    assert n(wl.WORKLOADS["mixed_k8v32"].with_(max_ctx=512)) == 2     # fp32 store
    assert n(wl.WORKLOADS["long_q4"].with_(max_ctx=512)) == 2         # 4-bit stores
    t = wl.WORKLOADS["tiny"]
    assert n(t, kvq.Plan(8, 32, 1 * 8 * 8 * 66 * 4)) == 1
    assert n(t, kvq.Plan(9, 32, 1 * 8 * 9 * 66 * 4)) == 2
    assert n(t, batch=0) == 0
    lay = _layout(t)
    with pytest.raises(kvq.KvqError):
        kvq.kvq_decode_launches(lay, 1, 7, kvq.Plan(2, 128, 1 << 20))    # heads not a multiple of kv heads
    with pytest.raises(kvq.KvqError):
        kvq.kvq_decode_launches(lay, 1, 8, kvq.Plan(2, 128, 16))         # plan workspace too small


def test_arrive_count():
    lay = kvq.make_layout(2, 128, 1024, 3)
    assert kvq.arrive_count(lay, 3, 8) == 3 * 8
    assert kvq.arrive_count(lay, 3, 40) == 3 * 40
    assert kvq.arrive_count(lay, 0, 8) == 1


@needs_lib
def test_chunk_attention_refusals():
    lay = _base()
    # an fp32 store: verify windows of at most 16 (token, head) rows per kv
    # head only (the decode kernel's chunk rows; 8 heads per kv head here)
    assert _chunk(_with(lay, v_dtype=kvq.KVQ_STORE_FP32)) == UNSUP
    assert _chunk(_with(lay, k_dtype=kvq.KVQ_STORE_FP32), n_tok=3) == UNSUP
    assert _chunk(_with(lay, v_dtype=kvq.KVQ_STORE_FP32), n_tok=2, batch=0) == 0
    assert _chunk(_with(lay, k_dtype=kvq.KVQ_STORE_FP32, v_dtype=kvq.KVQ_STORE_FP32), n_tok=1, batch=0) == 0
    assert _chunk(lay, k_scales=None) == NULL_
    assert _chunk(lay, q=None) == NULL_
    assert _chunk(lay, start=None) == NULL_
    assert _chunk(lay, out=None) == NULL_
    assert _chunk(lay, q=FAKE + 8) == ALIGN
    assert _chunk(lay, out=FAKE + 2) == ALIGN
    assert _chunk(lay, n_q=15) == SHAPE
    assert _chunk(lay, n_tok=-1) == SHAPE
    assert _chunk(lay, window=-1) == SHAPE
    assert _chunk(lay, plan=kvq.Plan(2, 100, 10 ** 9)) == SHAPE
    # split starts past 2^31 key positions (n_splits * chunk) are refused, not wrapped
    assert _chunk(lay, plan=kvq.Plan(4, 1 << 30, 10 ** 12)) == UNSUP
    assert _chunk(lay, plan=kvq.Plan(2, (1 << 30) + 32, 10 ** 12)) == UNSUP
    assert _chunk(lay, plan=kvq.Plan(2, 256, 1000)) == WS           # smaller than the partials
    assert _chunk(lay, ws_bytes=16) == WS
    assert _chunk(lay, ws=None) == WS
    assert _chunk(lay, batch=0) == 0 and _chunk(lay, n_tok=0) == 0


@needs_lib
@pytest.mark.parametrize("n_tok,start,window", [(2048, 30000, 0), (4, 131068, 0), (1024, 3072, 512), (1, 63, 0)])
def test_chunk_plan_covers_every_key_range(n_tok, start, window):
    w = wl.WORKLOADS["long"]
    lay = _layout(w)
    p = kvq.kvq_plan_chunk(lay, 1, n_tok, 16, start + n_tok, window, 256)
    l_eff = min(start + n_tok, window + n_tok) if window else start + n_tok
    assert p.chunk % 32 == 0 and 1 <= p.n_splits <= 8192
    assert p.n_splits * p.chunk >= l_eff
    assert p.ws_bytes == n_tok * 16 * p.n_splits * (256 + 2) * 4
    rows = n_tok * 8
    if rows >= 64 * 256:     # enough 64-row blocks to fill the chip: one split
        assert p.n_splits == 1
    if n_tok == 4:           # a verify window over 128K keys is split
        assert p.n_splits > 16


@needs_lib
@pytest.mark.parametrize("n_tok,L,window", [(1, 131072, 0), (2, 131072, 0), (1, 3333, 0), (2, 4096, 512),
                                            (4, 131072, 0)])
def test_short_int8_chunk_plan_follows_the_decode_rule(n_tok, L, window):
    """An int8 chunk with at most 32 (token, head) rows per kv head goes
    through the decode partial kernel (one workgroup of 16 or 32 rows per kv
    head and split) and takes the decode planner's split: at one token (the
    decode shape) the very same plan, at two and four the same key chunk (the
    chip-filling rule decides at these lengths)."""
    w = wl.WORKLOADS["long"]
    lay = _layout(w)
    pc = kvq.kvq_plan_chunk(lay, 1, n_tok, 16, L, window, 256)
    pd = kvq.kvq_plan(lay, 1, 16, L, window, 256)
    l_eff = min(L, window + n_tok) if window else L
    assert pc.n_splits * pc.chunk >= l_eff and pc.chunk % 32 == 0
    assert pc.ws_bytes == n_tok * 16 * pc.n_splits * (256 + 2) * 4
    if n_tok == 1 and not window:
        assert (pc.n_splits, pc.chunk) == (pd.n_splits, pd.chunk)
    if L == 131072:
        assert pd.chunk == pc.chunk == 1024


def _blob(lay, unpack=False, **kw):
    hdr = kw.pop("header", None)
    args = dict(k_store=FAKE, v_store=FAKE, k_scales=FAKE, v_scales=FAKE, seq=0, pos0=0, n_pos=8, buf=FAKE,
                buf_bytes=1 << 30)
    args.update(kw)
    lib = kvq.load()
    if not unpack:
        h = kvq.BlobHeader()
        return lib.kv_cache_pack(ctypes.byref(lay.c()), args["k_store"], args["v_store"], args["k_scales"],
                                 args["v_scales"], args["seq"], args["pos0"], args["n_pos"], args["buf"],
                                 args["buf_bytes"], ctypes.byref(h), None)
    return lib.kv_cache_unpack(ctypes.byref(lay.c()), args["k_store"], args["v_store"], args["k_scales"],
                               args["v_scales"], args["seq"], args["pos0"],
                               None if hdr is None else ctypes.byref(hdr), args["buf"], args["buf_bytes"], None)


def _header(lay, n_pos=8, **kw):
    h = kvq.BlobHeader(0x3151564B, 1, lay.n_kv_heads, lay.head_dim, lay.k_dtype, lay.v_dtype, lay.scale_group,
                       n_pos, kvq.kvq_blob_size(lay, n_pos))
    for k, v in kw.items():
        setattr(h, k, v)
    return h


MISMATCH = -7


@needs_lib
def test_blob_size_matches_the_oracle_payload():
    from oracle import kvq_oracle as orc
    for kdt, vdt, g, H in (("int8", "int8", 64, 2), ("int8", "fp32", 256, 2), ("fp32", "int8", 64, 8),
                           ("fp32", "fp32", 256, 1)):
        lay = kvq.make_layout(H, 256, 64, 1, k_dtype=kdt, v_dtype=vdt, scale_group=g)
        c = orc.Cache(1, 64, H, 256, g, kdt, vdt)
        for n in (0, 1, 7, 64):
            assert kvq.kvq_blob_size(lay, n) == len(orc.blob_payload(c, 0, 0, n))


@needs_lib
def test_blob_refusals():
    lay = _base()
    assert _blob(lay, k_scales=None) == NULL_
    assert _blob(lay, buf=None) == NULL_
    assert _blob(lay, buf=FAKE + 8) == ALIGN
    assert _blob(lay, pos0=1020, n_pos=8) == SHAPE          # past max_ctx
    assert _blob(lay, seq=-1) == SHAPE
    assert _blob(lay, buf_bytes=100) == WS
    assert _blob(lay, n_pos=0) == 0
    # unpack: the header must describe this layout
    assert _blob(lay, unpack=True, header=None) == NULL_
    assert _blob(lay, unpack=True, header=_header(lay, magic=0)) == MISMATCH
    assert _blob(lay, unpack=True, header=_header(lay, version=2)) == MISMATCH
    assert _blob(lay, unpack=True, header=_header(lay, k_dtype=kvq.KVQ_STORE_FP32)) == MISMATCH
    assert _blob(lay, unpack=True, header=_header(lay, scale_group=256)) == MISMATCH
    assert _blob(lay, unpack=True, header=_header(lay, head_dim=128)) == MISMATCH
    assert _blob(lay, unpack=True, header=_header(lay, n_kv_heads=4)) == MISMATCH
    assert _blob(lay, unpack=True, header=_header(lay, payload_bytes=123)) == MISMATCH
    # an int8 blob into an fp32 cache (the kv_int8 toggle of the pages)
    f32 = _with(lay, k_dtype=kvq.KVQ_STORE_FP32, v_dtype=kvq.KVQ_STORE_FP32)
    assert _blob(f32, unpack=True, header=_header(lay), k_scales=None, v_scales=None) == MISMATCH
    assert _blob(lay, unpack=True, header=_header(lay), buf_bytes=16) == WS
    assert _blob(lay, unpack=True, header=_header(lay, n_pos=0, payload_bytes=0)) == 0


@needs_lib
def test_shape_errors():
    lay = _base()
    assert _partial(lay, n_q=15) == SHAPE                    # n_q % n_kv != 0
    assert _append(_with(lay, slot_dim=128)) == SHAPE         # slot narrower than head_dim
    assert _append(_with(lay, s_pos=128)) == SHAPE            # rows of one head overlap
    assert _partial(lay, window=-1) == SHAPE
    assert _partial(lay, plan=kvq.Plan(4, 100, 10 ** 9)) == SHAPE   # chunk not a multiple of 32
    assert _partial(lay, plan=kvq.Plan(0, 256, 10 ** 9)) == SHAPE
    assert _partial(lay, plan=kvq.Plan(9000, 256, 10 ** 12)) == SHAPE
    assert _partial(lay, sm=float("nan")) == SHAPE
    assert _append(lay, batch=-1) == SHAPE


@needs_lib
def test_unsupported_requests_are_refused():
    lay = _base()
    # Strata PR 2698: head_dim must be a multiple of 64 for group-64 scales.
    assert _append(_with(lay, head_dim=96, slot_dim=96, s_pos=192, s_head=96, s_seq=192 * 1024)) == UNSUP
    assert _append(_with(lay, head_dim=512, slot_dim=512, s_pos=1024, s_head=512)) == UNSUP
    assert _append(_with(lay, scale_group=32)) == UNSUP
    assert _append(_with(lay, k_dtype=4)) == UNSUP
    big = kvq.make_layout(2, 256, 5_000_000, 1, scale_group=64)   # > 2 GiB per sequence slice
    assert _append(big) == UNSUP


@needs_lib
def test_alignment_errors():
    lay = _base()
    assert _append(lay, k_store=FAKE + 8) == ALIGN
    assert _append(lay, k_new=FAKE + 2) == ALIGN
    assert _partial(lay, q=FAKE + 4) == ALIGN
    assert _partial(lay, k_scales=FAKE + 2) == ALIGN         # group-64 scale rows are 8-byte loads
    assert _append(_with(lay, s_head=264, s_pos=528)) == ALIGN  # row offsets not multiples of 16 B
    assert _reduce(lay, out=FAKE + 2) == ALIGN


@needs_lib
def test_workspace_errors():
    lay = _base()
    plan = kvq.Plan(4, 256, 1 * 16 * 4 * 258 * 4)
    assert _partial(lay, plan=plan, ws=None) == WS
    assert _partial(lay, plan=plan, ws_bytes=plan.ws_bytes - 1) == WS
    assert _partial(lay, plan=kvq.Plan(4, 256, 100)) == WS
    assert _reduce(lay, plan=plan, ws_bytes=16) == WS


@needs_lib
def test_empty_batch_is_a_no_op():
    lay = _base()
    assert _append(lay, batch=0) == 0
    assert _append(lay, n_tok=0) == 0
    assert _partial(lay, batch=0, plan=kvq.Plan(4, 256, 0), ws_bytes=0) == 0
    assert _reduce(lay, batch=0, plan=kvq.Plan(4, 256, 0), ws_bytes=0) == 0


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(kvq, "_lib", None)
    monkeypatch.setattr(kvq, "lib_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(kvq.KvqLibraryMissing):
        kvq.kvq_plan(_base(), 1, 16, 100, 0, 256)


def _q4_layout(k="q4", v="q4", **kw):
    return kvq.make_layout(2, 256, 1024, 1, k_dtype=k, v_dtype=v, scale_group=64, **kw)


@needs_lib
def test_q4_layout_rules():
    """Strata PR 2698 'Not in this PR': the 4-bit stores rotate over head_dim
    256. A q4 element is half a byte, so row offsets in elements are multiples
    of 32; a q4 row has 8 fp16 scales (one per 32-value block), so the shared
    scale strides leave room for 8."""
    for k, v in (("q4", "q4"), ("int8", "q4"), ("q4", "int8"), ("fp32", "q4")):
        lay = _q4_layout(k, v)
        assert lay.ss_pos >= 8 * 2 and lay.ss_head == 8
        assert _append(lay, batch=0) == 0                     # a valid layout (nothing launched)
    q4 = _q4_layout()
    assert _append(_with(q4, head_dim=128, slot_dim=128, s_head=128, s_pos=256)) == UNSUP
    assert _append(_with(q4, slot_dim=272, s_head=272, s_pos=544, s_seq=544 * 1024), batch=0) == ALIGN
    assert _append(_with(q4, ss_pos=4, ss_head=2, ss_seq=4096), batch=0) == SHAPE   # no room for 8 scales
    assert _append(_with(q4, ss_head=4), batch=0) == ALIGN    # 8-scale rows are 16-byte aligned
    assert _append(q4, v_scales=None) == NULL_                 # a q4 store has scales too
    assert _append(q4, k_scales=FAKE + 8) == ALIGN
    k8v4 = _q4_layout("int8", "q4")
    assert _append(_with(k8v4, ss_pos=8, ss_head=4, ss_seq=8192), batch=0) == ALIGN


@needs_lib
def test_q4_entry_point_refusals():
    """Decode, the fused step and chunk attention take q4_0 and k8v4; every
    other combination with a q4 store is refused before any device call.
    The blob takes every combination (its size matches the oracle's payload)
    and refuses a blob of other store types."""
    assert _partial(_q4_layout("q4", "int8")) == UNSUP
    assert _partial(_q4_layout("q4", "fp32")) == UNSUP
    assert _partial(_q4_layout("fp32", "q4")) == UNSUP
    assert _partial(_q4_layout(), batch=0, plan=kvq.Plan(4, 256, 0), ws_bytes=0) == 0
    assert _partial(_q4_layout("int8", "q4"), batch=0, plan=kvq.Plan(4, 256, 0), ws_bytes=0) == 0
    assert _partial(_q4_layout(), k_scales=None) == NULL_
    assert _fused(_q4_layout("q4", "int8")) == UNSUP
    assert _fused(_q4_layout("fp32", "q4")) == UNSUP
    assert _fused(_q4_layout(), batch=0, plan=kvq.Plan(4, 256, 0), ws_bytes=0) == 0
    assert _fused(_q4_layout("int8", "q4"), k_new=None) == NULL_
    assert _chunk(_q4_layout("q4", "int8")) == UNSUP
    assert _chunk(_q4_layout("fp32", "q4")) == UNSUP
    assert _chunk(_q4_layout(), batch=0) == 0
    from oracle import kvq_oracle as orc
    for k, v in (("q4", "q4"), ("int8", "q4"), ("q4", "int8"), ("q4", "fp32")):
        lay = _q4_layout(k, v)
        c = orc.Cache(1, 40, 2, 256, 64, k, v)
        for n in (0, 1, 7, 32):
            assert kvq.kvq_blob_size(lay, n) == len(orc.blob_payload(c, 0, 0, n)), (k, v, n)
        assert _blob(lay, n_pos=0) == 0                        # a valid call (nothing launched)
    q4 = _q4_layout()
    assert _blob(q4, unpack=True, header=_header(_q4_layout("int8", "q4"))) == MISMATCH
    assert _blob(_base(), unpack=True, header=_header(q4)) == MISMATCH
    assert _blob(q4, v_scales=None) == NULL_


@needs_lib
def test_stream_reference_refusals():
    lib = kvq.load()
    assert lib.kvq_stream_read(None, 1024, FAKE, 256, None) == NULL_
    assert lib.kvq_stream_read(FAKE, 1024, None, 256, None) == NULL_
    assert lib.kvq_stream_read(FAKE + 8, 1024, FAKE, 256, None) == ALIGN
    assert lib.kvq_stream_read(FAKE, 1000, FAKE, 256, None) == SHAPE   # not a multiple of 16 bytes
    assert lib.kvq_stream_read(FAKE, 1024, FAKE, 0, None) == SHAPE
    assert lib.kvq_stream_read(FAKE, 0, FAKE, 256, None) == 0           # nothing to read, nothing launched
