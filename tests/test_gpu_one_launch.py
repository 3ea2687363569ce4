"""kv_decode_attn: the decode step (optional fused append, split-K partials,
combine) in one call, one kernel launch for small int8 plans, against the fp64
oracle and against the two-call path (kv_append_decode_splitk or
kv_decode_attn_splitk, then kv_decode_reduce).

genie-ai-runtime releases, v1.3.0 "split-K decode attention": per-split
online-softmax partials merged into the output; here the last workgroup of a
unit to finish merges them inside the partial kernel. The arrival counters
must be zero before and after every call, the appended cache rows bit-identical
to the append's, and every output within 2e-3 of the oracle.
"""
import math

import numpy as np
import pytest

import workloads as wl
from oracle import kvq_oracle as orc

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-3


def _oracle(w, b, L, q_b, window, sm):
    if L == 0:
        return np.zeros((w.n_q_heads, w.head_dim))
    lo = max(0, L - window) if window else 0
    cache = orc.Cache(1, L, w.n_kv_heads, w.head_dim, w.scale_group, w.k_dtype, w.v_dtype)
    cache.append(wl.kv_rows(w, "k", b, lo, L - lo)[None], wl.kv_rows(w, "v", b, lo, L - lo)[None], [lo])
    return orc.attend(q_b[None], cache, [L], window, sm)[0]


def _clone(cache):
    return {k: (None if t is None else t.clone()) for k, t in cache.items()}


def _same_cache(ca, cb):
    for name in ("k", "v", "k_scales", "v_scales"):
        if ca[name] is None:
            assert cb[name] is None
            continue
        a, b = ca[name], cb[name]
        if a.dtype == torch.float16:
            a, b = a.view(torch.int16), b.view(torch.int16)
        elif a.dtype == torch.float32:
            a, b = a.view(torch.int32), b.view(torch.int32)
        assert torch.equal(a, b), f"{name} differs between kv_decode_attn and the two-call step"


def _run(w, lens, plan=None, append=True):
    """The step at contexts lens through kv_decode_attn and through the two
    calls, from the same cache (positions [0, L_b - 1) filled when the token is
    appended in the step, [0, L_b) otherwise). Returns (one-call out, two-call
    out, one-call cache, two-call cache, plan)."""
    import int8_quantized_kv_quant_amd as kvq
    import kvq_setup as ks
    upto = np.maximum(lens - 1, 0) if append else lens
    lay, cache0 = ks.fill_cache(w, lens, upto=upto)
    q = torch.from_numpy(wl.queries(w)).cuda()
    ld = torch.from_numpy(lens.astype(np.int32)).cuda()
    sm = 1.0 / math.sqrt(w.head_dim)
    if plan is None:
        plan = kvq.kvq_plan(lay, w.batch, w.n_q_heads, w.max_ctx, w.window, ks.n_cu())
    new_kv = None
    if append:
        kn = np.stack([wl.kv_rows(w, "k", b, max(int(lens[b]) - 1, 0), 1)[0] for b in range(w.batch)])
        vn = np.stack([wl.kv_rows(w, "v", b, max(int(lens[b]) - 1, 0), 1)[0] for b in range(w.batch)])
        new_kv = (torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda())
    arrive = torch.zeros(kvq.arrive_count(lay, w.batch, w.n_q_heads), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(plan.ws_bytes, 16), dtype=torch.uint8, device="cuda")
    ca = _clone(cache0)
    out_a = kvq.decode(lay, ca, q, ld, w.window, sm, plan=plan, ws=ws, new_kv=new_kv, arrive=arrive)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(arrive)) == 0, "arrival counters not left at zero"
    cb = _clone(cache0)
    out_b = kvq.decode(lay, cb, q, ld, w.window, sm, plan=plan, new_kv=new_kv)
    torch.cuda.synchronize()
    return (out_a.cpu().numpy().astype(np.float64), out_b.cpu().numpy().astype(np.float64), ca, cb, plan)


def _check(w, lens, out_a, out_b):
    q = wl.queries(w)
    sm = 1.0 / math.sqrt(w.head_dim)
    for b in range(w.batch):
        L = int(lens[b])
        want = _oracle(w, b, L, q[b], w.window, sm)
        assert np.abs(out_a[b] - want).max() <= TOL, (w.name, b, L)
        assert np.abs(out_a[b] - out_b[b]).max() <= TOL, (w.name, b, L)
        if L == 0:
            assert not out_a[b].any()


GEMMA = wl.WORKLOADS["gemma"]   # 8 query heads of head_dim 256 per kv head: four 2-head units

# name: (workload, contexts, launches of kv_decode_attn under the planner's plan)
CASES = {
    "tiny": (wl.WORKLOADS["tiny"], [256], 1),                     # one 4-head unit per kv head
    "gemma_512": (GEMMA.with_(max_ctx=512), [512], 1),
    "gemma_1024": (GEMMA.with_(max_ctx=1024), [1024], 1),
    "gemma_4096": (GEMMA, [4096], 1),
    "gemma_ragged": (GEMMA.with_(batch=3, max_ctx=2048), [1, 700, 2048], 1),
    # 5 query heads per kv head at head_dim 256: units of 2, 2 and 1 heads
    "gqa5_d256": (wl.Workload("gqa5", 2, 10, 2, 256, 256, 64, 1024, 0, 173, contexts=(1024,)), [1000, 77], 1),
    # 20 query heads per kv head at head_dim 64: units of 8, 8 and 4 heads
    "gqa20": (wl.Workload("gqa20", 2, 40, 2, 64, 64, 64, 1024, 0, 171, contexts=(1024,)), [1000, 333], 1),
    # 16 heads per kv head at head_dim 128: four 4-head units
    "gqa16_d128": (wl.Workload("gqa16", 1, 16, 1, 128, 128, 64, 1024, 0, 174, contexts=(1024,)), [1024], 1),
    "ragged_empty": (wl.WORKLOADS["batched"].with_(batch=4, max_ctx=512), [512, 0, 1, 300], 1),
    # two launches through the same call: an fp32 store
    "k8v32": (wl.WORKLOADS["mixed_k8v32"].with_(max_ctx=2048), [1500], 2),
}


def _launches(w, plan):
    import int8_quantized_kv_quant_amd as kvq
    import kvq_setup as ks
    return kvq.kvq_decode_launches(ks.layout_for(w), w.batch, w.n_q_heads, plan)


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("append", [True, False])
def test_one_call_step_against_oracle(case, append):
    w, lens, launches = CASES[case]
    lens = np.array(lens, dtype=np.int64)
    out_a, out_b, ca, cb, plan = _run(w, lens, append=append)
    assert _launches(w, plan) == launches
    _same_cache(ca, cb)
    _check(w, lens, out_a, out_b)


@pytest.mark.parametrize("n_splits,chunk", [(1, 1024), (2, 512), (3, 384), (8, 128), (9, 128), (16, 64)])
def test_forced_split_counts(n_splits, chunk):
    """One launch up to 8 splits (including plans whose last splits are empty
    for the shorter sequences), two launches beyond; every one against the
    oracle."""
    import int8_quantized_kv_quant_amd as kvq
    w = wl.Workload("forced", 3, 16, 2, 256, 256, 64, 1024, 0, 172, contexts=(1024,))
    lens = np.array([1024, 200, 641], dtype=np.int64)
    plan = kvq.Plan(n_splits, chunk, w.batch * w.n_q_heads * n_splits * (w.head_dim + 2) * 4)
    assert _launches(w, plan) == (1 if n_splits <= 8 else 2)
    out_a, out_b, ca, cb, _ = _run(w, lens, plan=plan)
    _same_cache(ca, cb)
    _check(w, lens, out_a, out_b)


def test_q4_layouts_through_the_one_call():
    """4-bit stores run the two launches inside kv_decode_attn."""
    for name in ("long_q4", "long_k8v4"):
        w = wl.WORKLOADS[name].with_(max_ctx=2048)
        lens = np.array([1777], dtype=np.int64)
        out_a, out_b, ca, cb, plan = _run(w, lens)
        assert _launches(w, plan) == 2
        _same_cache(ca, cb)
        _check(w, lens, out_a, out_b)


def test_one_launch_step_in_a_graph():
    """Captured once (one kernel node), replayed at growing contexts with the
    token rows and the length changed on the device between replays: every
    replay within 2e-3 of the oracle, bit-identical to the same call run
    eagerly (the combine reads the splits in a fixed order whichever workgroup
    runs it), the counters back at zero after every replay."""
    import int8_quantized_kv_quant_amd as kvq
    import kvq_setup as ks
    w = GEMMA
    L0 = 3000
    lay, cache = ks.fill_cache(w, np.array([L0 + 8]), upto=np.array([L0 - 1]))
    plan = kvq.kvq_plan(lay, 1, w.n_q_heads, w.max_ctx, w.window, ks.n_cu())
    assert kvq.kvq_decode_launches(lay, 1, w.n_q_heads, plan) == 1
    ws = torch.empty(plan.ws_bytes, dtype=torch.uint8, device="cuda")
    arrive = torch.zeros(kvq.arrive_count(lay, 1, w.n_q_heads), dtype=torch.int32, device="cuda")
    out = torch.empty((1, w.n_q_heads, w.head_dim), dtype=torch.float16, device="cuda")
    q = torch.from_numpy(wl.queries(w)).cuda()
    seq_len = torch.tensor([L0], dtype=torch.int32, device="cuda")
    k_new = torch.empty((1, w.n_kv_heads, w.head_dim), dtype=torch.float16, device="cuda")
    v_new = torch.empty_like(k_new)
    sm = 1.0 / math.sqrt(w.head_dim)

    def step(c, o):
        kvq.kv_decode_attn(lay, c["k"], c["v"], c["k_scales"], c["v_scales"], k_new, v_new, q, 1, w.n_q_heads,
                           seq_len, w.window, sm, plan, ws, ws.numel(), arrive, o,
                           torch.cuda.current_stream().cuda_stream)

    def set_token(L):
        seq_len.fill_(L)
        k_new.copy_(torch.from_numpy(wl.kv_rows(w, "k", 0, L - 1, 1)))
        v_new.copy_(torch.from_numpy(wl.kv_rows(w, "v", 0, L - 1, 1)))

    set_token(L0)
    eager_cache = _clone(cache)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(_clone(cache), out)  # warm-up outside the graph (on a copy)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(cache, out)
    qh = wl.queries(w)
    for L in range(L0, L0 + 6):
        set_token(L)
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        assert int(torch.count_nonzero(arrive)) == 0
        eager = torch.empty_like(out)
        step(eager_cache, eager)
        torch.cuda.synchronize()
        assert torch.equal(eager.view(torch.int16), out.view(torch.int16)), L
        want = _oracle(w, 0, L, qh[0], w.window, sm)
        assert np.abs(got[0] - want).max() <= TOL, L
    _same_cache(cache, eager_cache)
