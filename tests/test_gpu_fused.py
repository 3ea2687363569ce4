"""The decode step with its quantize-append fused into the partial kernel
(kv_append_decode_splitk) against the unfused pair (kv_quant_append, then
kv_decode_attn_splitk) and the fp64 oracle.

genie-ai-runtime v0.1.0-alpha.12, "Path I series" #64/#65: the new token is
converted with its scales captured, and attention reads every position with
its (position, kv head) scale. The fused call must leave the cache exactly as
the append would (codes and scales bit-identical, nothing else written) and
give the same attention output within the decode tolerance.
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
    lo = max(0, L - window) if window else 0
    cache = orc.Cache(1, L, w.n_kv_heads, w.head_dim, w.scale_group, w.k_dtype, w.v_dtype)
    cache.append(wl.kv_rows(w, "k", b, lo, L - lo)[None], wl.kv_rows(w, "v", b, lo, L - lo)[None], [lo])
    return orc.attend(q_b[None], cache, [L], window, sm)[0]


def _clone(cache):
    return {k: (None if t is None else t.clone()) for k, t in cache.items()}


def _step_pair(w, lens, plan=None):
    """Fill positions [0, L_b - 1) of every sequence, then run the decode step
    at context L_b twice: unfused (append + partials + reduce) and fused.
    Returns (unfused out, fused out, unfused cache, fused cache)."""
    import int8_quantized_kv_quant_amd as kvq
    import kvq_setup as ks
    upto = np.maximum(lens - 1, 0)
    lay, cache0 = ks.fill_cache(w, lens, upto=upto)
    kn = np.stack([wl.kv_rows(w, "k", b, max(int(lens[b]) - 1, 0), 1)[0] for b in range(w.batch)])
    vn = np.stack([wl.kv_rows(w, "v", b, max(int(lens[b]) - 1, 0), 1)[0] for b in range(w.batch)])
    k_new = torch.from_numpy(kn).cuda()
    v_new = torch.from_numpy(vn).cuda()
    q = torch.from_numpy(wl.queries(w)).cuda()
    ld = torch.from_numpy(lens.astype(np.int32)).cuda()
    sm = 1.0 / math.sqrt(w.head_dim)
    n_cu = ks.n_cu()

    ca = _clone(cache0)
    start = torch.from_numpy((lens - 1).astype(np.int32)).cuda()
    kvq.kv_quant_append(lay, ca["k"], ca["v"], ca["k_scales"], ca["v_scales"], k_new, v_new, start, w.batch, 1)
    out_a = kvq.decode(lay, ca, q, ld, w.window, sm, plan=plan, n_cu=n_cu)

    cb = _clone(cache0)
    out_b = kvq.decode(lay, cb, q, ld, w.window, sm, plan=plan, n_cu=n_cu, new_kv=(k_new, v_new))
    torch.cuda.synchronize()
    return (out_a.cpu().numpy().astype(np.float64), out_b.cpu().numpy().astype(np.float64), ca, cb)


def _same_cache(ca, cb):
    for name in ("k", "v", "k_scales", "v_scales"):
        if ca[name] is None:
            assert cb[name] is None
            continue
        a, b = ca[name], cb[name]
        if a.dtype == torch.float16:   # compare scales as bit patterns
            a, b = a.view(torch.int16), b.view(torch.int16)
        elif a.dtype == torch.float32:
            a, b = a.view(torch.int32), b.view(torch.int32)
        assert torch.equal(a, b), f"{name} differs between the fused and the unfused step"


CASES = {
    "tiny": (wl.WORKLOADS["tiny"], [256]),
    "gemma_window": (wl.WORKLOADS["gemma"].with_(max_ctx=2048), [1500]),
    "long_like": (wl.WORKLOADS["long"].with_(max_ctx=8192), [5000]),
    "batched_ragged": (wl.WORKLOADS["batched"].with_(batch=4, max_ctx=4096), [4096, 1, 1027, 2500]),
    "k8v32": (wl.WORKLOADS["mixed_k8v32"].with_(max_ctx=4096), [3001]),
    "k32v8": (wl.WORKLOADS["mixed_k32v8"].with_(max_ctx=4096), [2048]),
    "k32v32": (wl.WORKLOADS["tiny"].with_(k_dtype="fp32", v_dtype="fp32"), [200]),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_fused_step_equals_append_then_decode(case):
    w, lens = CASES[case]
    lens = np.array(lens, dtype=np.int64)
    out_a, out_b, ca, cb = _step_pair(w, lens)
    _same_cache(ca, cb)
    q = wl.queries(w)
    sm = 1.0 / math.sqrt(w.head_dim)
    for b in range(w.batch):
        want = _oracle(w, b, int(lens[b]), q[b], w.window, sm)
        assert np.abs(out_b[b] - want).max() <= TOL, (case, b)
        assert np.abs(out_b[b] - out_a[b]).max() <= TOL, (case, b)


def test_new_row_alone_and_on_a_split_boundary():
    """L = 1: the new row is the only position (output = its value row).
    L - 1 on a split start: that split's tiles are empty and the new row is all
    it holds. L = 0: nothing is appended and the output is zero."""
    import int8_quantized_kv_quant_amd as kvq
    w = wl.Workload("edge", 4, 8, 2, 128, 128, 64, 1024, 0, 160, contexts=(1024,))
    lens = np.array([1, 257, 0, 513], dtype=np.int64)
    plan = kvq.Plan(4, 256, 4 * 8 * 4 * 130 * 4)   # splits start at 0, 256, 512, 768
    out_a, out_b, ca, cb = _step_pair(w, lens, plan=plan)
    _same_cache(ca, cb)
    q = wl.queries(w)
    sm = 1.0 / math.sqrt(w.head_dim)
    for b in (0, 1, 3):
        want = _oracle(w, b, int(lens[b]), q[b], 0, sm)
        assert np.abs(out_b[b] - want).max() <= TOL, b
    assert not out_b[2].any()


@pytest.mark.parametrize("name", ["long", "long_q4", "long_k8v4"])
def test_fused_step_in_a_graph_matches_eager(name):
    """Captured once, replayed at growing contexts with the token rows and the
    lengths changed on the device between replays: every replay is within
    2e-3 of the oracle at its context, equals the same fused step run eagerly
    bit for bit, and leaves the same cache (int8 and the 4-bit layouts)."""
    import int8_quantized_kv_quant_amd as kvq
    import kvq_setup as ks
    w = wl.WORKLOADS[name].with_(max_ctx=4096)
    L0 = 3000
    lay, cache = ks.fill_cache(w, np.array([L0]), upto=np.array([L0 - 1]))
    plan = kvq.kvq_plan(lay, 1, w.n_q_heads, w.max_ctx, 0, ks.n_cu())
    ws = torch.zeros(plan.ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((1, w.n_q_heads, w.head_dim), dtype=torch.float16, device="cuda")
    q = torch.from_numpy(wl.queries(w)).cuda()
    seq_len = torch.tensor([L0], dtype=torch.int32, device="cuda")
    k_new = torch.empty((1, w.n_kv_heads, w.head_dim), dtype=torch.float16, device="cuda")
    v_new = torch.empty_like(k_new)
    sm = 1.0 / math.sqrt(w.head_dim)

    def step(c):
        kvq.kv_append_decode_splitk(lay, c["k"], c["v"], c["k_scales"], c["v_scales"], k_new, v_new, q, 1,
                                    w.n_q_heads, seq_len, 0, sm, plan, ws, ws.numel())
        kvq.kv_decode_reduce(lay, ws, ws.numel(), seq_len, 1, w.n_q_heads, 0, plan, out)

    def load_token(L):
        k_new.copy_(torch.from_numpy(wl.kv_rows(w, "k", 0, L - 1, 1)[0]))
        v_new.copy_(torch.from_numpy(wl.kv_rows(w, "v", 0, L - 1, 1)[0]))
        seq_len.fill_(L)

    eager_cache = _clone(cache)
    load_token(L0)
    step(_clone(cache))  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(cache)
    torch.cuda.synchronize()
    for L in (L0, L0 + 1, L0 + 2, L0 + 3):
        load_token(L)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        want = _oracle(w, 0, L, wl.queries(w)[0], 0, sm)
        e = float(np.abs(got[0].cpu().numpy().astype(np.float64) - want).max())
        assert e <= TOL, f"graph replay at L={L}: max abs err {e:.3g} against the oracle"
        out.zero_()
        step(eager_cache)
        torch.cuda.synchronize()
        assert torch.equal(got, out), f"graph replay differs from the eager fused step at L={L}"
    _same_cache(eager_cache, cache)
