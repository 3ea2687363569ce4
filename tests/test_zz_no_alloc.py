"""kv_decode_attn_static, the decode entry point that allocates nothing (for
callers that cannot allocate: graph capture, serving loops), against the
existing pair kv_decode_attn_splitk + kv_decode_reduce with a caller
workspace: bit-identical outputs on consecutive calls that shrink (the static
scratch keeps the previous call's partials), and the oracle's output within
2e-3 on the first."""
import math

import numpy as np
import pytest

import workloads as wl
from oracle import kvq_oracle as orc

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-3


def _pair_and_static(w, lens, label):
    import int8_quantized_kv_quant_amd as kvq
    import kvq_setup as ks
    lens = np.asarray(lens, dtype=np.int32)
    lay, cache = ks.fill_cache(w, lens)
    q = torch.from_numpy(wl.queries(w)).cuda()
    ld = torch.from_numpy(lens).cuda()
    sm = 1.0 / math.sqrt(w.head_dim)
    plan = kvq.kvq_plan(lay, w.batch, w.n_q_heads, int(lens.max()), w.window, ks.n_cu())
    assert plan.ws_bytes <= kvq.STATIC_SCRATCH_BYTES
    print(f"[static] {label}: lens {lens.tolist()} plan {plan.n_splits} x {plan.chunk}", flush=True)
    ref = kvq.decode(lay, cache, q, ld, w.window, sm, plan=plan)
    got = torch.full_like(ref, float("nan"))
    kvq.kv_decode_attn_static(lay, cache["k"], cache["v"], cache["k_scales"], cache["v_scales"], q, w.batch,
                              w.n_q_heads, ld, w.window, sm, plan, got)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"{label}: differs from the workspace pair"
    return got.cpu().numpy().astype(np.float64)


def _oracle(w, b, L, q_b):
    lo = max(0, L - w.window) if w.window else 0
    c = orc.Cache(1, L, w.n_kv_heads, w.head_dim, w.scale_group, w.k_dtype, w.v_dtype)
    c.append(wl.kv_rows(w, "k", b, lo, L - lo)[None], wl.kv_rows(w, "v", b, lo, L - lo)[None], [lo])
    return orc.attend(q_b[None], c, [L], w.window, 1.0 / math.sqrt(w.head_dim))[0]


def test_static_scratch_matches_the_workspace_pair_on_shrinking_calls():
    # 1: long-context layout (16 query / 2 kv heads, head_dim 256, group-64
    #    scales), two sequences, the planner's plan
    w1 = wl.WORKLOADS["long"].with_(batch=2, max_ctx=20000)
    got = _pair_and_static(w1, [20000, 7777], "long")
    q1 = wl.queries(w1)
    e = max(float(np.abs(got[b] - _oracle(w1, b, L, q1[b])).max()) for b, L in enumerate((20000, 7777)))
    print(f"[static] long: max abs err {e:.3g} against the oracle", flush=True)
    assert e <= TOL
    # 2: smaller, the 4-bit layout (q4_0) with a sliding window
    _pair_and_static(wl.WORKLOADS["long_q4"].with_(max_ctx=3000, window=700), [3000], "q4_0 window 700")
    # 3: smaller still, the tiny workload (8 query / 2 kv heads, head_dim 64, context 256)
    w3 = wl.WORKLOADS["tiny"]
    got = _pair_and_static(w3, [256], "tiny")
    e = float(np.abs(got[0] - _oracle(w3, 0, 256, wl.queries(w3)[0])).max())
    assert e <= TOL
