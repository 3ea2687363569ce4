"""Chunk attention (kv_chunk_attn: several consecutive query tokens per
sequence, causal inside the chunk) on the GPU against the fp64 oracle
(oracle.attend_chunk): max abs error <= 2e-3 (fp32 accumulation, fp16 output)
on prompt chunks and verify windows, windows, every GQA grouping and the
ragged row blocks of a chunk, the chunk kernels and the decode kernels' chunk
rows (int8, 4-bit and fp32 stores).

Strata PR 2698, "What it does": the prompt chunk and the verify windows read
the same int8 cache as decode, dequantized on the fly; the 4-bit layouts of
"Not in this PR" (q4_0, k8v4) are covered the same way.
"""
import math

import numpy as np
import pytest

import workloads as wl
from oracle import kvq_oracle as orc

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-3


def _run(w, starts, n_tok, window, plan=None, tokens=None):
    """Fill positions [0, start_b + n_tok) of every sequence, run the chunk
    attention on the GPU and the oracle on the host (all tokens, or the listed
    (b, t) pairs); returns (gpu [B][T][Hq][d], oracle, plan)."""
    import int8_quantized_kv_quant_amd as kvq
    import kvq_setup as ks
    starts = np.asarray(starts, dtype=np.int64)
    ends = np.minimum(starts + n_tok, w.max_ctx)
    lay, cache = ks.fill_cache(w, ends)
    q = wl.chunk_queries(w, n_tok)
    sm = 1.0 / math.sqrt(w.head_dim)
    if plan is None:
        plan = kvq.kvq_plan_chunk(lay, w.batch, n_tok, w.n_q_heads, int(ends.max()), window, ks.n_cu())
    got = kvq.chunk_attn(lay, cache, torch.from_numpy(q).cuda(),
                         torch.from_numpy(starts.astype(np.int32)).cuda(), window, sm, plan=plan)
    torch.cuda.synchronize()
    got = got.cpu().numpy().astype(np.float64)
    oc = orc.Cache(w.batch, w.max_ctx, w.n_kv_heads, w.head_dim, w.scale_group, w.k_dtype, w.v_dtype)
    for b in range(w.batch):
        lo = max(0, int(starts[b]) + 1 - window) if window else 0
        n = int(ends[b]) - lo
        if n > 0:
            one = np.array([lo])
            rows_k = wl.kv_rows(w, "k", b, lo, n)[None]
            rows_v = wl.kv_rows(w, "v", b, lo, n)[None]
            sub = orc.Cache(1, w.max_ctx, w.n_kv_heads, w.head_dim, w.scale_group, w.k_dtype, w.v_dtype)
            sub.append(rows_k, rows_v, one)
            for s in ("k", "v"):
                oc.data[s][b] = sub.data[s][0]
                if oc.scales[s] is not None:
                    oc.scales[s][b] = sub.scales[s][0]
    want = orc.attend_chunk(q, oc, starts, window, sm, tokens=tokens)
    return got, want, plan


def _check(got, want, tokens=None, label=""):
    pairs = tokens if tokens is not None else [(b, t) for b in range(got.shape[0]) for t in range(got.shape[1])]
    worst = 0.0
    for b, t in pairs:
        worst = max(worst, float(np.abs(got[b, t] - want[b, t]).max()))
    print(f"[chunk] {label} max abs err {worst:.3g}", flush=True)
    assert worst <= TOL, label


CASES = {
    # name: (workload, starts, n_tok, window)
    "tiny_prompt": (wl.WORKLOADS["tiny"].with_(batch=2, max_ctx=512), [0, 37], 5, 0),
    "gemma_window_chunk": (wl.WORKLOADS["gemma"].with_(max_ctx=1024), [600], 40, 512),
    "long_prompt_ragged_blocks": (wl.WORKLOADS["long"].with_(max_ctx=4096), [3000], 130, 0),
    "batched_three": (wl.WORKLOADS["batched"].with_(batch=3, max_ctx=2304), [100, 2000, 0], 33, 0),
    "verify_window_long": (wl.WORKLOADS["long"].with_(max_ctx=8192), [6000], 4, 0),
    "mha_g1": (wl.Workload("mha", 1, 4, 4, 128, 128, 64, 1024, 0, 170), [300], 70, 0),
    "g16_d64": (wl.Workload("g16", 1, 32, 2, 64, 64, 64, 1024, 0, 171), [500], 9, 0),
    "window_smaller_than_chunk": (wl.WORKLOADS["long"].with_(max_ctx=2048), [1000], 100, 64),
    # head_dim <= 128 with >= 1024 rows per kv head: two row blocks per wavefront
    "batched_two_row_blocks": (wl.WORKLOADS["batched"].with_(batch=2, max_ctx=2048), [500, 1400], 300, 0),
    "g16_d64_two_row_blocks": (wl.Workload("g16b", 1, 32, 2, 64, 64, 64, 1024, 0, 172), [600], 80, 100),
    # the 4-bit layouts (Strata PR 2698 "Not in this PR": q4_0, k8v4): rotated
    # query, Q4_0 keys and values, output rotated back
    "q4_prompt_ragged_blocks": (wl.WORKLOADS["long_q4"].with_(max_ctx=4096), [3000], 130, 0),
    "q4_verify_window": (wl.WORKLOADS["long_q4"].with_(max_ctx=8192), [6000], 4, 0),
    "q4_batch_g16": (wl.WORKLOADS["long_q4"].with_(batch=2, n_q_heads=32, max_ctx=1024), [100, 600], 33, 0),
    "k8v4_window_smaller_than_chunk": (wl.WORKLOADS["long_k8v4"].with_(max_ctx=2048), [1000], 100, 64),
    "k8v4_mha_g1": (wl.WORKLOADS["long_k8v4"].with_(n_q_heads=2, max_ctx=1024), [300], 70, 0),
    # k8v4 with one int8 key scale per row (scale group = head_dim)
    "k8v4_row_scales_prompt": (wl.WORKLOADS["long_k8v4"].with_(scale_group=256, max_ctx=2048), [1000], 70, 0),
    # int8 chunks with at most 32 (token, head) rows per kv head run through
    # the decode partial kernel (one or two 16-row blocks per workgroup,
    # per-row causal limits): 16, 12 and 32 rows, a second block of one row,
    # one row per token (G = 1) with a window narrower than the chunk, a first
    # token at position 0, group-64 and row scales (verify_window_long and
    # tiny_prompt above: 32 and 20 rows)
    "rows_verify_long_t2": (wl.WORKLOADS["long"].with_(max_ctx=8192), [6000], 2, 0),
    "rows_gemma_window_t2": (wl.WORKLOADS["gemma"].with_(max_ctx=1024), [700], 2, 512),
    "rows_gemma_window_t4": (wl.WORKLOADS["gemma"].with_(max_ctx=1024), [900], 4, 512),
    "rows_batched_ragged_t3": (wl.WORKLOADS["batched"].with_(batch=3, max_ctx=2304), [100, 2000, 0], 3, 0),
    "rows_tiny_d64_t4": (wl.WORKLOADS["tiny"].with_(batch=2, max_ctx=512), [0, 37], 4, 0),
    "rows_mha_t16_window5": (wl.Workload("mha16", 1, 4, 4, 128, 128, 128, 1024, 0, 173), [300], 16, 5),
    "rows_mha_d64_t16": (wl.Workload("mha64", 2, 2, 2, 64, 64, 64, 1024, 0, 174), [0, 900], 16, 0),
    "rows_mha_t17_two_blocks": (wl.Workload("mha17", 1, 4, 4, 128, 128, 128, 1024, 0, 175), [300], 17, 0),
    "rows_gemma_t4_batch2": (wl.WORKLOADS["gemma"].with_(batch=2, max_ctx=1024), [0, 1000], 4, 512),
    "rows_batched_t8_d128": (wl.WORKLOADS["batched"].with_(batch=2, max_ctx=2048), [1500, 17], 8, 0),
    # the 4-bit layouts with at most 32 rows per kv head: the 4-bit decode
    # partial kernel in 16-row workgroups (rotated query rows per (token,
    # head), per-row limits; q4_verify_window above: two workgroups)
    "rows_q4_t2": (wl.WORKLOADS["long_q4"].with_(max_ctx=8192), [6000], 2, 0),
    "rows_q4_g16_batch2": (wl.WORKLOADS["long_q4"].with_(batch=2, n_q_heads=32, max_ctx=1024), [0, 600], 1, 0),
    "rows_q4_t2_window": (wl.WORKLOADS["long_q4"].with_(max_ctx=2048), [1500], 2, 300),
    "rows_k8v4_t2_window": (wl.WORKLOADS["long_k8v4"].with_(max_ctx=2048), [1500], 2, 300),
    "rows_k8v4_row_scales_t2": (wl.WORKLOADS["long_k8v4"].with_(scale_group=256, max_ctx=2048), [1500], 2, 0),
    "rows_k8v4_mha_t16": (wl.WORKLOADS["long_k8v4"].with_(n_q_heads=2, max_ctx=1024), [700], 16, 0),
    "rows_q4_mha_t17_two_workgroups": (wl.WORKLOADS["long_q4"].with_(n_q_heads=2, max_ctx=1024), [500], 17, 40),
    # an fp32 store (k8v32, k32v8, k32v32): verify windows of at most 16 rows
    # per kv head through the decode partial kernel's mixed and fp32 paths
    "rows_k8v32_t2": (wl.WORKLOADS["mixed_k8v32"].with_(max_ctx=4096), [3000], 2, 0),
    "rows_k32v8_t2_window": (wl.WORKLOADS["mixed_k32v8"].with_(max_ctx=4096), [3000], 2, 700),
    "rows_k32v32_batch2_d128": (wl.Workload("k32v32", 2, 8, 2, 128, 128, 128, 1024, 0, 178,
                                            k_dtype="fp32", v_dtype="fp32"), [0, 900], 4, 0),
    "rows_k8v32_mha_t16_d64": (wl.Workload("k8v32m", 1, 2, 2, 64, 64, 64, 1024, 0, 179,
                                           k_dtype="int8", v_dtype="fp32"), [500], 16, 30),
    # just past 32 rows: the chunk kernel
    "chunk_mha_t33": (wl.Workload("mha33", 1, 4, 4, 128, 128, 128, 1024, 0, 176), [300], 33, 7),
    "chunk_gemma_t8_batch2": (wl.WORKLOADS["gemma"].with_(batch=2, max_ctx=1024), [0, 1000], 8, 512),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_chunk_matches_oracle(case):
    w, starts, n_tok, window = CASES[case]
    print(f"[chunk] {case}: B={w.batch} T={n_tok} starts={starts} W={window}", flush=True)
    got, want, plan = _run(w, starts, n_tok, window)
    print(f"[chunk] {case}: plan {plan.n_splits} x {plan.chunk}", flush=True)
    _check(got, want, label=case)


@pytest.mark.parametrize("name", ["long", "long_q4", "long_k8v4"])
def test_forced_splits_equal_one_split(name):
    """The same chunk with the keys split 1, 3 and 17 ways: every result within
    the tolerance of the oracle (the combine of kv_decode_reduce per row)."""
    import int8_quantized_kv_quant_amd as kvq
    w = wl.WORKLOADS[name].with_(max_ctx=2048)
    T = 24
    for ns, chunk in ((1, 2048), (3, 704), (17, 128)):
        plan = kvq.Plan(ns, chunk, w.batch * T * w.n_q_heads * ns * (w.head_dim + 2) * 4)
        got, want, _ = _run(w, [1500], T, 0, plan=plan)
        _check(got, want, label=f"splits {ns}")


def test_rows_path_forced_splits():
    """Verify windows of 16 and 24 rows (2 and 3 tokens x 8 heads) through the
    decode partial kernel with the keys split 1, 3 and 17 ways, and a window:
    every result within the tolerance of the oracle."""
    import int8_quantized_kv_quant_amd as kvq
    w = wl.WORKLOADS["long"].with_(max_ctx=4096)
    for T, ns, chunk, window in ((2, 1, 4096, 0), (2, 3, 1376, 0), (2, 17, 128, 0), (2, 5, 224, 1000),
                                 (3, 17, 128, 0), (3, 5, 224, 1000)):
        plan = kvq.Plan(ns, chunk, w.batch * T * w.n_q_heads * ns * (w.head_dim + 2) * 4)
        got, want, _ = _run(w, [3100], T, window, plan=plan)
        _check(got, want, label=f"rows T={T} splits {ns} window {window}")


@pytest.mark.parametrize("n_tok", [2, 4, 8])
def test_rows_path_full_size_verify_window(n_tok):
    """Verify tokens at the end of the 128K context of the long workload (16
    query / 2 kv heads, head_dim 256, group-64 scales; one 16-row block, two
    blocks in one workgroup, and 64 rows through the chunk kernel) with the
    planner's split, every output against the oracle."""
    w = wl.WORKLOADS["long"]
    got, want, plan = _run(w, [131072 - n_tok], n_tok, 0)
    print(f"[chunk] 128K verify T={n_tok} plan {plan.n_splits} x {plan.chunk}", flush=True)
    _check(got, want, label=f"128K verify window T={n_tok}")


@pytest.mark.parametrize("name,n_tok", [("long_q4", 2), ("long_q4", 4), ("long_k8v4", 2)])
def test_rows_path_q4_full_size_verify_window(name, n_tok):
    """Verify tokens at the end of the 128K context over the 4-bit layouts (16
    query / 2 kv heads, head_dim 256; one and two 16-row workgroups per kv
    head) through the 4-bit decode partial kernel with the planner's split,
    every output against the oracle."""
    w = wl.WORKLOADS[name]
    got, want, plan = _run(w, [131072 - n_tok], n_tok, 0)
    print(f"[chunk] {name} 128K verify T={n_tok} plan {plan.n_splits} x {plan.chunk}", flush=True)
    _check(got, want, label=f"{name} 128K verify window T={n_tok}")


def test_rows_path_token_past_the_cache_end():
    """The rows path with its second token at max_ctx: the first token sees
    every key, the second gets a zero row."""
    w = wl.WORKLOADS["long"].with_(max_ctx=1024)
    got, want, _ = _run(w, [1023], 2, 0)
    _check(got[:, :1], want[:, :1], label="inside")
    assert not got[:, 1:].any()


@pytest.mark.parametrize("name", ["long", "long_q4", "long_k8v4"])
def test_single_token_chunk_equals_decode(name):
    """n_tok = 1 at start L - 1 is decode attention at context L."""
    import int8_quantized_kv_quant_amd as kvq
    import kvq_setup as ks
    w = wl.WORKLOADS[name].with_(max_ctx=4096)
    L = 3333
    lay, cache = ks.fill_cache(w, np.array([L]))
    q1 = wl.chunk_queries(w, 1)
    sm = 1 / 16
    got = kvq.chunk_attn(lay, cache, torch.from_numpy(q1).cuda(), torch.tensor([L - 1], dtype=torch.int32).cuda(),
                         0, sm, max_seq_len=L)
    dec = kvq.decode(lay, cache, torch.from_numpy(q1[:, 0].copy()).cuda(),
                     torch.tensor([L], dtype=torch.int32).cuda(), 0, sm, n_cu=ks.n_cu())
    torch.cuda.synchronize()
    assert np.abs(got[:, 0].float().cpu().numpy() - dec.float().cpu().numpy()).max() <= TOL


def test_tokens_past_the_cache_end_get_zero_rows():
    """A chunk that would run past max_ctx (a device precondition violation):
    tokens at or beyond max_ctx see no key and get zero rows; the others are
    exact; nothing outside the cache is read."""
    w = wl.WORKLOADS["long"].with_(max_ctx=1024)
    got, want, _ = _run(w, [1000], 40, 0)
    _check(got[:, :24], want[:, :24], label="inside")
    assert not got[:, 24:].any()


@pytest.mark.parametrize("name", ["long", "long_q4"])
def test_full_size_prompt_chunk_sampled(name):
    """The bench's prefill shape: 2048 tokens at position 30000 over the 128K
    layout of the long workload (16 query / 2 kv heads, head_dim 256, group-64
    scales; or its q4_0 form); sampled tokens against the oracle."""
    w = wl.WORKLOADS[name].with_(max_ctx=32768)
    T, start = 2048, 30000
    toks = [(0, 0), (0, 1), (0, 777), (0, 1500), (0, 2046), (0, 2047)]
    got, want, plan = _run(w, [start], T, 0, tokens=toks)
    print(f"[chunk] full-size plan {plan.n_splits} x {plan.chunk}", flush=True)
    _check(got, want, tokens=toks, label="full-size")


@pytest.mark.parametrize("n_tok", [4, 8])
def test_rows_path_batched_serving_shape(n_tok):
    """Verify windows for all 64 sequences of the batched-serving layout (32
    query / 8 kv heads, head_dim 128, group-64 scales; 16 and 32 (token, head)
    rows per kv head) at ragged starts, with the planner's split over the whole
    batch: every token of a sample of sequences (the first, one ending at the
    cache's end and two others; only these hold the workload's rows, the other
    caches stay zero) against the oracle."""
    import int8_quantized_kv_quant_amd as kvq
    import kvq_setup as ks
    w = wl.WORKLOADS["batched"].with_(max_ctx=2048)
    rng = np.random.default_rng(55)
    starts = rng.integers(0, 2048 - n_tok + 1, w.batch).astype(np.int64)
    starts[0], starts[1] = 0, 2048 - n_tok
    sample = [0, 1, 37, 63]
    ends = starts + n_tok
    lay, cache = ks.fill_cache(w, ends, seqs=sample)
    q = wl.chunk_queries(w, n_tok)
    sm = 1.0 / math.sqrt(w.head_dim)
    plan = kvq.kvq_plan_chunk(lay, w.batch, n_tok, w.n_q_heads, int(ends.max()), 0, ks.n_cu())
    got = kvq.chunk_attn(lay, cache, torch.from_numpy(q).cuda(), torch.from_numpy(starts.astype(np.int32)).cuda(),
                         0, sm, plan=plan)
    torch.cuda.synchronize()
    got = got.cpu().numpy().astype(np.float64)
    print(f"[chunk] batched T={n_tok} plan {plan.n_splits} x {plan.chunk}", flush=True)
    worst = 0.0
    for b in sample:
        oc = orc.Cache(1, w.max_ctx, w.n_kv_heads, w.head_dim, w.scale_group, w.k_dtype, w.v_dtype)
        oc.append(wl.kv_rows(w, "k", b, 0, int(ends[b]))[None], wl.kv_rows(w, "v", b, 0, int(ends[b]))[None], [0])
        want = orc.attend_chunk(q[b:b + 1], oc, starts[b:b + 1], 0, sm)
        worst = max(worst, float(np.abs(got[b] - want[0]).max()))
    print(f"[chunk] batched T={n_tok} max abs err {worst:.3g}", flush=True)
    assert worst <= TOL
