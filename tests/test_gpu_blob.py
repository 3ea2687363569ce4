"""Cache blob (kv_cache_pack / kv_cache_unpack) on the GPU: the payload is
bit-identical to the oracle's blob of the same cache rows, and a blob placed
into a cache of another layout order gives the same attention output, bit for
bit, as the cache it came from.

genie-ai-runtime release v0.1.0-alpha.11, "--int8-kv triage", and release
v0.1.0-alpha.12, "Path F (#45) interop guard": saved int8 caches must carry
their scales."""
import math

import numpy as np
import pytest

import workloads as wl
from oracle import kvq_oracle as orc

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _oracle_cache(w, b, L):
    c = orc.Cache(1, L, w.n_kv_heads, w.head_dim, w.scale_group, w.k_dtype, w.v_dtype)
    c.append(wl.kv_rows(w, "k", b, 0, L)[None], wl.kv_rows(w, "v", b, 0, L)[None], [0])
    return c


CASES = {
    "long_k8v8_g64": (wl.WORKLOADS["long"].with_(max_ctx=4096, batch=2), 1, 1000, 1500),
    "gemma_slot512_per_row": (wl.WORKLOADS["gemma"].with_(max_ctx=2048), 0, 0, 1111),
    "k8v32": (wl.WORKLOADS["mixed_k8v32"].with_(max_ctx=2048), 0, 37, 700),
    "k32v8": (wl.WORKLOADS["mixed_k32v8"].with_(max_ctx=2048), 0, 5, 64),
    "batched_d128": (wl.WORKLOADS["batched"].with_(batch=3, max_ctx=1024), 2, 100, 333),
    "q4_0": (wl.WORKLOADS["long_q4"].with_(max_ctx=2048, batch=2), 1, 9, 1001),
    "k8v4": (wl.WORKLOADS["long_k8v4"].with_(max_ctx=2048), 0, 0, 777),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_pack_equals_the_oracle_blob(case):
    import int8_quantized_kv_quant_amd as kvq
    import kvq_setup as ks
    w, b, pos0, n = CASES[case]
    lens = np.full(w.batch, pos0 + n)
    lay, cache = ks.fill_cache(w, lens)
    size = kvq.kvq_blob_size(lay, n)
    dst = torch.full((size + 64,), 0x5A, dtype=torch.uint8, device="cuda")
    hdr = kvq.kv_cache_pack(lay, cache["k"], cache["v"], cache["k_scales"], cache["v_scales"], b, pos0, n, dst, size)
    torch.cuda.synchronize()
    oc = _oracle_cache(w, b, pos0 + n)
    want = np.frombuffer(orc.blob_payload(oc, 0, pos0, n), dtype=np.uint8)
    got = dst[:size].cpu().numpy()
    assert hdr.payload_bytes == size == len(want)
    assert np.array_equal(got, want)
    assert (dst[size:].cpu().numpy() == 0x5A).all(), "pack wrote past the payload"
    oh = orc.blob_header(oc, n)
    assert (hdr.magic, hdr.version, hdr.n_kv_heads, hdr.head_dim, hdr.k_dtype, hdr.v_dtype, hdr.scale_group,
            hdr.n_pos) == (oh["magic"], oh["version"], oh["n_kv_heads"], oh["head_dim"], oh["k_dtype"],
                           oh["v_dtype"], oh["scale_group"], oh["n_pos"])


@pytest.mark.parametrize("case", ["long_k8v8_g64", "k8v32", "batched_d128", "q4_0", "k8v4"])
def test_unpacked_into_another_layout_attends_identically(case):
    """Pack positions [0, L) of one sequence, place them into a heads-major
    cache, and decode both: the outputs are bit-identical, and the rows outside
    the placed range are untouched."""
    import int8_quantized_kv_quant_amd as kvq
    import kvq_setup as ks
    w, b, pos0, n = CASES[case]
    L = pos0 + n
    lay, cache = ks.fill_cache(w, np.full(w.batch, L))
    size = kvq.kvq_blob_size(lay, L)
    blob = torch.empty(size, dtype=torch.uint8, device="cuda")
    hdr = kvq.kv_cache_pack(lay, cache["k"], cache["v"], cache["k_scales"], cache["v_scales"], b, 0, L, blob, size)
    lay2 = ks.layout_for(w, "head")
    cache2 = kvq.alloc_cache(lay2, w.batch, fill=0)
    kvq.kv_cache_unpack(lay2, cache2["k"], cache2["v"], cache2["k_scales"], cache2["v_scales"], b, 0, hdr, blob, size)
    q = torch.from_numpy(wl.queries(w)).cuda()
    ld = torch.from_numpy(np.full(w.batch, L, dtype=np.int32)).cuda()
    sm = 1.0 / math.sqrt(w.head_dim)
    plan = kvq.kvq_plan(lay, w.batch, w.n_q_heads, L, 0, ks.n_cu())
    o1 = kvq.decode(lay, cache, q, ld, 0, sm, plan=plan)
    o2 = kvq.decode(lay2, cache2, q, ld, 0, sm, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(o1[b], o2[b])
    for s, dt in (("k", w.k_dtype), ("v", w.v_dtype)):
        other = [x for x in range(w.batch) if x != b]
        if other:
            pos = np.arange(0, L, 97)
            rows = (ks.q4_rows_of(lay2, cache2[s], other[0], pos, 0) if dt == "q4"
                    else ks.rows_of(lay2, cache2[s], other[0], pos, 0))
            assert not rows.any()
