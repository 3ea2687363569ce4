"""GPU-side set-up of the synthetic workloads: uploads the seeded inputs of
``workloads`` and fills a cache with the library's own ``kv_quant_append``.

Plumbing only (allocation, upload, pointer offsets, download); the method's
arithmetic all happens in libkvq's kernels. Used by the GPU tests, the smoke
check and the benchmark.
"""
from __future__ import annotations

import numpy as np
import torch

import int8_quantized_kv_quant_amd as kvq
import workloads as wl


def layout_for(w: wl.Workload, order: str = "pos", max_ctx: int | None = None) -> kvq.Layout:
    return kvq.make_layout(w.n_kv_heads, w.head_dim, max_ctx or w.max_ctx, w.batch,
                           slot_dim=w.slot_dim, k_dtype=w.k_dtype, v_dtype=w.v_dtype,
                           scale_group=w.scale_group, order=order)


def _store_view(t: torch.Tensor, off: int) -> torch.Tensor:
    return t[off:]


def _seq_store(lay: kvq.Layout, t: torch.Tensor, dtype: int, b: int) -> torch.Tensor:
    """View of a flat store from sequence b on (a q4 store holds two elements per byte)."""
    off = b * lay.s_seq
    return t[off // 2:] if dtype == kvq.KVQ_STORE_Q4 else t[off:]


def append_rows(lay: kvq.Layout, cache: dict, b: int, start: int, k_rows: np.ndarray,
                v_rows: np.ndarray, device="cuda") -> None:
    """kv_quant_append of host fp16 rows [n][n_kv][d] of sequence b at `start`."""
    n = k_rows.shape[0]
    kn = torch.from_numpy(np.ascontiguousarray(k_rows)).to(device)
    vn = torch.from_numpy(np.ascontiguousarray(v_rows)).to(device)
    sp = torch.tensor([start], dtype=torch.int32, device=device)
    ks = cache["k_scales"]
    vs = cache["v_scales"]
    kvq.kv_quant_append(
        lay, _seq_store(lay, cache["k"], lay.k_dtype, b), _seq_store(lay, cache["v"], lay.v_dtype, b),
        None if ks is None else _store_view(ks, b * lay.ss_seq),
        None if vs is None else _store_view(vs, b * lay.ss_seq),
        kn, vn, sp, 1, n)


def append_rows_device(lay: kvq.Layout, cache: dict, b: int, start: int, k_rows, v_rows) -> None:
    """kv_quant_append of device fp16 rows [n][n_kv][d] of sequence b at `start`."""
    sp = torch.tensor([start], dtype=torch.int32, device=k_rows.device)
    ks = cache["k_scales"]
    vs = cache["v_scales"]
    kvq.kv_quant_append(
        lay, _seq_store(lay, cache["k"], lay.k_dtype, b), _seq_store(lay, cache["v"], lay.v_dtype, b),
        None if ks is None else _store_view(ks, b * lay.ss_seq),
        None if vs is None else _store_view(vs, b * lay.ss_seq),
        k_rows.contiguous(), v_rows.contiguous(), sp, 1, k_rows.shape[0])


def fill_cache(w: wl.Workload, lens: np.ndarray, order: str = "pos", device="cuda",
               block: int = 16384, upto=None, fill: int = 0, seqs=None):
    """Allocate the cache of workload w and append positions [0, upto_b) of every
    sequence in `seqs` (default: all; upto defaults to lens) in blocks of `block`
    tokens. Sequences not listed keep the fill value."""
    lay = layout_for(w, order)
    cache = kvq.alloc_cache(lay, w.batch, device=device, fill=fill)
    upto = lens if upto is None else upto
    for b in (range(w.batch) if seqs is None else seqs):
        L = int(upto[b])
        p = 0
        while p < L:
            n = min(block, L - p)
            append_rows(lay, cache, b, p, wl.kv_rows(w, "k", b, p, n), wl.kv_rows(w, "v", b, p, n), device)
            p += n
    return lay, cache


def rows_of(lay: kvq.Layout, store: torch.Tensor, b: int, positions, h: int, width: int | None = None):
    """Host copy of the rows (b, positions, h) of a flat store: [n][width]."""
    width = width or lay.head_dim
    pos = torch.as_tensor(np.asarray(positions, dtype=np.int64), device=store.device)
    base = b * lay.s_seq + h * lay.s_head + pos * lay.s_pos
    idx = base[:, None] + torch.arange(width, device=store.device)[None, :]
    return store[idx].cpu().numpy()


def q4_rows_of(lay: kvq.Layout, store: torch.Tensor, b: int, positions, h: int):
    """Host copy of the packed bytes of rows (b, positions, h) of a q4 store
    (a uint8 tensor, two codes per byte): [n][head_dim / 2]."""
    pos = torch.as_tensor(np.asarray(positions, dtype=np.int64), device=store.device)
    base = (b * lay.s_seq + h * lay.s_head + pos * lay.s_pos) // 2
    idx = base[:, None] + torch.arange(lay.head_dim // 2, device=store.device)[None, :]
    return store[idx].cpu().numpy()


def scales_of(lay: kvq.Layout, scales: torch.Tensor, b: int, positions, h: int, n: int | None = None):
    """Host copy of the n (default: an int8 store's count) fp16 scales of rows
    (b, positions, h): [len(positions)][n]."""
    pos = torch.as_tensor(np.asarray(positions, dtype=np.int64), device=scales.device)
    base = b * lay.ss_seq + h * lay.ss_head + pos * lay.ss_pos
    idx = base[:, None] + torch.arange(n or lay.n_groups, device=scales.device)[None, :]
    return scales[idx].cpu().numpy()


def n_cu(device="cuda") -> int:
    return torch.cuda.get_device_properties(device).multi_processor_count
