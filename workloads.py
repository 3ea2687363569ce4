"""Seeded synthetic inputs for the INT8 KV-cache decode path.

This module only draws random numbers and describes shapes. It holds none of
the method's arithmetic (no quantization, no attention): both the CPU oracle
and the HIP path consume the arrays produced here, so that they are compared
on identical inputs.

Shapes follow the workloads the source pages discuss:

* ``tiny``     -- one decode step, 8 query / 2 kv heads, head_dim 64, context
                  256, one scale per (position, kv head).
* ``gemma``    -- a Gemma-style sliding layer: 8 query / 1 kv head, head_dim 256
                  stored in a 512-wide cache slot, window 512, contexts
                  512..4096 (genie-ai-runtime releases, v1.2.1 "Bugs fixed" and
                  v1.3.0 "Details").
* ``long``     -- 16 query / 2 kv heads, head_dim 256, one fp16 scale per 64
                  values, context 131072 (Strata pull request 2698, "What it
                  does"); K carries 1 % outlier channels scaled by 20.
* ``batched``  -- 64 sequences with lengths uniform in [1024, 32768], 32 query /
                  8 kv heads, head_dim 128, group-64 scales.
* ``mixed``    -- k8v32 / k32v8 stores (Strata pull request 2698), 30000
                  positions prefilled, a 2048-token chunk appended at 30000,
                  then a decode step at context 32048.

Every value is ``standard_normal`` float32 rounded to float16, drawn from
``numpy.random.default_rng`` streams whose seeds are derived from the workload
seed, the sequence index and the tensor kind, so any sequence can be
regenerated on its own without materialising the others.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Sequence

import numpy as np

# Stream identifiers mixed into the per-tensor seeds.
_KIND = {"q": 1, "k": 2, "v": 3, "lens": 4, "outlier": 5}


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    slot_dim: int
    scale_group: int          # == head_dim: one scale per (position, kv head)
    max_ctx: int              # positions allocated per sequence
    window: int               # 0 = no sliding window
    seed: int
    k_dtype: str = "int8"     # "int8", "fp32" or "q4" (rotated Q4_0 blocks, head_dim 256)
    v_dtype: str = "int8"
    contexts: Sequence[int] = field(default_factory=tuple)  # decode contexts (batch 1)
    outlier_frac: float = 0.0  # fraction of K channels scaled by outlier_gain
    outlier_gain: float = 1.0
    ragged: tuple = ()        # (lo, hi) inclusive length range for ragged batches
    prefill: int = 0          # positions filled before the appended chunk
    append: int = 0           # tokens quantize-appended as one chunk

    @property
    def group_size(self) -> int:
        return self.scale_group

    @property
    def n_groups(self) -> int:
        return self.head_dim // self.scale_group

    @property
    def gqa(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def with_(self, **kw) -> "Workload":
        d = {f: getattr(self, f) for f in self.__dataclass_fields__}
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 8, 2, 64, 64, 64, 256, 0, 0, contexts=(256,)),
    "gemma": Workload("gemma", 1, 8, 1, 256, 512, 256, 4096, 512, 1,
                      contexts=(512, 1024, 2048, 4096)),
    "long": Workload("long", 1, 16, 2, 256, 256, 64, 131072, 0, 2,
                     contexts=(131072,), outlier_frac=0.01, outlier_gain=20.0),
    "batched": Workload("batched", 64, 32, 8, 128, 128, 64, 32768, 0, 3,
                        ragged=(1024, 32768)),
    "mixed_k8v32": Workload("mixed_k8v32", 1, 16, 2, 256, 256, 64, 32768, 0, 4,
                            k_dtype="int8", v_dtype="fp32", contexts=(32048,),
                            prefill=30000, append=2048),
    "mixed_k32v8": Workload("mixed_k32v8", 1, 16, 2, 256, 256, 64, 32768, 0, 4,
                            k_dtype="fp32", v_dtype="int8", contexts=(32048,),
                            prefill=30000, append=2048),
    # the long-context shape with the 4-bit stores (Strata PR 2698, "Not in
    # this PR": q4_0 for K and V, k8v4 for V only, head_dim 256)
    "long_q4": Workload("long_q4", 1, 16, 2, 256, 256, 64, 131072, 0, 2, k_dtype="q4", v_dtype="q4",
                        contexts=(131072,), outlier_frac=0.01, outlier_gain=20.0),
    "long_k8v4": Workload("long_k8v4", 1, 16, 2, 256, 256, 64, 131072, 0, 2, k_dtype="int8", v_dtype="q4",
                          contexts=(131072,), outlier_frac=0.01, outlier_gain=20.0),
}


def _rng(seed: int, kind: str, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(seed), _KIND[kind], int(index)])


def _normal_f16(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16)


def seq_lens(w: Workload, context: int | None = None) -> np.ndarray:
    """int32 [batch] context lengths (positions in cache, current token included)."""
    if w.ragged:
        lo, hi = w.ragged
        return _rng(w.seed, "lens").integers(lo, hi + 1, w.batch).astype(np.int32)
    L = context if context is not None else w.contexts[-1]
    return np.full(w.batch, L, dtype=np.int32)


def queries(w: Workload, seed_offset: int = 0) -> np.ndarray:
    """float16 [batch][n_q_heads][head_dim]."""
    return _normal_f16(_rng(w.seed + seed_offset, "q"), (w.batch, w.n_q_heads, w.head_dim))


def chunk_queries(w: Workload, n_tok: int, seed_offset: int = 0) -> np.ndarray:
    """float16 [batch][n_tok][n_q_heads][head_dim]: query rows of a chunk of
    n_tok consecutive tokens per sequence (its own stream, apart from the
    single-token queries)."""
    return _normal_f16(_rng(w.seed + seed_offset, "q", 1), (w.batch, n_tok, w.n_q_heads, w.head_dim))


def outlier_channels(w: Workload) -> np.ndarray:
    """int64 [n_kv_heads][n_out]: K channels scaled by outlier_gain (per kv head)."""
    n_out = int(round(w.outlier_frac * w.head_dim))
    rng = _rng(w.seed, "outlier")
    if n_out == 0:
        return np.zeros((w.n_kv_heads, 0), dtype=np.int64)
    return np.stack([rng.choice(w.head_dim, n_out, replace=False)
                     for _ in range(w.n_kv_heads)]).astype(np.int64)


def kv_rows(w: Workload, kind: str, b: int, start: int, n: int) -> np.ndarray:
    """float16 [n][n_kv_heads][head_dim] rows for positions [start, start+n) of sequence b.

    Rows are drawn in fixed blocks of 1024 positions so that any sub-range
    regenerates bit-identically.
    """
    assert kind in ("k", "v")
    out = np.empty((n, w.n_kv_heads, w.head_dim), dtype=np.float16)
    blk = 1024
    chans = outlier_channels(w) if kind == "k" else None
    p = start
    while p < start + n:
        bi = p // blk
        rng = _rng(w.seed, kind, b * 1_000_003 + bi)
        block = rng.standard_normal((blk, w.n_kv_heads, w.head_dim), dtype=np.float32)
        if chans is not None and chans.shape[1]:
            for h in range(w.n_kv_heads):
                block[:, h, chans[h]] *= np.float32(w.outlier_gain)
        block = block.astype(np.float16)
        lo = p - bi * blk
        take = min(blk - lo, start + n - p)
        out[p - start:p - start + take] = block[lo:lo + take]
        p += take
    return out


def uniform_rows(seed: int, shape, scale: float = 1.0) -> np.ndarray:
    """float16 array of N(0, scale^2) values for edge-case tests."""
    rng = np.random.default_rng([int(seed), 99])
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(np.float16)


def kv_bytes_per_step(w: Workload, lens: np.ndarray) -> int:
    """Algorithmic bytes the decode step must read: codes (1 B, or 1/2 B for a
    q4 store) or fp32 values (4 B) for every attended position, plus the fp16
    scales of int8 and q4 stores.
    The slot tail beyond head_dim is not read and not counted."""
    per_pos = 0
    for dt in (w.k_dtype, w.v_dtype):
        if dt == "int8":
            per_pos += w.head_dim + 2 * w.n_groups
        elif dt == "q4":  # two codes per byte, one fp16 scale per 32 values
            per_pos += w.head_dim // 2 + 2 * (w.head_dim // 32)
        else:
            per_pos += 4 * w.head_dim
    total = 0
    for L in lens.tolist():
        lo = max(0, L - w.window) if w.window else 0
        total += (L - lo) * w.n_kv_heads * per_pos
    return int(total)
