"""Python binding of libkvq (include/kvq.h): INT8 KV-cache decode attention on MI355X.

Argument marshalling only. Every step of the decode path -- quantize-append,
split-K partials, reduce -- runs in the HIP kernels of ``libkvq.so``; PyTorch is
used for device memory and the current stream. If the library has not been
built, importing works but every call raises ``KvqLibraryMissing``: there is
no CPU fallback.

Build with ``python -m int8_quantized_kv_quant_amd.build_lib``.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

__all__ = [
    "KVQ_STORE_INT8", "KVQ_STORE_FP32", "KVQ_STORE_Q4", "KvqError", "KvqLibraryMissing", "Layout", "Plan",
    "lib_path", "load", "kvq_version", "kvq_status_string", "kvq_plan", "kv_quant_append",
    "kv_decode_attn_splitk", "kv_append_decode_splitk", "kv_decode_reduce", "kvq_plan_chunk",
    "kv_chunk_attn", "kvq_blob_size", "kv_cache_pack", "kv_cache_unpack", "kvq_stream_read", "BlobHeader",
    "kv_decode_attn_static", "STATIC_SCRATCH_BYTES", "kv_decode_attn", "arrive_count", "kvq_decode_launches",
    "make_layout",
    "alloc_cache", "decode", "chunk_attn",
    "EXPORTED_SYMBOLS",
]

KVQ_STORE_INT8 = 1
KVQ_STORE_FP32 = 2
KVQ_STORE_Q4 = 3
_DT = {"int8": KVQ_STORE_INT8, "fp32": KVQ_STORE_FP32, "q4": KVQ_STORE_Q4}
Q4_BLOCK = 32  # values per Q4_0 block (one fp16 scale each)

EXPORTED_SYMBOLS = ("kvq_plan", "kv_quant_append", "kv_decode_attn_splitk", "kv_append_decode_splitk",
                    "kv_decode_reduce", "kvq_plan_chunk", "kv_chunk_attn", "kvq_blob_size", "kv_cache_pack",
                    "kv_cache_unpack", "kvq_stream_read", "kvq_status_string", "kvq_version",
                    "kv_decode_attn_static", "kv_decode_attn", "kvq_decode_launches")

# Bytes of the library's static device scratch (KVQ_STATIC_SCRATCH_BYTES).
STATIC_SCRATCH_BYTES = 16 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_HERE, "libkvq.so")


class KvqLibraryMissing(RuntimeError):
    pass


class KvqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {kvq_status_string(status)} (status {status})")


class _Layout(ctypes.Structure):
    _fields_ = [("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("slot_dim", ctypes.c_int32), ("k_dtype", ctypes.c_int32),
                ("v_dtype", ctypes.c_int32), ("scale_group", ctypes.c_int32),
                ("max_ctx", ctypes.c_int64),
                ("s_seq", ctypes.c_int64), ("s_pos", ctypes.c_int64), ("s_head", ctypes.c_int64),
                ("ss_seq", ctypes.c_int64), ("ss_pos", ctypes.c_int64), ("ss_head", ctypes.c_int64)]


class _Plan(ctypes.Structure):
    _fields_ = [("n_splits", ctypes.c_int32), ("chunk", ctypes.c_int32), ("ws_bytes", ctypes.c_int64)]


@dataclass(frozen=True)
class Layout:
    """Mirror of kvq_layout. Strides are in elements (see include/kvq.h)."""
    n_kv_heads: int
    head_dim: int
    slot_dim: int
    k_dtype: int
    v_dtype: int
    scale_group: int
    max_ctx: int
    s_seq: int
    s_pos: int
    s_head: int
    ss_seq: int
    ss_pos: int
    ss_head: int

    def c(self) -> _Layout:
        return _Layout(*[getattr(self, f[0]) for f in _Layout._fields_])

    @property
    def n_groups(self) -> int:
        """Scales per row of an int8 store."""
        return self.head_dim // self.scale_group

    def groups_of(self, dtype: int) -> int:
        """Scales per row of a store of this type (0: none)."""
        if dtype == KVQ_STORE_Q4:
            return self.head_dim // Q4_BLOCK
        return self.n_groups if dtype == KVQ_STORE_INT8 else 0


@dataclass(frozen=True)
class Plan:
    n_splits: int
    chunk: int
    ws_bytes: int

    def c(self) -> _Plan:
        return _Plan(self.n_splits, self.chunk, self.ws_bytes)


_lib = None


def load():
    """Load libkvq.so (once). Raises KvqLibraryMissing if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    p = lib_path()
    if not os.path.exists(p):
        raise KvqLibraryMissing(f"{p} not built; run `python -m int8_quantized_kv_quant_amd.build_lib`")
    lib = ctypes.CDLL(p)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    LP, PP = ctypes.POINTER(_Layout), ctypes.POINTER(_Plan)
    lib.kvq_plan.argtypes = [LP, i32, i32, i32, i32, i32, PP]
    lib.kv_quant_append.argtypes = [LP, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp]
    lib.kv_decode_attn_splitk.argtypes = [LP, vp, vp, vp, vp, vp, i32, i32, vp, i32, f32, PP, vp, i64, vp]
    lib.kv_append_decode_splitk.argtypes = [LP, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, i32, f32, PP, vp,
                                            i64, vp]
    lib.kv_decode_reduce.argtypes = [LP, vp, i64, vp, i32, i32, i32, PP, vp, vp]
    lib.kv_decode_attn_static.argtypes = [LP, vp, vp, vp, vp, vp, i32, i32, vp, i32, f32, PP, vp, vp]
    lib.kv_decode_attn.argtypes = [LP, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, i32, f32, PP, vp, i64, vp, vp,
                                   vp]
    lib.kvq_decode_launches.argtypes = [LP, i32, i32, PP, ctypes.POINTER(i32)]
    lib.kvq_plan_chunk.argtypes = [LP, i32, i32, i32, i32, i32, i32, PP]
    HP = ctypes.POINTER(BlobHeader)
    lib.kvq_blob_size.argtypes = [LP, i32, ctypes.POINTER(i64)]
    lib.kv_cache_pack.argtypes = [LP, vp, vp, vp, vp, i32, i32, i32, vp, i64, HP, vp]
    lib.kv_cache_unpack.argtypes = [LP, vp, vp, vp, vp, i32, i32, HP, vp, i64, vp]
    lib.kv_chunk_attn.argtypes = [LP, vp, vp, vp, vp, vp, i32, i32, i32, vp, i32, f32, PP, vp, i64, vp, vp]
    lib.kvq_stream_read.argtypes = [vp, i64, vp, i32, vp]
    lib.kvq_status_string.argtypes = [ctypes.c_int]
    lib.kvq_status_string.restype = ctypes.c_char_p
    lib.kvq_version.argtypes = []
    for fn in ("kvq_plan", "kv_quant_append", "kv_decode_attn_splitk", "kv_append_decode_splitk",
               "kv_decode_reduce", "kvq_plan_chunk", "kv_chunk_attn", "kvq_blob_size", "kv_cache_pack",
               "kv_cache_unpack", "kvq_stream_read", "kvq_version", "kv_decode_attn_static", "kv_decode_attn",
               "kvq_decode_launches"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def kvq_status_string(status: int) -> str:
    return load().kvq_status_string(int(status)).decode()


def kvq_version() -> int:
    return load().kvq_version()


def _check(fn: str, st: int):
    if st != 0:
        raise KvqError(fn, st)


def _ptr(x) -> int | None:
    """Device/host address of a tensor (or an int address, or None -> NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        if not torch.cuda.is_available():
            return None
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def kvq_plan(layout: Layout, batch: int, n_q_heads: int, max_seq_len: int, window: int,
             n_cu: int) -> Plan:
    out = _Plan()
    _check("kvq_plan", load().kvq_plan(ctypes.byref(layout.c()), batch, n_q_heads, max_seq_len,
                                       window, n_cu, ctypes.byref(out)))
    return Plan(out.n_splits, out.chunk, out.ws_bytes)


def kv_quant_append(layout: Layout, k_store, v_store, k_scales, v_scales, k_new, v_new, start_pos,
                    batch: int, n_tok: int, stream=None) -> None:
    _check("kv_quant_append", load().kv_quant_append(
        ctypes.byref(layout.c()), _ptr(k_store), _ptr(v_store), _ptr(k_scales), _ptr(v_scales),
        _ptr(k_new), _ptr(v_new), _ptr(start_pos), batch, n_tok, _stream(stream)))


def kv_decode_attn_splitk(layout: Layout, k_store, v_store, k_scales, v_scales, q, batch: int,
                          n_q_heads: int, seq_lens, window: int, sm_scale: float, plan: Plan,
                          ws, ws_bytes: int, stream=None) -> None:
    _check("kv_decode_attn_splitk", load().kv_decode_attn_splitk(
        ctypes.byref(layout.c()), _ptr(k_store), _ptr(v_store), _ptr(k_scales), _ptr(v_scales),
        _ptr(q), batch, n_q_heads, _ptr(seq_lens), window, sm_scale, ctypes.byref(plan.c()),
        _ptr(ws), ws_bytes, _stream(stream)))


def kv_append_decode_splitk(layout: Layout, k_store, v_store, k_scales, v_scales, k_new, v_new, q,
                            batch: int, n_q_heads: int, seq_lens, window: int, sm_scale: float,
                            plan: Plan, ws, ws_bytes: int, stream=None) -> None:
    _check("kv_append_decode_splitk", load().kv_append_decode_splitk(
        ctypes.byref(layout.c()), _ptr(k_store), _ptr(v_store), _ptr(k_scales), _ptr(v_scales),
        _ptr(k_new), _ptr(v_new), _ptr(q), batch, n_q_heads, _ptr(seq_lens), window, sm_scale,
        ctypes.byref(plan.c()), _ptr(ws), ws_bytes, _stream(stream)))


def kv_decode_reduce(layout: Layout, ws, ws_bytes: int, seq_lens, batch: int, n_q_heads: int,
                     window: int, plan: Plan, out, stream=None) -> None:
    _check("kv_decode_reduce", load().kv_decode_reduce(
        ctypes.byref(layout.c()), _ptr(ws), ws_bytes, _ptr(seq_lens), batch, n_q_heads, window,
        ctypes.byref(plan.c()), _ptr(out), _stream(stream)))


def kv_decode_attn(layout: Layout, k_store, v_store, k_scales, v_scales, k_new, v_new, q, batch: int,
                   n_q_heads: int, seq_lens, window: int, sm_scale: float, plan: Plan, ws, ws_bytes: int,
                   arrive, out, stream=None) -> None:
    """Append (k_new, v_new non-None) + partials + combine into out in one call;
    arrive: zeroed int32/uint32 device counters (arrive_count of them), left
    zero by every call."""
    _check("kv_decode_attn", load().kv_decode_attn(
        ctypes.byref(layout.c()), _ptr(k_store), _ptr(v_store), _ptr(k_scales), _ptr(v_scales), _ptr(k_new),
        _ptr(v_new), _ptr(q), batch, n_q_heads, _ptr(seq_lens), window, sm_scale, ctypes.byref(plan.c()), _ptr(ws),
        ws_bytes, _ptr(arrive), _ptr(out), _stream(stream)))


def kvq_decode_launches(layout: Layout, batch: int, n_q_heads: int, plan: Plan) -> int:
    """Kernel launches kv_decode_attn makes for these arguments (1, 2, or 0)."""
    n = ctypes.c_int32(-1)
    _check("kvq_decode_launches", load().kvq_decode_launches(ctypes.byref(layout.c()), batch, n_q_heads,
                                                             ctypes.byref(plan.c()), ctypes.byref(n)))
    return n.value


def arrive_count(layout: Layout, batch: int, n_q_heads: int) -> int:
    """Number of kv_decode_attn arrival counters: batch * n_q_heads."""
    return max(1, batch * n_q_heads)


def kv_decode_attn_static(layout: Layout, k_store, v_store, k_scales, v_scales, q, batch: int, n_q_heads: int,
                          seq_lens, window: int, sm_scale: float, plan: Plan, out, stream=None) -> None:
    """Partials + combine with the partials in the library's static scratch
    (no workspace argument; nothing allocated)."""
    _check("kv_decode_attn_static", load().kv_decode_attn_static(
        ctypes.byref(layout.c()), _ptr(k_store), _ptr(v_store), _ptr(k_scales), _ptr(v_scales), _ptr(q), batch,
        n_q_heads, _ptr(seq_lens), window, sm_scale, ctypes.byref(plan.c()), _ptr(out), _stream(stream)))


def kvq_plan_chunk(layout: Layout, batch: int, n_tok: int, n_q_heads: int, max_seq_len: int, window: int,
                   n_cu: int) -> Plan:
    out = _Plan()
    _check("kvq_plan_chunk", load().kvq_plan_chunk(ctypes.byref(layout.c()), batch, n_tok, n_q_heads,
                                                   max_seq_len, window, n_cu, ctypes.byref(out)))
    return Plan(out.n_splits, out.chunk, out.ws_bytes)


def kv_chunk_attn(layout: Layout, k_store, v_store, k_scales, v_scales, q, batch: int, n_tok: int,
                  n_q_heads: int, start_pos, window: int, sm_scale: float, plan: Plan, ws, ws_bytes: int, out,
                  stream=None) -> None:
    _check("kv_chunk_attn", load().kv_chunk_attn(
        ctypes.byref(layout.c()), _ptr(k_store), _ptr(v_store), _ptr(k_scales), _ptr(v_scales), _ptr(q),
        batch, n_tok, n_q_heads, _ptr(start_pos), window, sm_scale, ctypes.byref(plan.c()), _ptr(ws), ws_bytes,
        _ptr(out), _stream(stream)))


class BlobHeader(ctypes.Structure):
    """kvq_blob_header: the layout facts a cache blob carries."""
    _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_uint32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("k_dtype", ctypes.c_int32), ("v_dtype", ctypes.c_int32),
                ("scale_group", ctypes.c_int32), ("n_pos", ctypes.c_int32), ("payload_bytes", ctypes.c_int64)]


def kvq_stream_read(buf, n_bytes: int, sink, n_cu: int, stream=None) -> None:
    """The read-only streaming reference (measurement only)."""
    _check("kvq_stream_read", load().kvq_stream_read(_ptr(buf), n_bytes, _ptr(sink), n_cu, _stream(stream)))


def kvq_blob_size(layout: Layout, n_pos: int) -> int:
    out = ctypes.c_int64()
    _check("kvq_blob_size", load().kvq_blob_size(ctypes.byref(layout.c()), n_pos, ctypes.byref(out)))
    return out.value


def kv_cache_pack(layout: Layout, k_store, v_store, k_scales, v_scales, seq: int, pos0: int, n_pos: int, dst,
                  dst_bytes: int, stream=None) -> BlobHeader:
    hdr = BlobHeader()
    _check("kv_cache_pack", load().kv_cache_pack(
        ctypes.byref(layout.c()), _ptr(k_store), _ptr(v_store), _ptr(k_scales), _ptr(v_scales), seq, pos0, n_pos,
        _ptr(dst), dst_bytes, ctypes.byref(hdr), _stream(stream)))
    return hdr


def kv_cache_unpack(layout: Layout, k_store, v_store, k_scales, v_scales, seq: int, pos0: int,
                    header: BlobHeader, src, src_bytes: int, stream=None) -> None:
    _check("kv_cache_unpack", load().kv_cache_unpack(
        ctypes.byref(layout.c()), _ptr(k_store), _ptr(v_store), _ptr(k_scales), _ptr(v_scales), seq, pos0,
        ctypes.byref(header), _ptr(src), src_bytes, _stream(stream)))


# --------------------------------------------------------------------------
# Allocation helpers (memory plumbing; no arithmetic of the method)
# --------------------------------------------------------------------------

def make_layout(n_kv_heads: int, head_dim: int, max_ctx: int, batch: int = 1, slot_dim: int | None = None,
                k_dtype: str = "int8", v_dtype: str = "int8", scale_group: int | None = None,
                order: str = "pos") -> Layout:
    """Dense cache layout. order="pos": [seq][pos][head][slot] (positions major,
    as the genie pool indexes its scales); order="head": [seq][head][pos][slot]."""
    slot = slot_dim or head_dim
    g = scale_group or head_dim
    # the scale arrays share their strides: room for the longer scale row
    ng = max(head_dim // Q4_BLOCK if dt == "q4" else head_dim // g for dt in (k_dtype, v_dtype))
    if order == "pos":
        s_head, s_pos, s_seq = slot, n_kv_heads * slot, max_ctx * n_kv_heads * slot
        ss_head, ss_pos, ss_seq = ng, n_kv_heads * ng, max_ctx * n_kv_heads * ng
    elif order == "head":
        s_pos, s_head, s_seq = slot, max_ctx * slot, n_kv_heads * max_ctx * slot
        ss_pos, ss_head, ss_seq = ng, max_ctx * ng, n_kv_heads * max_ctx * ng
    else:
        raise ValueError(order)
    return Layout(n_kv_heads, head_dim, slot, _DT[k_dtype], _DT[v_dtype], g, max_ctx,
                  s_seq, s_pos, s_head, ss_seq, ss_pos, ss_head)


def alloc_cache(layout: Layout, batch: int, device="cuda", fill=0):
    """Torch tensors for a dense cache of `batch` sequences: dict with k, v
    (int8, float32, or uint8 holding two 4-bit codes per byte; flat) and
    k_scales, v_scales (float16 flat or None)."""
    import torch
    n = batch * layout.s_seq
    ns = batch * layout.ss_seq
    out = {}
    for s, dt in (("k", layout.k_dtype), ("v", layout.v_dtype)):
        if dt == KVQ_STORE_INT8:
            out[s] = torch.full((n,), fill, dtype=torch.int8, device=device)
            out[s + "_scales"] = torch.zeros((ns,), dtype=torch.float16, device=device)
        elif dt == KVQ_STORE_Q4:
            out[s] = torch.full((n // 2,), fill, dtype=torch.uint8, device=device)
            out[s + "_scales"] = torch.zeros((ns,), dtype=torch.float16, device=device)
        else:
            out[s] = torch.full((n,), fill, dtype=torch.float32, device=device)
            out[s + "_scales"] = None
    return out


def decode(layout: Layout, cache: dict, q, seq_lens, window: int, sm_scale: float | None = None,
           plan: Plan | None = None, ws=None, out=None, n_cu: int | None = None, stream=None,
           new_kv=None, arrive=None):
    """One decode step: kv_decode_attn_splitk then kv_decode_reduce on the
    current stream; with new_kv = (k_new, v_new) (fp16 [batch][n_kv][head_dim] on
    the device) the token's quantize-append is fused in (kv_append_decode_splitk,
    appending at position seq_lens[b] - 1). With arrive (zeroed int32 device
    counters, arrive_count of them) the step is one kv_decode_attn call instead.
    q: fp16 [batch][n_q][head_dim] on the device; seq_lens: int32 [batch] on the
    device. Returns the fp16 output."""
    import torch
    batch, n_q, d = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if plan is None:
        if n_cu is None:
            n_cu = torch.cuda.get_device_properties(q.device).multi_processor_count
        plan = kvq_plan(layout, batch, n_q, layout.max_ctx, window, n_cu)
    if ws is None:
        ws = torch.empty(max(plan.ws_bytes, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((batch, n_q, d), dtype=torch.float16, device=q.device)
    if arrive is not None:
        k_new, v_new = new_kv if new_kv is not None else (None, None)
        kv_decode_attn(layout, cache["k"], cache["v"], cache["k_scales"], cache["v_scales"], k_new, v_new, q,
                       batch, n_q, seq_lens, window, sm_scale, plan, ws, ws.numel(), arrive, out, stream)
        return out
    if new_kv is None:
        kv_decode_attn_splitk(layout, cache["k"], cache["v"], cache["k_scales"], cache["v_scales"], q,
                              batch, n_q, seq_lens, window, sm_scale, plan, ws, ws.numel(), stream)
    else:
        kv_append_decode_splitk(layout, cache["k"], cache["v"], cache["k_scales"], cache["v_scales"],
                                new_kv[0], new_kv[1], q, batch, n_q, seq_lens, window, sm_scale, plan,
                                ws, ws.numel(), stream)
    kv_decode_reduce(layout, ws, ws.numel(), seq_lens, batch, n_q, window, plan, out, stream)
    return out


def chunk_attn(layout: Layout, cache: dict, q, start_pos, window: int, sm_scale: float | None = None,
               plan: Plan | None = None, max_seq_len: int | None = None, ws=None, out=None,
               n_cu: int | None = None, stream=None):
    """Chunk attention (kv_chunk_attn) of q fp16 [batch][n_tok][n_q][head_dim]
    at device positions start_pos (int32 [batch]) over the cache. Returns the
    fp16 output [batch][n_tok][n_q][head_dim]."""
    import torch
    batch, n_tok, n_q, d = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if plan is None:
        if n_cu is None:
            n_cu = torch.cuda.get_device_properties(q.device).multi_processor_count
        plan = kvq_plan_chunk(layout, batch, n_tok, n_q, max_seq_len or layout.max_ctx, window, n_cu)
    if ws is None:
        ws = torch.empty(max(plan.ws_bytes, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((batch, n_tok, n_q, d), dtype=torch.float16, device=q.device)
    kv_chunk_attn(layout, cache["k"], cache["v"], cache["k_scales"], cache["v_scales"], q, batch, n_tok, n_q,
                  start_pos, window, sm_scale, plan, ws, ws.numel(), out, stream)
    return out
