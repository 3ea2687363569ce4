"""CPU oracle for the INT8 KV cache: quantize-append, single-token decode attention
and chunk (several query tokens, causal) attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The library
(``int8_quantized_kv_quant_amd``) never imports, links or calls it, and this
module shares no code, table or helper with the HIP path.

Everything is plain numpy in float64 unless a page fixes the precision (the
scales are float16 because the pages store them that way). It is slow and
written to be checked by eye against the pages:

* genie-ai-runtime release v0.1.0-alpha.12 ("Path I: INT8 KV cache"), the
  "Path I series" table: one scale per (layer, position, kv head), captured by
  a per-head conversion (#64); attention dequantizes with the scale of its
  position and kv head (#65).
* genie-ai-runtime release v0.1.0-alpha.11, "--int8-kv triage": a missing
  scale must not silently become 1.0, and the scale rows are one per kv head.
* genie-ai-runtime releases, v1.3.0 "split-K decode attention": the KV range
  is split into blocks that each form an online-softmax partial, and a reduce
  combines them; results equal the single-pass kernel. "Details": sliding
  window mask, Gemma slot width (v1.2.1 "Bugs fixed").
* Strata pull request 2698, "What it does": int8 codes, each 64-value group
  sharing an FP16 scale equal to its absmax / 127; in k8v32 / k32v8 only
  one of the two stores is quantized, and the fp32 one enters attention as is.
* Strata pull request 2698, "Not in this PR": the 4-bit stores (q4_0 for both,
  k8v4 for V only) use a Hadamard rotation over head_dim 256 with Q4_0
  blocks; K is rotated together with the queries, V is rotated and the output
  is rotated back.

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * the fp16 scale is the round-to-nearest-even fp16 value of absmax / 127;
  * codes are computed against that stored fp16 scale, rounded half to even,
    and clamped to [-127, 127];
  * a group whose scale is 0 has all-zero codes;
  * the softmax scale is a parameter (1/sqrt(head_dim) in the workloads);
  * query head h uses kv head h // (n_q_heads / n_kv_heads);
  * with window W > 0 the query at position L-1 sees keys p with
    L - W <= p < L (exactly W keys once L >= W);
  * an empty context (L = 0) yields an all-zero output row;
  * a 4-bit store is the published Q4_0 block format (32 values, one fp16
    scale d = the value of largest magnitude / -8, codes 0..15 with offset 8)
    over the row after the orthonormal Walsh-Hadamard rotation H / 16, the
    rotation evaluated in float32 butterflies so that codes are decided in
    float32 on both sides.
The GQA mapping, the softmax scale and the window inequality are not fixed by
the pages (parity unpinned against the pages; pinned only against this
module's stated definition by brute force).
"""
from __future__ import annotations

import numpy as np

CODE_MAX = 127          # symmetric int8 range used by the codes
SCALE_DIVISOR = 127.0   # scale = group absmax / 127 (Strata PR 2698, "What it does")


# --------------------------------------------------------------------------
# Quantization (a1 of the hot path)
# --------------------------------------------------------------------------

def scale_from_absmax(absmax) -> np.ndarray:
    """FP16 scale of a group from its absolute maximum: the fp16 value nearest
    to absmax / 127 (ties to even).

    Strata pull request 2698, "What it does": a 64-value group shares one FP16
    scale, its absmax / 127. The float64 quotient is rounded once to
    float16 by numpy (round-to-nearest-even)."""
    a = np.asarray(absmax, dtype=np.float64)
    return (a / SCALE_DIVISOR).astype(np.float16)


def quantize_rows(x, group: int):
    """Quantize rows of fp16 values in groups of ``group`` consecutive elements.

    x: float16 [..., d] with d % group == 0.
    Returns (codes int8 [..., d], scales float16 [..., d // group]).

    Per group: a = max |x_i|; s = scale_from_absmax(a); c_i = the integer
    nearest to x_i / s (ties to even) clamped to [-127, 127]; c = 0 where s = 0.
    genie v0.1.0-alpha.12 "Path I series" (#64, per-head conversion and scale
    capture) with group == head_dim; Strata PR 2698 "What it does" with
    group == 64."""
    x = np.asarray(x, dtype=np.float16)
    d = x.shape[-1]
    if d % group:
        raise ValueError("the scale group must divide head_dim")
    xg = x.astype(np.float64).reshape(x.shape[:-1] + (d // group, group))
    a = np.abs(xg).max(axis=-1)
    s16 = scale_from_absmax(a)
    s = s16.astype(np.float64)[..., None]
    safe = np.where(s > 0.0, s, 1.0)
    q = np.where(s > 0.0, xg / safe, 0.0)
    c = np.clip(np.rint(q), -CODE_MAX, CODE_MAX).astype(np.int8)
    return c.reshape(x.shape), s16


def dequantize_rows(codes, scales, group: int) -> np.ndarray:
    """x_hat = code * scale in float64 (exact: an 8-bit integer times an fp16).

    genie v0.1.0-alpha.12 "Path I series" (#65): attention dequantizes each
    position with the scale stored for that position and kv head."""
    c = np.asarray(codes).astype(np.float64)
    d = c.shape[-1]
    cg = c.reshape(c.shape[:-1] + (d // group, group))
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)[..., None]
    return (cg * s).reshape(c.shape)


# --------------------------------------------------------------------------
# 4-bit stores (Q4_0 blocks after a 256-point Hadamard rotation)
# --------------------------------------------------------------------------
# Strata PR 2698, "Not in this PR": --kv q4_0 and k8v4 use a Hadamard rotation
# over head_dim 256 (FWHT-256) with Q4_0 blocks; keys are rotated (and the
# queries with them), values are rotated and the output is rotated back. The
# pages name the pieces but do not spell them out; this oracle takes the
# published definitions of the Q4_0 block and of the Walsh-Hadamard transform.

Q4_BLOCK = 32
ROT_DIM = 256


def hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix: H[i, j] = (-1)^popcount(i & j), float64."""
    i = np.arange(n)
    bits = np.bitwise_and.outer(i, i)
    par = np.zeros_like(bits)
    while bits.any():
        par ^= bits & 1
        bits >>= 1
    return np.where(par == 1, -1.0, 1.0)


def rotate_exact(x) -> np.ndarray:
    """Orthonormal rotation y = H x / 16 over the last axis (256), in float64.
    H / 16 is symmetric and its own inverse."""
    x = np.asarray(x, dtype=np.float64)
    return x @ hadamard(ROT_DIM) / 16.0


def rotate_f32(x) -> np.ndarray:
    """The same rotation as the quantizer computes it: float32 butterflies
    (a, b) -> (a + b, a - b) at strides 1, 2, 4, ..., 128, then * (1/16)
    (exact). Both the oracle and the kernel decide Q4_0 codes from these
    float32 values."""
    y = np.asarray(x, dtype=np.float16).astype(np.float32)
    shape = y.shape
    y = y.reshape(-1, ROT_DIM)
    h = 1
    while h < ROT_DIM:
        v = y.reshape(y.shape[0], ROT_DIM // (2 * h), 2, h)
        a, b = v[:, :, 0, :], v[:, :, 1, :]
        y = np.stack([a + b, a - b], axis=2).reshape(-1, ROT_DIM)
        h *= 2
    return (y * np.float32(1.0 / 16.0)).reshape(shape)


def quantize_q4_0(y):
    """Q4_0 blocks of 32 float32 values (the published block format): m = the
    value of largest magnitude (the first one on ties), d = m / -8 in float32,
    stored as fp16 (round to nearest even); codes q = min(15, trunc(x * (1/d) +
    8.5)) with 1/d, the product and the sum in float32 (1/d = 0 when d = 0, so a
    zero block has codes 8); value = (q - 8) * d_fp16.

    y: float32 [..., n] (n % 32 == 0). Returns (codes uint8 [..., n] in 0..15,
    scales float16 [..., n // 32])."""
    y = np.asarray(y, dtype=np.float32)
    n = y.shape[-1]
    yb = y.reshape(y.shape[:-1] + (n // Q4_BLOCK, Q4_BLOCK))
    idx = np.argmax(np.abs(yb), axis=-1)  # first index of the largest magnitude
    m = np.take_along_axis(yb, idx[..., None], axis=-1)[..., 0]
    d = (m / np.float32(-8.0)).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(d != 0, np.float32(1.0) / d, np.float32(0.0)).astype(np.float32)
    x0 = (yb * inv[..., None]).astype(np.float32)
    t = (x0 + np.float32(8.5)).astype(np.float32)
    q = np.minimum(15, np.trunc(t).astype(np.int32)).astype(np.uint8)
    return q.reshape(y.shape), d.astype(np.float16)


def dequantize_q4_0(codes, scales) -> np.ndarray:
    """(q - 8) * d in float64 (exact)."""
    c = np.asarray(codes).astype(np.float64) - 8.0
    n = c.shape[-1]
    cb = c.reshape(c.shape[:-1] + (n // Q4_BLOCK, Q4_BLOCK))
    return (cb * np.asarray(scales, dtype=np.float16).astype(np.float64)[..., None]).reshape(c.shape)


def pack_q4(codes) -> np.ndarray:
    """Bytes of Q4_0 blocks: in each block of 32, byte j (j < 16) holds value j
    in its low nibble and value j + 16 in its high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    n = c.shape[-1]
    cb = c.reshape(c.shape[:-1] + (n // Q4_BLOCK, 2, Q4_BLOCK // 2))
    return (cb[..., 0, :] | (cb[..., 1, :] << 4)).reshape(c.shape[:-1] + (n // 2,)).astype(np.uint8)


def unpack_q4(packed) -> np.ndarray:
    """Codes (uint8, 0..15) of Q4_0 bytes laid out as pack_q4 writes them."""
    p = np.asarray(packed, dtype=np.uint8)
    n = p.shape[-1] * 2
    pb = p.reshape(p.shape[:-1] + (n // Q4_BLOCK, Q4_BLOCK // 2))
    return np.concatenate([pb & 0x0F, pb >> 4], axis=-1).reshape(p.shape[:-1] + (n,)).astype(np.uint8)


class Cache:
    """Logical KV cache of one layer: per store either int8 codes + fp16 scales
    or fp32 values, indexed [seq][position][kv head][element] (positions
    major, as the genie pool indexes its scales by position * n_kv_heads +
    kv head, "Path I series" #65).

    Strata PR 2698 "What it does": k8v8 quantizes both stores, k8v32 only K,
    k32v8 only V; an fp32 store keeps the values themselves."""

    def __init__(self, batch, max_ctx, n_kv_heads, head_dim, group,
                 k_dtype="int8", v_dtype="int8"):
        self.batch, self.max_ctx = batch, max_ctx
        self.n_kv_heads, self.head_dim, self.group = n_kv_heads, head_dim, group
        self.dtypes = {"k": k_dtype, "v": v_dtype}
        self.data, self.scales = {}, {}
        for s in ("k", "v"):
            shape = (batch, max_ctx, n_kv_heads, head_dim)
            if self.dtypes[s] == "int8":
                self.data[s] = np.zeros(shape, dtype=np.int8)
                self.scales[s] = np.zeros(shape[:-1] + (head_dim // group,), dtype=np.float16)
            elif self.dtypes[s] == "fp32":
                self.data[s] = np.zeros(shape, dtype=np.float32)
                self.scales[s] = None
            elif self.dtypes[s] == "q4":
                if head_dim != ROT_DIM:
                    raise ValueError("4-bit stores rotate over head_dim 256")
                self.data[s] = np.zeros(shape, dtype=np.uint8)  # codes 0..15, unpacked
                self.scales[s] = np.zeros(shape[:-1] + (head_dim // Q4_BLOCK,), dtype=np.float16)
            else:
                raise ValueError(self.dtypes[s])

    def append(self, k_new, v_new, start_pos):
        """Quantize-append: rows k_new/v_new float16 [batch][n_tok][n_kv][d]
        land at positions start_pos[b] .. start_pos[b] + n_tok - 1.

        int8 stores get codes + scales from quantize_rows; fp32 stores get the
        fp16 values widened exactly (Strata PR 2698: k8v32 / k32v8 leave one
        of the two stores unquantized)."""
        n_tok = k_new.shape[1]
        for s, new in (("k", k_new), ("v", v_new)):
            new = np.asarray(new, dtype=np.float16)
            for b in range(self.batch):
                p0 = int(start_pos[b])
                if self.dtypes[s] == "int8":
                    c, sc = quantize_rows(new[b], self.group)
                    self.data[s][b, p0:p0 + n_tok] = c
                    self.scales[s][b, p0:p0 + n_tok] = sc
                elif self.dtypes[s] == "q4":
                    c, sc = quantize_q4_0(rotate_f32(new[b]))
                    self.data[s][b, p0:p0 + n_tok] = c
                    self.scales[s][b, p0:p0 + n_tok] = sc
                else:
                    self.data[s][b, p0:p0 + n_tok] = new[b].astype(np.float32)

    def values(self, s, b, lo, hi, h):
        """float64 [hi-lo][d]: dequantized (or widened) rows of store s; rows of a
        4-bit store stay in the rotated basis (see rotated())."""
        if self.dtypes[s] == "int8":
            return dequantize_rows(self.data[s][b, lo:hi, h], self.scales[s][b, lo:hi, h], self.group)
        if self.dtypes[s] == "q4":
            return dequantize_q4_0(self.data[s][b, lo:hi, h], self.scales[s][b, lo:hi, h])
        return self.data[s][b, lo:hi, h].astype(np.float64)

    def rotated(self, s) -> bool:
        """A 4-bit store holds rotated rows: a rotated K store needs rotated
        queries, a rotated V store a rotated-back output."""
        return self.dtypes[s] == "q4"


# --------------------------------------------------------------------------
# Decode attention (a3 + a4 of the hot path)
# --------------------------------------------------------------------------

def attended_range(L: int, window: int):
    """Positions [lo, L) that the query at position L-1 attends to.
    genie releases v1.3.0 "Details" (sliding-window mask) and v1.1.0 (512-token
    sliding window); the inequality L - W <= p is this oracle's reading."""
    lo = max(0, L - window) if window > 0 else 0
    return lo, L


def attend_one(q, K, V, sm_scale: float) -> np.ndarray:
    """Softmax attention of query rows q [G][d] over keys K [n][d] and values
    V [n][d], all float64: out = softmax(sm_scale * q K^T) V, two-pass
    (max, then exp and sum)."""
    z = sm_scale * (np.asarray(q, np.float64) @ K.T)
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e @ V) / e.sum(axis=1, keepdims=True)


def attend(q, cache: Cache, seq_lens, window: int, sm_scale: float, heads=None) -> np.ndarray:
    """Decode attention of q float16 [batch][n_q][d] over the cache.

    Query head h reads kv head h // G with G = n_q / n_kv (GQA, this oracle's
    reading). Returns float64 [batch][n_q][d]; rows with an empty range are 0.
    ``heads`` optionally restricts the work to a list of (b, h_q) pairs (the
    other rows are left at 0)."""
    q = np.asarray(q, dtype=np.float16)
    B, Hq, d = q.shape
    Hkv = cache.n_kv_heads
    G = Hq // Hkv
    out = np.zeros((B, Hq, d), dtype=np.float64)
    want = None if heads is None else set((int(b), int(h)) for b, h in heads)
    for b in range(B):
        lo, hi = attended_range(int(seq_lens[b]), window)
        if hi <= lo:
            continue
        for hk in range(Hkv):
            hq = [h for h in range(hk * G, (hk + 1) * G) if want is None or (b, h) in want]
            if not hq:
                continue
            K = cache.values("k", b, lo, hi, hk)
            V = cache.values("v", b, lo, hi, hk)
            qq = q[b, hq].astype(np.float64)
            if cache.rotated("k"):
                qq = rotate_exact(qq)
            o = attend_one(qq, K, V, sm_scale)
            out[b, hq] = rotate_exact(o) if cache.rotated("v") else o
    return out


# --------------------------------------------------------------------------
# Chunk attention: several consecutive query tokens per sequence
# --------------------------------------------------------------------------

def attend_chunk(q, cache: Cache, start_pos, window: int, sm_scale: float, tokens=None) -> np.ndarray:
    """Attention of a chunk of n_tok consecutive query tokens per sequence over
    the cache: q float16 [batch][n_tok][n_q][d]; token t of sequence b sits at
    position P = start_pos[b] + t, its own K/V row already in the cache, and
    attends to the keys p with lo <= p <= P, lo = max(0, P + 1 - window) when
    window > 0 (causal inside the chunk; the decode reading applied to each
    token as if it were the last of a context of P + 1 positions).

    Strata PR 2698, "What it does": the prompt chunk and the verify windows
    read the same int8 cache, dequantized on the fly; genie-ai-runtime release
    v0.1.0-alpha.11, "--int8-kv triage": the batched prefill attention must read
    the scales as decode does. Query head h reads kv head h // G (G = n_q /
    n_kv). Returns float64 [batch][n_tok][n_q][d]. ``tokens`` optionally
    restricts the work to a list of (b, t) pairs (the other rows stay 0)."""
    q = np.asarray(q, dtype=np.float16)
    B, T, Hq, d = q.shape
    Hkv = cache.n_kv_heads
    G = Hq // Hkv
    out = np.zeros((B, T, Hq, d), dtype=np.float64)
    want = None if tokens is None else set((int(b), int(t)) for b, t in tokens)
    for b in range(B):
        for t in range(T):
            if want is not None and (b, t) not in want:
                continue
            P = int(start_pos[b]) + t
            lo = max(0, P + 1 - window) if window > 0 else 0
            for hk in range(Hkv):
                K = cache.values("k", b, lo, P + 1, hk)
                V = cache.values("v", b, lo, P + 1, hk)
                qq = q[b, t, hk * G:(hk + 1) * G].astype(np.float64)
                if cache.rotated("k"):
                    qq = rotate_exact(qq)
                z = sm_scale * (qq @ K.T)
                e = np.exp(z - z.max(axis=1, keepdims=True))
                o = (e @ V) / e.sum(axis=1, keepdims=True)
                out[b, t, hk * G:(hk + 1) * G] = rotate_exact(o) if cache.rotated("v") else o
    return out


def split_partials(q, K, V, sm_scale: float, bounds):
    """Online-softmax partials of one (query group, kv head) over the position
    ranges [bounds[i], bounds[i+1]) -- genie releases v1.3.0: each split block
    forms an online-softmax partial.

    Returns m [S][G] (max score), l [S][G] (sum of exp(z - m)), O [S][G][d]
    (sum of exp(z - m) * v); an empty split has m = -inf, l = 0, O = 0."""
    q = np.asarray(q, np.float64)
    G, d = q.shape
    S = len(bounds) - 1
    m = np.full((S, G), -np.inf)
    l = np.zeros((S, G))
    O = np.zeros((S, G, d))
    for s in range(S):
        a, b = bounds[s], bounds[s + 1]
        if b <= a:
            continue
        z = sm_scale * (q @ K[a:b].T)
        m[s] = z.max(axis=1)
        e = np.exp(z - m[s][:, None])
        l[s] = e.sum(axis=1)
        O[s] = e @ V[a:b]
    return m, l, O


def combine_partials(m, l, O) -> np.ndarray:
    """Reduce of the split partials (genie releases v1.3.0, "split-K decode
    attention": the per-split partials of each head merged in a second pass):
    M = max_s m_s, w_s = exp(m_s - M), out = sum_s w_s O_s / sum_s w_s l_s.
    Empty splits weigh 0; all-empty -> 0."""
    M = m.max(axis=0)
    out = np.zeros(O.shape[1:])
    ok = np.isfinite(M)
    if not ok.any():
        return out
    w = np.where(np.isfinite(m), np.exp(m - np.where(ok, M, 0.0)[None, :]), 0.0)
    num = np.einsum("sg,sgd->gd", w, O)
    den = (w * l).sum(axis=0)
    out[ok] = num[ok] / den[ok][:, None]
    return out


# --------------------------------------------------------------------------
# Cache sizes (the pages' worked byte counts)
# --------------------------------------------------------------------------

_DTYPE_BYTES = {"int8": 1, "fp16": 2, "fp32": 4}


def cell_bytes(n_kv_heads: int, head_dim: int, group: int, dtype: str,
               scale_bytes: int = 2) -> int:
    """Bytes one store spends on one position of one layer (all kv heads):
    values plus, for int8, one scale per group. Strata PR 2698 "What it does"
    counts 528 B per cell for int8 + FP16 group-64 scales against 2048 B for
    FP32 at head_dim 256."""
    if dtype == "q4":  # two codes per byte and one fp16 scale per 32 values
        return n_kv_heads * (head_dim // 2 + (head_dim // Q4_BLOCK) * 2)
    b = n_kv_heads * head_dim * _DTYPE_BYTES[dtype]
    if dtype == "int8":
        b += n_kv_heads * (head_dim // group) * scale_bytes
    return b


def pool_bytes(n_layers: int, ctx: int, n_kv_heads: int, head_dim: int, dtype: str,
               scale_bytes: int = 2):
    """(body, scales) bytes of a K+V pool with one scale per (layer, position,
    kv head) when dtype is int8 -- genie v0.1.0-alpha.12 "Headline result"
    (KV pool memory) and "Path I series" #63 (separate scales region)."""
    body = 2 * n_layers * ctx * n_kv_heads * head_dim * _DTYPE_BYTES[dtype]
    scales = 2 * n_layers * ctx * n_kv_heads * scale_bytes if dtype == "int8" else 0
    return body, scales


# --------------------------------------------------------------------------
# Cache blob: codes with their scales and the layout facts they need
# --------------------------------------------------------------------------

BLOB_MAGIC = 0x3151564B   # "KVQ1" read as a little-endian uint32
BLOB_VERSION = 1


def blob_payload(cache: Cache, b: int, pos0: int, n_pos: int) -> bytes:
    """Payload of the cache blob of positions [pos0, pos0 + n_pos) of
    sequence b: K values, V values, then for each int8 or q4 store its fp16
    scales, every region positions-major ([position][kv head][...]) and padded
    to a multiple of 16 bytes. A q4 store's values are its Q4_0 bytes (two
    codes per byte, pack_q4) and its scales the 8 block scales of each row.

    genie-ai-runtime release v0.1.0-alpha.11, "--int8-kv triage": a saved
    cache must carry the scales region too; release v0.1.0-alpha.12, "Path F
    (#45) interop guard": int8 bytes saved without their per-head scales give
    garbage when read back. The blob therefore always holds, for an int8
    store, the scales next to the codes."""
    def pad(x: bytes) -> bytes:
        return x + b"\0" * (-len(x) % 16)
    parts = []
    for s in ("k", "v"):
        vals = cache.data[s][b, pos0:pos0 + n_pos]
        if cache.dtypes[s] == "q4":
            vals = pack_q4(vals)
        parts.append(pad(np.ascontiguousarray(vals).tobytes()))
    for s in ("k", "v"):
        if cache.scales[s] is not None:
            parts.append(pad(np.ascontiguousarray(cache.scales[s][b, pos0:pos0 + n_pos]).tobytes()))
    return b"".join(parts)


def blob_header(cache: Cache, n_pos: int) -> dict:
    """The facts a reader must match before it may place the payload: format
    magic and version, kv heads, head_dim, both store types, scale group and
    the number of positions, plus the payload size."""
    dt = {"int8": 1, "fp32": 2, "q4": 3}
    return {"magic": BLOB_MAGIC, "version": BLOB_VERSION, "n_kv_heads": cache.n_kv_heads,
            "head_dim": cache.head_dim, "k_dtype": dt[cache.dtypes["k"]], "v_dtype": dt[cache.dtypes["v"]],
            "scale_group": cache.group, "n_pos": n_pos}


def blob_restore(cache: Cache, header: dict, payload: bytes, b: int, pos0: int) -> None:
    """Place a blob's payload at positions [pos0, pos0 + n_pos) of sequence b,
    refusing (ValueError) a blob whose layout facts differ from the cache's."""
    want = blob_header(cache, header["n_pos"])
    for k, v in want.items():
        if header.get(k) != v:
            raise ValueError(f"blob {k} {header.get(k)} does not match the cache ({v})")
    n = header["n_pos"]
    off = 0
    for s in ("k", "v"):
        arr = cache.data[s][b, pos0:pos0 + n]
        if cache.dtypes[s] == "q4":
            nb = arr.size // 2
            packed = np.frombuffer(payload[off:off + nb], dtype=np.uint8).reshape(arr.shape[:-1] + (arr.shape[-1] // 2,))
            cache.data[s][b, pos0:pos0 + n] = unpack_q4(packed)
        else:
            nb = arr.nbytes
            cache.data[s][b, pos0:pos0 + n] = np.frombuffer(payload[off:off + nb], dtype=arr.dtype).reshape(arr.shape)
        off += nb + (-nb % 16)
    for s in ("k", "v"):
        if cache.scales[s] is not None:
            arr = cache.scales[s][b, pos0:pos0 + n]
            nb = arr.nbytes
            cache.scales[s][b, pos0:pos0 + n] = np.frombuffer(payload[off:off + nb], dtype=np.float16).reshape(arr.shape)
            off += nb + (-nb % 16)
    if off != len(payload):
        raise ValueError("blob payload size does not match its header")
