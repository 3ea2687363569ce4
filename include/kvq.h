/*
 * kvq.h -- C ABI of the INT8 KV-cache decode path for AMD Instinct MI355X (gfx950).
 *
 * The library implements one decode step of attention over a KV cache whose
 * K and V stores hold int8 codes with FP16 scales (or, per store, fp32 values):
 *
 *   kv_quant_append        quantize new K/V rows and write them into the cache
 *   kv_decode_attn_splitk  split-K partial attention of one query token per
 *                          sequence (online-softmax partials per split)
 *   kv_append_decode_splitk  the decode step's one-token quantize-append fused
 *                          into kv_decode_attn_splitk
 *   kv_decode_reduce       combine the split partials into the fp16 output
 *   kv_decode_attn         append + partials + combine in one call (one launch
 *                          for small int8 plans)
 *   kv_decode_attn_static  partials + combine in one call, with the partials
 *                          in the library's static device scratch (no
 *                          workspace, no allocation)
 *   kv_chunk_attn          attention of a chunk of consecutive query tokens per
 *                          sequence (prompt chunk, verify window): causal
 *                          inside the chunk, partials + combine in one call
 *   kv_cache_pack / kv_cache_unpack  a sequence's cache positions as one
 *                          contiguous blob (codes with their scales) and back
 *   kvq_plan               host-only choice of the split count and workspace
 *   kvq_plan_chunk         the same for kv_chunk_attn
 *   kvq_stream_read        a read-only streaming reference for measurements
 *
 * Sources of the method (web pages; cited by title and section):
 *   [G12]  genie-ai-runtime release v0.1.0-alpha.12, "Path I: INT8 KV cache",
 *          table "Path I series": a separate scales region in the KV pool (#63),
 *          per-head conversion with scale capture (#64), attention dequantizes
 *          each position with its (position, kv head) scale (#65).
 *   [G11]  genie-ai-runtime release v0.1.0-alpha.11, "--int8-kv triage": a null
 *          scale pointer silently became scale 1.0; the conversion ran with one
 *          row instead of one per kv head.
 *   [G130] genie-ai-runtime releases, v1.3.0 "split-K decode attention" and its
 *          "Details": the KV range of each head is split over blocks, each block
 *          forms an online-softmax partial and a second kernel merges them; the
 *          split count is fixed on the host while positions come from the
 *          device; sliding-window mask and slot width are honoured.
 *   [G121] genie-ai-runtime releases, v1.2.1 "Bugs fixed": head_dim 256 stored
 *          in a 512-wide cache slot; strides must come from the slot width.
 *   [S2698] Strata pull request 2698 (int8 K/V cache), "What it does": int8
 *          codes, each 64-value group sharing an FP16 scale (its absmax /
 *          127); the host refuses a head_dim not divisible by 64; k8v32 and
 *          k32v8 leave one store unquantized, attended as fp32.
 *          "Not in this PR": 4-bit stores (q4_0 for K and V, k8v4 for V only)
 *          use a Hadamard rotation over head_dim 256 with Q4_0 blocks; K is
 *          rotated after RoPE together with the queries, V is rotated and the
 *          output rotated back.
 *
 * Conventions for every entry point:
 *   - All tensors are caller-owned device memory unless stated; the library
 *     allocates nothing, keeps no state between calls and never synchronizes.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it and the call returns at once.
 *   - Arguments are validated first; on any error a negative kvq_status is
 *     returned and nothing is enqueued. A launch failure returns KVQ_ERR_HIP.
 *   - fp16 data is passed as uint16_t bit patterns (IEEE binary16).
 *   - Device-side preconditions that cannot be checked without a sync are
 *     listed per call; violating them never makes a kernel read or write
 *     outside the buffers described by the layout.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_NULL = -1,        /* a required pointer is NULL (scales of an int8 store included, [G11]) */
  KVQ_ERR_SHAPE = -2,       /* inconsistent sizes or strides */
  KVQ_ERR_UNSUPPORTED = -3, /* a valid request this library does not implement (e.g. head_dim 96) */
  KVQ_ERR_ALIGN = -4,       /* a pointer or stride breaks the alignment the loads need */
  KVQ_ERR_WORKSPACE = -5,   /* workspace missing or smaller than kvq_plan_t.ws_bytes */
  KVQ_ERR_HIP = -6,         /* the HIP runtime reported an error at launch */
  KVQ_ERR_MISMATCH = -7,    /* a cache blob whose layout facts differ from the target cache's */
  KVQ_ERR_SCRATCH = -8      /* the partials exceed the static scratch of kv_decode_attn_static */
} kvq_status;

/* Store element types ([S2698]: fp32 = the unquantized store; q4 = the 4-bit
 * store of [S2698 "Not in this PR"]).
 * KVQ_STORE_Q4 holds each row rotated, y = H x / 16 with H the 256 x 256
 * Sylvester Hadamard matrix (H[i][j] = (-1)^popcount(i & j); H / 16 is
 * orthonormal and its own inverse), as Q4_0 blocks: per 32 values one fp16
 * scale d and 32 4-bit codes q (value (q - 8) * d), byte j of a block's 16
 * bytes holding value j in its low nibble and value j + 16 in its high one.
 * Requires head_dim 256. */
enum { KVQ_STORE_INT8 = 1, KVQ_STORE_FP32 = 2, KVQ_STORE_Q4 = 3 };

/* Layout of one layer's KV cache.
 *
 * Each store (K and V) is an array of rows; the row of (sequence b, position p,
 * kv head h) starts at element  b*s_seq + p*s_pos + h*s_head  and holds
 * head_dim contiguous elements (int8 codes, fp32 values, or 4-bit codes: a q4
 * element is half a byte, so element e sits at byte e / 2). A row may sit in
 * a wider slot (slot_dim >= head_dim, [G121]); elements [head_dim, slot_dim)
 * are never read or written. K and V use the same element strides.
 *
 * Each int8 store has an fp16 scale array: the scales of row (b, p, h) start at
 * element  b*ss_seq + p*ss_pos + h*ss_head  and are head_dim/scale_group
 * consecutive values, scale j covering elements [j*g, (j+1)*g) of the row.
 * scale_group == head_dim gives one scale per (position, kv head) [G12 #64];
 * scale_group == 64 gives one scale per 64 values [S2698]. A q4 store has
 * head_dim / 32 scales per row, one per Q4_0 block (scale_group applies to
 * int8 stores only). Both scale arrays use the same strides, which must leave
 * room for the larger of the two stores' scale rows. An fp32 store has no
 * scales.
 *
 * Supported: head_dim in {64, 128, 256}; scale_group in {64, head_dim}; every
 * combination of k_dtype/v_dtype in {KVQ_STORE_INT8, KVQ_STORE_FP32}
 * (k8v8, k8v32, k32v8, k32v32); at head_dim 256 also q4 K and V (q4_0) and
 * int8 K with q4 V (k8v4) -- the other combinations with a q4 store are
 * refused (KVQ_ERR_UNSUPPORTED). Row offsets in bytes must be multiples of 16;
 * scale-row offsets in bytes multiples of 2 * (scales per row) of each store
 * that has scales; the byte extent of one sequence (max_ctx positions) must
 * stay below 2^31.
 */
typedef struct {
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t slot_dim;
  int32_t k_dtype;
  int32_t v_dtype;
  int32_t scale_group;
  int64_t max_ctx;              /* positions allocated per sequence */
  int64_t s_seq, s_pos, s_head; /* element strides of the stores */
  int64_t ss_seq, ss_pos, ss_head; /* element strides of the fp16 scale arrays */
} kvq_layout;

/* Split plan of one decode step ([G130]: split count fixed on the host).
 * The attended range [lo, L) of a sequence with context L (lo = max(0, L -
 * window) if window > 0, else 0) is cut into blocks of 128 positions from lo;
 * with S = min(n_splits, ceil((L - lo) / chunk)) (the splits that contiguous
 * ranges of chunk positions would use), decode split s < S covers blocks
 * s, s + S, s + 2*S, ... (block-cyclic) and splits s >= S are empty, so every
 * context length is covered whatever the planned one. kv_chunk_attn splits
 * the keys of a kv head's query rows the same way (from the lo of its first
 * token to the position of its last) when it runs a chunk of at most 32
 * (token, head) rows per kv head (16 with an fp32 store), otherwise
 * contiguously: [lo + s*chunk,
 * lo + (s+1)*chunk), the last split running to the chunk's end. Either way
 * every key is covered whatever the plan. ws_bytes is the workspace that
 * kv_decode_attn_splitk (or kv_chunk_attn) writes and kv_decode_reduce reads. */
typedef struct {
  int32_t n_splits;
  int32_t chunk;       /* positions per split, a multiple of 32 */
  int64_t ws_bytes;
} kvq_plan_t;

/* kvq_plan -- host only, no device call.
 * Chooses n_splits/chunk for `batch` sequences of at most `max_seq_len`
 * positions (window > 0 limits the attended range to `window` keys) on a device
 * with `n_cu` compute units, so that the partial kernel's grid covers the chip
 * while the partial workspace stays a small fraction of the KV bytes read.
 * Fewer than 64 attended positions always get a single split ([G130] keeps a
 * single-block kernel below 64 tokens). Writes *out; returns KVQ_OK or an error
 * for invalid layout/sizes. */
int kvq_plan(const kvq_layout* layout, int32_t batch, int32_t n_q_heads,
             int32_t max_seq_len, int32_t window, int32_t n_cu, kvq_plan_t* out);

/* kv_quant_append -- quantize n_tok new K and V rows per sequence into the cache.
 * [G12 #64], [S2698 "What it does"].
 *   k_new, v_new  fp16 [batch][n_tok][n_kv_heads][head_dim], contiguous, 16-byte aligned.
 *   d_start_pos   device int32 [batch]: row t of sequence b lands at position
 *                 d_start_pos[b] + t.
 *   k_store/v_store, k_scales/v_scales  as described by `layout`; scales must be
 *                 non-NULL for an int8 store and are ignored for an fp32 store.
 * Per group of scale_group values x of a row: a = max|x|; the fp16 scale is the
 * round-to-nearest-even fp16 value of a/127 (fp32 division, correctly rounded);
 * code = clamp(round-half-even(x / scale), -127, 127), 0 when the scale is 0.
 * An fp32 store receives the fp16 values widened exactly.
 * A q4 store ([S2698 "Not in this PR"]) receives the rotated row as Q4_0
 * blocks: the rotation is evaluated in fp32 as butterflies (a, b) -> (a + b,
 * a - b) over index pairs at distance 1, 2, 4, ..., 128 in that order, then
 * multiplied by 1/16; per block of 32 rotated values y, m is the value of
 * largest magnitude (the first one on ties), d = m / -8 (fp32), stored as its
 * round-to-nearest-even fp16 value, and q = min(15, trunc(y * r + 8.5)) with
 * r = 1/d (0 when d = 0), the reciprocal, product and sum each rounded to fp32
 * (no fused multiply-add), as the published Q4_0 quantizer does.
 * Device precondition: 0 <= d_start_pos[b] and d_start_pos[b] + n_tok <= max_ctx;
 * rows that would land outside [0, max_ctx) are not written. */
int kv_quant_append(const kvq_layout* layout, void* k_store, void* v_store,
                    uint16_t* k_scales, uint16_t* v_scales,
                    const uint16_t* k_new, const uint16_t* v_new,
                    const int32_t* d_start_pos, int32_t batch, int32_t n_tok,
                    void* stream);

/* kv_decode_attn_splitk -- split-K partials of single-token decode attention.
 * [G130 "split-K decode attention"], [G12 #65], [S2698].
 *   q           fp16 [batch][n_q_heads][head_dim], contiguous, 16-byte aligned.
 *               Query head hq reads kv head hq / (n_q_heads / n_kv_heads).
 *   d_seq_lens  device int32 [batch]: context length L_b (positions 0..L_b-1 are
 *               in the cache, the query token's own K/V included).
 *   window      0 = attend to all L_b positions; > 0 = only the last `window`.
 *   sm_scale    softmax scale applied to q.k (e.g. 1/sqrt(head_dim)).
 *   plan        from kvq_plan for at least this batch, n_q_heads and window.
 *   ws          device workspace of at least plan->ws_bytes bytes, 16-byte aligned;
 *               written here, read by kv_decode_reduce on the same stream. Every
 *               split records its (max, sum) pair, a split with no position in
 *               the attended range as (-inf, 0); its output row is then left
 *               unwritten. No initialization of ws is needed.
 * Device precondition: 0 <= d_seq_lens[b] <= max_ctx (larger values are clamped
 * to max_ctx). Keys are dequantized as code * scale; the fp32 store is read as
 * the fp16 values kv_quant_append widened into it. With a q4 K store the query
 * is rotated the same way (H q / 16, rounded to fp16) before q.k; with a q4 V
 * store each split's partial output is rotated back (H o / 16, fp32), so the
 * reduced output is in the original basis ([S2698 "Not in this PR"]). */
int kv_decode_attn_splitk(const kvq_layout* layout,
                          const void* k_store, const void* v_store,
                          const uint16_t* k_scales, const uint16_t* v_scales,
                          const uint16_t* q, int32_t batch, int32_t n_q_heads,
                          const int32_t* d_seq_lens, int32_t window, float sm_scale,
                          const kvq_plan_t* plan, void* ws, int64_t ws_bytes,
                          void* stream);

/* kv_append_decode_splitk -- one decode step's quantize-append fused into the
 * split-K partials. [G12 #64, #65], [G130], [S2698 "What it does"].
 * For each sequence b with 1 <= L_b = d_seq_lens[b] <= max_ctx, the new token's
 * K and V rows of every kv head are quantized exactly as kv_quant_append does
 * (d_start_pos[b] = L_b - 1, n_tok = 1) and written to row L_b - 1 of the
 * stores and scales; the partials are those of kv_decode_attn_splitk over
 * [lo, L_b) with that row in place. The workgroup whose blocks hold position
 * L_b - 1 takes the new row from its own quantizer, so within the call nothing
 * reads that row from memory. A sequence with L_b = 0 or L_b > max_ctx gets
 * no append (as kv_quant_append drops such rows) and the partials of
 * kv_decode_attn_splitk.
 *   k_new, v_new  fp16 [batch][n_kv_heads][head_dim] (one token per sequence),
 *                 contiguous, 16-byte aligned.
 *   other arguments as for kv_decode_attn_splitk; the stores and scales are
 *   written, so they are not const here. Combine with kv_decode_reduce.
 * Codes and scales are bit-identical to kv_quant_append's; the output of the
 * reduce differs from the unfused pair only in the order in which the new
 * position's term is summed. Layouts with a q4 store: q4_0 and k8v4 as in
 * kv_decode_attn_splitk (the new row rotated and quantized exactly as
 * kv_quant_append does); the other combinations are refused
 * (KVQ_ERR_UNSUPPORTED). */
int kv_append_decode_splitk(const kvq_layout* layout, void* k_store, void* v_store,
                            uint16_t* k_scales, uint16_t* v_scales,
                            const uint16_t* k_new, const uint16_t* v_new,
                            const uint16_t* q, int32_t batch, int32_t n_q_heads,
                            const int32_t* d_seq_lens, int32_t window, float sm_scale,
                            const kvq_plan_t* plan, void* ws, int64_t ws_bytes,
                            void* stream);

/* kv_decode_reduce -- combine the partials of kv_decode_attn_splitk.
 * [G130 "split-K decode attention": a separate kernel merges the split
 * partials]. For each (b, hq): with split maxima
 * m_s, sums l_s and unnormalized outputs O_s, M = max m_s, w_s = exp(m_s - M),
 * out = sum_s w_s O_s / sum_s w_s l_s, rounded to fp16 (nearest even).
 * Splits recorded as empty add nothing; a sequence with no attended position
 * (L_b = 0) gets an all-zero row.
 *   out  fp16 [batch][n_q_heads][head_dim], contiguous, 16-byte aligned.
 * The other arguments must equal those of the preceding kv_decode_attn_splitk
 * (they are validated; the combine itself reads only ws, so it does not wait
 * on d_seq_lens). */
int kv_decode_reduce(const kvq_layout* layout, const void* ws, int64_t ws_bytes,
                     const int32_t* d_seq_lens, int32_t batch, int32_t n_q_heads,
                     int32_t window, const kvq_plan_t* plan, uint16_t* out,
                     void* stream);

/* kv_decode_attn -- a whole decode step in one call: the new token's
 * quantize-append (when k_new, v_new are given), the split-K partials and
 * their combine into the fp16 output. [G130 "split-K decode attention" and
 * "Details"], [G12 #64, #65], [S2698 "What it does"].
 * The output is what kv_append_decode_splitk (k_new and v_new non-null) or
 * kv_decode_attn_splitk (both null), followed by kv_decode_reduce, computes
 * with the same plan, up to the order of the fp32 sums of the combine; the
 * cache rows appended are bit-identical to theirs.
 * Plans of at most 8 splits over int8 K and V stores run as ONE kernel
 * launch: the query heads of a kv head are taken in units of at most
 * 512 / head_dim of them (16 at most), every workgroup writes its unit's
 * partial through to memory and counts its arrival in d_arrive, and the last
 * workgroup of each unit combines that unit's splits and writes its rows of
 * out (the genie reduce's arithmetic, inside the partial kernel; no
 * workgroup waits for another). Other plans and stores run the partial
 * kernel and the reduce, two launches; kvq_decode_launches tells which.
 *   d_arrive  device uint32 [batch * n_q_heads], 4-byte aligned: zero before
 *             the first call that uses it; every call leaves it zero. Calls
 *             that share it (or ws) must not overlap on the device.
 *   out       fp16 [batch][n_q_heads][head_dim], contiguous, 16-byte aligned.
 *   other arguments as for kv_append_decode_splitk; k_new and v_new are both
 *   null or both non-null (KVQ_ERR_NULL otherwise).
 * Errors as kv_append_decode_splitk / kv_decode_attn_splitk; nothing is
 * enqueued when a check fails. */
int kv_decode_attn(const kvq_layout* layout, void* k_store, void* v_store,
                   uint16_t* k_scales, uint16_t* v_scales,
                   const uint16_t* k_new, const uint16_t* v_new,
                   const uint16_t* q, int32_t batch, int32_t n_q_heads,
                   const int32_t* d_seq_lens, int32_t window, float sm_scale,
                   const kvq_plan_t* plan, void* ws, int64_t ws_bytes,
                   uint32_t* d_arrive, uint16_t* out, void* stream);

/* kvq_decode_launches -- host only, no device call. The number of kernel
 * launches kv_decode_attn makes for these arguments: 1 (the one-launch step),
 * 2 (partials, then the reduce) or 0 (batch 0). Writes *launches; returns
 * KVQ_OK or the error kv_decode_attn would return for the layout, heads and
 * plan. */
int kvq_decode_launches(const kvq_layout* layout, int32_t batch, int32_t n_q_heads,
                        const kvq_plan_t* plan, int32_t* launches);

/* kv_decode_attn_static -- for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): kv_decode_attn_splitk followed by kv_decode_reduce, with the
 * split partials kept in a device array of the library instead of a caller
 * workspace. Nothing is allocated by the call: the array is a fixed part of
 * the library on each device (KVQ_STATIC_SCRATCH_BYTES, held until the
 * process ends); the first call on a device looks up its address there.
 *   Arguments as for kv_decode_attn_splitk (no ws, ws_bytes) and
 *   out  fp16 [batch][n_q_heads][head_dim], contiguous, 16-byte aligned.
 * The output is that of kv_decode_attn_splitk + kv_decode_reduce with the same
 * plan. Returns KVQ_ERR_SCRATCH, with nothing enqueued, when the plan's
 * partials (plan->ws_bytes) exceed KVQ_STATIC_SCRATCH_BYTES; the other errors
 * as kv_decode_attn_splitk. No part of the scratch needs to start at zero.
 * All calls on one device share the array: calls that overlap on a device
 * (two streams, or two host threads, without ordering between them) race and
 * give undefined output. */
#define KVQ_STATIC_SCRATCH_BYTES (16ll << 20) /* 16 MiB per device */
int kv_decode_attn_static(const kvq_layout* layout,
                          const void* k_store, const void* v_store,
                          const uint16_t* k_scales, const uint16_t* v_scales,
                          const uint16_t* q, int32_t batch, int32_t n_q_heads,
                          const int32_t* d_seq_lens, int32_t window, float sm_scale,
                          const kvq_plan_t* plan, uint16_t* out, void* stream);

/* kvq_plan_chunk -- host only, no device call. Split plan of kv_chunk_attn
 * for `batch` sequences of `n_tok` query tokens whose last token sits below
 * position max_seq_len (the largest start + n_tok). Chunks with many query
 * rows run one split per (sequence, kv head, 64-row block); a few tokens over
 * a long prefix (a verify window) get their keys split so that the grid covers
 * the chip. Chunks with at most 32 (token, head) rows per kv head (16 with
 * an fp32 store) run through the decode partial kernels and get kvq_plan's
 * split rule.
 * ws_bytes = batch * n_tok * n_q_heads * n_splits * (head_dim + 2) * 4.
 * Writes *out; returns KVQ_OK or an error for invalid layout/sizes. */
int kvq_plan_chunk(const kvq_layout* layout, int32_t batch, int32_t n_tok, int32_t n_q_heads,
                   int32_t max_seq_len, int32_t window, int32_t n_cu, kvq_plan_t* out);

/* kv_chunk_attn -- attention of a chunk of n_tok consecutive query tokens per
 * sequence over the int8 cache, into `out`. [S2698 "What it does": the prompt
 * chunk and the verify windows read the same int8 cache, dequantized on the
 * fly], [G11 "--int8-kv triage": the batched prefill attention reads the
 * scales as decode does], [G130 "split-K decode attention"].
 * Token t of sequence b sits at position P = d_start_pos[b] + t; its own K and
 * V rows must already be in the cache (kv_quant_append of the chunk first). It
 * attends to the keys lo <= p <= P with lo = max(0, P + 1 - window) when
 * window > 0, else 0 (causal inside the chunk). Keys are dequantized as code *
 * scale, exactly as in kv_decode_attn_splitk; query head hq reads kv head
 * hq / (n_q_heads / n_kv_heads).
 *   q            fp16 [batch][n_tok][n_q_heads][head_dim], contiguous, 16-byte aligned.
 *   d_start_pos  device int32 [batch].
 *   plan         from kvq_plan_chunk for at least this batch, n_tok and n_q_heads.
 *   ws           device workspace of at least plan->ws_bytes bytes, 16-byte
 *                aligned (split partials of rows (b, t, hq); no initialization).
 *   out          fp16 [batch][n_tok][n_q_heads][head_dim], contiguous, 16-byte aligned.
 * Store types: int8 K and V, or the 4-bit layouts q4_0 and k8v4 (the query
 * rotated for a q4 K store and the output rotated back, as in
 * kv_decode_attn_splitk); with an fp32 store (k8v32, k32v8, k32v32) only
 * chunks of at most 16 (token, head) rows per kv head (verify windows);
 * other combinations and longer chunks over fp32 stores are refused
 * (KVQ_ERR_UNSUPPORTED). Two kernels are enqueued on `stream`: the partials
 * and the combine of kv_decode_reduce. The partials of a chunk with at most
 * 32 (token, head) rows per kv head (16 with an fp32 store) come from the
 * decode partial kernels,
 * whose query rows are then (token, head) pairs with their own causal limits
 * (a verify window reads every key once, or once per 16 rows over a 4-bit
 * layout); larger chunks from the chunk kernels.
 * Device precondition: 0 <= d_start_pos[b] and d_start_pos[b] + n_tok <= max_ctx;
 * a token that would sit at or beyond max_ctx sees no key and gets a zero row. */
int kv_chunk_attn(const kvq_layout* layout, const void* k_store, const void* v_store,
                  const uint16_t* k_scales, const uint16_t* v_scales,
                  const uint16_t* q, int32_t batch, int32_t n_tok, int32_t n_q_heads,
                  const int32_t* d_start_pos, int32_t window, float sm_scale,
                  const kvq_plan_t* plan, void* ws, int64_t ws_bytes, uint16_t* out,
                  void* stream);

/* Cache blob: positions [pos0, pos0 + n_pos) of one sequence as one
 * contiguous payload that carries, for every int8 store, the fp16 scales next
 * to the codes ([G11 "--int8-kv triage": saving a cache means saving its scale
 * region as well], [G12 "Path F (#45) interop guard": int8 bytes saved without
 * their per-head scales read back as garbage]).
 * Payload (device memory): K values, V values, then the K scales and the V
 * scales of int8 and q4 stores; each region positions-major ([position]
 * [kv head][the row's bytes: head_dim codes, fp32 values, or head_dim / 2
 * Q4_0 bytes] or [the row's scales: head_dim / scale_group, or head_dim / 32
 * for q4]) and padded to a multiple of 16 bytes. The header (host memory) holds the facts a reader must
 * match; it is independent of the strides, so a blob can be placed into a
 * cache with another layout order. */
#define KVQ_BLOB_MAGIC 0x3151564Bu /* "KVQ1" */
#define KVQ_BLOB_VERSION 1u
typedef struct {
  uint32_t magic;
  uint32_t version;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t k_dtype;
  int32_t v_dtype;
  int32_t scale_group;
  int32_t n_pos;
  int64_t payload_bytes;
} kvq_blob_header;

/* kvq_blob_size -- host only: payload bytes of a blob of n_pos positions. */
int kvq_blob_size(const kvq_layout* layout, int32_t n_pos, int64_t* payload_bytes);

/* kv_cache_pack -- copy positions [pos0, pos0 + n_pos) of sequence `seq` into
 * the payload `dst` (device, 16-byte aligned, at least the payload size) and
 * fill *header. Requires 0 <= pos0, pos0 + n_pos <= max_ctx; `seq` must be a
 * sequence of the stores (not checkable here). Scales must be non-NULL for
 * int8 stores. Enqueued on `stream`; the header is valid on return. */
int kv_cache_pack(const kvq_layout* layout, const void* k_store, const void* v_store,
                  const uint16_t* k_scales, const uint16_t* v_scales, int32_t seq, int32_t pos0,
                  int32_t n_pos, void* dst, int64_t dst_bytes, kvq_blob_header* header, void* stream);

/* kv_cache_unpack -- place a blob at positions [pos0, pos0 + header->n_pos) of
 * sequence `seq`. Returns KVQ_ERR_MISMATCH, with nothing enqueued, when the
 * header's magic, version, kv heads, head_dim, store types, scale group or
 * payload size differ from this layout's (e.g. an int8 blob for an fp32
 * cache); KVQ_ERR_WORKSPACE when src_bytes is smaller than the payload. */
int kv_cache_unpack(const kvq_layout* layout, void* k_store, void* v_store, uint16_t* k_scales,
                    uint16_t* v_scales, int32_t seq, int32_t pos0, const kvq_blob_header* header,
                    const void* src, int64_t src_bytes, void* stream);

/* kvq_stream_read -- measurement reference, not part of the method: reads
 * `bytes` of device memory at `buf` (16-byte aligned, bytes a multiple of 16)
 * once with 128-bit loads and discards them, on `n_cu` compute units' worth of
 * workgroups. Its bytes per second are what a kernel that only streams can
 * take of this GPU's HBM, the reference beside the 8 TB/s peak for the decode
 * kernels' KV bytes per second. `sink` (device, 4 bytes) is written only in
 * the practically impossible case that the XOR of a lane's loads equals a
 * fixed constant. Enqueued on `stream`. */
int kvq_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t n_cu, void* stream);

/* Text for a kvq_status value (static storage). */
const char* kvq_status_string(int status);

/* Library version as (major << 16) | (minor << 8) | patch. */
int kvq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
