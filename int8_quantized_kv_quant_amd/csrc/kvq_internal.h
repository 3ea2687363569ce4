// Internal declarations shared by the host code and the HIP kernels of libkvq.
// Nothing here is part of the C ABI (include/kvq.h is).
#pragma once

#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

constexpr int kTile = 32;            // positions per MFMA tile step of a wave
constexpr int kMaxSplits = 8192;     // bound on plan.n_splits
constexpr int kHeadsPerBlock = 16;   // query heads one wave carries (MFMA M/N = 16)
constexpr int kPartialWaves = 4;     // wavefronts per partial-kernel workgroup
constexpr int kMinSplitChunk = kPartialWaves * kTile;  // planner: one tile per wavefront at least
constexpr int kChunkWaves = 4;       // wavefronts per chunk-attention workgroup
// kv_decode_attn: plans of at most this many splits over int8 K and V run as
// one launch (the last workgroup of a unit combines its splits in registers).
constexpr int kOneLaunchMaxSplits = 8;

// A layout with a 4-bit store.
inline bool has_q4(const kvq_layout& L) { return L.k_dtype == KVQ_STORE_Q4 || L.v_dtype == KVQ_STORE_Q4; }

// (token, head) query rows per chunk-attention workgroup: 16 per wavefront,
// or 32 (two row blocks sharing each key and value operand) for head_dim <= 128
// when the chunk has rows enough; at head_dim 256 two row blocks exceed the
// register file (measured slower).
inline int chunk_rows_per_wg(int64_t n_tok, int64_t G, int head_dim) {
  return (head_dim <= 128 && n_tok * G >= 1024) ? 32 * kChunkWaves : 16 * kChunkWaves;
}

// Row blocks of a chunk of n_tok tokens whose G query heads share a kv head.
inline int chunk_row_blocks(int64_t n_tok, int64_t G, int head_dim) {
  const int64_t r = chunk_rows_per_wg(n_tok, G, head_dim);
  return (int)((n_tok * G + r - 1) / r);
}

// Chunk-attention workgroups that fit on one compute unit at once, from the
// kernel's footprint on gfx950 (three LDS stages and the fp16 value tile per
// workgroup): with one row block per wavefront ~250 VGPRs and 67 KB at D = 256
// (two), ~150 VGPRs and 34 KB at D = 128 (three), ~110 VGPRs at D = 64 (four);
// with two row blocks 256 VGPRs + AGPRs at D = 256 (one), ~230 at D = 128
// (two), ~150 at D = 64 (three).
inline int resident_chunk_wgs_per_cu(const kvq_layout& L, int rows_per_wg) {
  const bool two = rows_per_wg == 32 * kChunkWaves;
  if (has_q4(L)) return 2;  // the 4-bit chunk kernel: ~210 VGPRs, 51-61 KB of LDS
  if (L.head_dim == 256) return two ? 1 : 2;
  if (L.head_dim == 128) return two ? 2 : 3;
  return two ? 3 : 4;
}

// Byte sizes of one store element (int8 and fp32 stores).
inline int store_elem_bytes(int dtype) { return dtype == KVQ_STORE_INT8 ? 1 : 4; }

// Bytes of `elems` consecutive elements of a store (a q4 element is half a byte).
inline int64_t store_bytes(int64_t elems, int dtype) {
  return dtype == KVQ_STORE_Q4 ? elems / 2 : elems * store_elem_bytes(dtype);
}

// Values per Q4_0 block (one fp16 scale each).
constexpr int kQ4Block = 32;

// Number of fp16 scales per row (0 for an fp32 store).
inline int scales_per_row(const kvq_layout& L, int dtype) {
  if (dtype == KVQ_STORE_Q4) return L.head_dim / kQ4Block;
  return dtype == KVQ_STORE_INT8 ? L.head_dim / L.scale_group : 0;
}


// Store combinations with a q4 store that the decode kernels implement: q4 K
// and V (q4_0), int8 K with q4 V (k8v4).
inline bool q4_decode_supported(const kvq_layout& L) {
  return L.v_dtype == KVQ_STORE_Q4 && (L.k_dtype == KVQ_STORE_Q4 || L.k_dtype == KVQ_STORE_INT8);
}

// Checks a layout on its own (no pointers). Returns KVQ_OK or an error code.
int check_layout(const kvq_layout* L);

// Checks pointer alignment of a store and its scale array for `L`.
int check_store_ptrs(const kvq_layout& L, int dtype, const void* store, const void* scales);

// Bytes of one region of a cache blob: padded to 16.
inline int64_t blob_region_bytes(int64_t bytes) { return (bytes + 15) / 16 * 16; }

// Payload bytes of a cache blob of n_pos positions: K values, V values, then
// the fp16 scales of each int8 or q4 store, every region padded to 16 bytes.
inline int64_t blob_payload_bytes(const kvq_layout& L, int64_t n_pos) {
  const int64_t rows = n_pos * L.n_kv_heads;
  int64_t b = 0;
  for (int dt : {L.k_dtype, L.v_dtype}) b += blob_region_bytes(store_bytes(rows * L.head_dim, dt));
  for (int dt : {L.k_dtype, L.v_dtype}) b += blob_region_bytes(rows * scales_per_row(L, dt) * 2);
  return b;
}

// Attended-range length bound used by the planner.
inline int64_t effective_len(int64_t max_len, int32_t window) {
  return window > 0 && window < max_len ? window : max_len;
}

// Bytes of K and V (codes and scales, without slot padding) of one position
// of one kv head.
inline int64_t kv_bytes_per_pos(const kvq_layout& L) {
  int64_t b = 0;
  for (int dt : {L.k_dtype, L.v_dtype}) b += store_bytes(L.head_dim, dt) + 2 * scales_per_row(L, dt);
  return b;
}

// Query rows per workgroup of the chunk-rows path of the int8 / fp32 decode
// kernel (launch_chunk_rows): one block of 16 (token, head) rows, or, with
// int8 K and V and more than 16 rows per kv head, two sharing every key and
// value operand.
inline int chunk_rows_per_block(const kvq_layout& L, int64_t n_tok, int64_t G) {
  const bool i8 = L.k_dtype == KVQ_STORE_INT8 && L.v_dtype == KVQ_STORE_INT8;
  return i8 && n_tok * G > kHeadsPerBlock ? 32 : 16;
}

// (token, head) rows per kv head up to which a chunk over a 4-bit layout goes
// through the 4-bit decode partial kernel, in 16-row workgroups (each reading
// every key). Measured at 128K keys, 8 heads per kv head (kv_chunk_attn
// alone): 1 / 2 / 4 tokens q4_0 30 / 32 / 46 us against 65 / 63 / 67 us with
// the 4-bit chunk kernel, k8v4 28 / 29 / 41 us against 54 us; even without
// any on-chip reuse of the second workgroup's reads two decode-sized passes
// stay below the chunk kernel's time.
constexpr int64_t kQ4RowsMax = 32;

// A chunk goes through the decode partial kernels ("chunk rows") when a kv
// head has at most this many (token, head) rows: its rows share every key
// tile, the waves and splits divide the keys, where the chunk kernels would
// give a short verify window few workgroups with long key ranges.
//  - int8 K and V: 32 rows, one workgroup. Measured (kv_chunk_attn alone):
//    128K keys, 8 heads per kv head, 1 / 2 / 4 tokens 32 / 32 / 42 us against
//    50 / 50 / 49 us with the chunk kernel; 64 sequences of 32K keys, 4 heads
//    per kv head, 1 to 8 tokens 0.75-0.86 ms against 1.40-1.46 ms. With 64
//    rows (two such workgroups, each reading the keys) the chunk kernel is
//    faster (128K, 8 tokens: 57 against 60 us).
//  - the 4-bit layouts: kQ4RowsMax.
//  - an fp32 store (k8v32, k32v8, k32v32): 16 rows, one workgroup; the chunk
//    kernels take int8 and 4-bit stores only, so longer chunks over these
//    layouts are refused.
inline int64_t chunk_rows_max(const kvq_layout& L) {
  if (has_q4(L)) return kQ4RowsMax;
  if (L.k_dtype == KVQ_STORE_INT8 && L.v_dtype == KVQ_STORE_INT8) return 2 * kHeadsPerBlock;
  return kHeadsPerBlock;
}
inline bool chunk_as_rows(const kvq_layout& L, int64_t n_tok, int64_t G) { return n_tok * G <= chunk_rows_max(L); }

// Workspace bytes for a plan.
inline int64_t workspace_bytes(int64_t batch, int64_t n_q, int64_t n_splits, int64_t head_dim) {
  return batch * n_q * n_splits * (head_dim + 2) * 4;
}

// Bytes of the library's static device scratch (kv_decode_attn_static).
constexpr int64_t kStaticScratchBytes = KVQ_STATIC_SCRATCH_BYTES;

// The device address of the static scratch on the current device (looked up
// once per device, kvq_static.hip). Returns KVQ_OK or KVQ_ERR_HIP.
int static_scratch(void** out);

// Kernel launchers (defined in the .hip files). They assume validated input.
int launch_append(const kvq_layout& L, void* k_store, void* v_store, uint16_t* k_scales,
                  uint16_t* v_scales, const uint16_t* k_new, const uint16_t* v_new,
                  const int32_t* d_start_pos, int32_t batch, int32_t n_tok, void* stream);

// k_new / v_new non-null: the fused append of kv_append_decode_splitk.
// out and arrive non-null: the one-launch step of kv_decode_attn (int8 K and V
// stores, one_launch_ok): the last workgroup of each unit writes the output.
int launch_partial(const kvq_layout& L, const void* k_store, const void* v_store,
                   const uint16_t* k_scales, const uint16_t* v_scales, const uint16_t* k_new,
                   const uint16_t* v_new, const uint16_t* q, int32_t batch, int32_t n_q_heads,
                   const int32_t* d_seq_lens, int32_t window, float sm_scale, const kvq_plan_t& plan,
                   void* ws, void* stream, uint16_t* out = nullptr, uint32_t* arrive = nullptr);

// The one-launch step of kv_decode_attn: query heads per unit (sequence, kv
// head, head block), at most kOneLaunchMaxRowValues (query head x dim) values
// per unit: min(G, 16, 512 / head_dim) -- 2 heads at head_dim 256, 4 at 128,
// 8 at 64. Every workgroup writes its unit's partial through to memory, and
// measured against the partials + reduce that hand-off pays when the partial
// is small: with 8 heads x 256 dims per unit (8 KB per split) one launch was
// 0.3-0.7 us slower per step, with 4 x 256 0.2-0.7 us faster and with
// 2 x 256 faster again (Gemma 4K 9.8 -> 8.9 us); 1 x 256 ties with 2 x 256.
constexpr int kOneLaunchMaxRowValues = 512;
inline int one_launch_rows(int64_t head_dim, int64_t G) {
  int64_t r = G < kHeadsPerBlock ? G : kHeadsPerBlock;
  if (r * head_dim > kOneLaunchMaxRowValues) r = kOneLaunchMaxRowValues / head_dim;
  return (int)(r > 0 ? r : 1);
}

// Whether kv_decode_attn runs the plan as one launch: int8 K and V stores, at
// most kOneLaunchMaxSplits splits, and a partial region that one buffer
// resource covers.
inline bool one_launch_ok(const kvq_layout& L, int64_t batch, int64_t n_q_heads, const kvq_plan_t& plan) {
  return L.k_dtype == KVQ_STORE_INT8 && L.v_dtype == KVQ_STORE_INT8 && plan.n_splits <= kOneLaunchMaxSplits &&
         workspace_bytes(batch, n_q_heads, plan.n_splits, L.head_dim) <= 0x7fffffff;
}

int launch_chunk(const kvq_layout& L, const void* k_store, const void* v_store, const uint16_t* k_scales,
                 const uint16_t* v_scales, const uint16_t* q, int32_t batch, int32_t n_tok, int32_t n_q_heads,
                 const int32_t* d_start_pos, int32_t window, float sm_scale, const kvq_plan_t& plan, void* ws,
                 void* stream);

// Chunk attention through the decode partial kernel (int8 K and V): the
// (token, head) rows of a kv head in blocks of 16, every key read once per
// block. For chunks with few rows per kv head (a verify window).
int launch_chunk_rows(const kvq_layout& L, const void* k_store, const void* v_store, const uint16_t* k_scales,
                      const uint16_t* v_scales, const uint16_t* q, int32_t batch, int32_t n_tok, int32_t n_q_heads,
                      const int32_t* d_start_pos, int32_t window, float sm_scale, const kvq_plan_t& plan, void* ws,
                      void* stream);

// Chunk attention over a layout with a q4 store (q4_decode_supported).
int launch_chunk_q4(const kvq_layout& L, const void* k_store, const void* v_store, const uint16_t* k_scales,
                    const uint16_t* v_scales, const uint16_t* q, int32_t batch, int32_t n_tok, int32_t n_q_heads,
                    const int32_t* d_start_pos, int32_t window, float sm_scale, const kvq_plan_t& plan, void* ws,
                    void* stream);

int launch_blob(const kvq_layout& L, void* k_store, void* v_store, uint16_t* k_scales, uint16_t* v_scales,
                int32_t seq, int32_t pos0, int32_t n_pos, void* blob, bool unpack, void* stream);

// Chunk attention through the 4-bit decode partial kernel (q4_0, k8v4): the
// (token, head) rows of a kv head in blocks of 16, one workgroup per block.
int launch_chunk_rows_q4(const kvq_layout& L, const void* k_store, const void* v_store, const uint16_t* k_scales,
                         const uint16_t* v_scales, const uint16_t* q, int32_t batch, int32_t n_tok, int32_t n_q_heads,
                         const int32_t* d_start_pos, int32_t window, float sm_scale, const kvq_plan_t& plan, void* ws,
                         void* stream);

// Partials of a layout with a q4 store (q4_decode_supported).
// k_new / v_new non-null: the fused append of kv_append_decode_splitk.
int launch_partial_q4(const kvq_layout& L, const void* k_store, const void* v_store, const uint16_t* k_scales,
                      const uint16_t* v_scales, const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q,
                      int32_t batch, int32_t n_q_heads, const int32_t* d_seq_lens, int32_t window, float sm_scale,
                      const kvq_plan_t& plan, void* ws, void* stream);

// The read-only streaming reference of kvq_stream_read.
int launch_stream(const void* buf, int64_t bytes, uint32_t* sink, int n_cu, void* stream);

int launch_reduce(const kvq_layout& L, const void* ws, int32_t batch, int32_t n_q_heads,
                  const kvq_plan_t& plan, uint16_t* out, void* stream);

}  // namespace kvq
