// Host side of libkvq: argument validation, the split planner and the C-ABI
// entry points. Validation always runs before any HIP call, so every error path
// can be exercised without a device.
#include <limits.h>
#include <algorithm>
#include <stddef.h>

#include "kvq_internal.h"

namespace kvq {

static bool aligned(const void* p, uint64_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_layout(const kvq_layout* L) {
  if (!L) return KVQ_ERR_NULL;
  if (L->n_kv_heads < 1 || L->head_dim < 1 || L->max_ctx < 1) return KVQ_ERR_SHAPE;
  // Strata PR 2698 "What it does": the host refuses a head_dim not divisible by
  // 64; the library also bounds it to the instantiated tile shapes.
  if (L->head_dim % 64 != 0) return KVQ_ERR_UNSUPPORTED;
  if (L->head_dim != 64 && L->head_dim != 128 && L->head_dim != 256) return KVQ_ERR_UNSUPPORTED;
  if (L->slot_dim < L->head_dim) return KVQ_ERR_SHAPE;  // genie v1.2.1: slot >= head_dim
  for (int dt : {L->k_dtype, L->v_dtype})
    if (dt != KVQ_STORE_INT8 && dt != KVQ_STORE_FP32 && dt != KVQ_STORE_Q4) return KVQ_ERR_UNSUPPORTED;
  // Strata PR 2698 "Not in this PR": the 4-bit stores rotate over head_dim 256.
  if (has_q4(*L) && L->head_dim != 256) return KVQ_ERR_UNSUPPORTED;
  const bool any_i8 = L->k_dtype == KVQ_STORE_INT8 || L->v_dtype == KVQ_STORE_INT8;
  if (any_i8 && L->scale_group != 64 && L->scale_group != L->head_dim) return KVQ_ERR_UNSUPPORTED;
  if (L->s_seq < 0 || L->s_pos < 0 || L->s_head < 0) return KVQ_ERR_SHAPE;
  if (L->ss_seq < 0 || L->ss_pos < 0 || L->ss_head < 0) return KVQ_ERR_SHAPE;
  // A row never overlaps the next position's row of the same head: the kernels
  // rely on it to make positions past the context read as zero.
  if (L->s_pos < L->head_dim) return KVQ_ERR_SHAPE;
  for (int dt : {L->k_dtype, L->v_dtype}) {
    // Row offsets in bytes are multiples of 16 (for a q4 store, whose element
    // is half a byte: element offsets multiples of 32).
    if (dt == KVQ_STORE_Q4) {
      if ((L->s_seq | L->s_pos | L->s_head) & 31) return KVQ_ERR_ALIGN;
    } else {
      const int64_t eb = store_elem_bytes(dt);
      if ((L->s_seq * eb) % 16 || (L->s_pos * eb) % 16 || (L->s_head * eb) % 16) return KVQ_ERR_ALIGN;
    }
    // One (sequence, head) slice is addressed with 32-bit offsets.
    const int64_t extent = store_bytes((L->max_ctx - 1) * L->s_pos + L->head_dim, dt);
    if (extent > (int64_t)INT_MAX) return KVQ_ERR_UNSUPPORTED;
  }
  for (int dt : {L->k_dtype, L->v_dtype}) {
    const int64_t ng = scales_per_row(*L, dt);
    if (!ng) continue;
    if (L->ss_pos < ng) return KVQ_ERR_SHAPE;
    const int64_t a = 2 * ng;
    if ((L->ss_seq * 2) % a || (L->ss_pos * 2) % a || (L->ss_head * 2) % a) return KVQ_ERR_ALIGN;
    const int64_t extent = ((L->max_ctx - 1) * L->ss_pos + ng) * 2;
    if (extent > (int64_t)INT_MAX) return KVQ_ERR_UNSUPPORTED;
  }
  return KVQ_OK;
}

int check_store_ptrs(const kvq_layout& L, int dtype, const void* store, const void* scales) {
  if (!store) return KVQ_ERR_NULL;
  if (!aligned(store, 16)) return KVQ_ERR_ALIGN;
  if (const int ng = scales_per_row(L, dtype)) {
    // genie v0.1.0-alpha.11 "--int8-kv triage": a missing scale pointer must be
    // refused, never read as scale 1.0.
    if (!scales) return KVQ_ERR_NULL;
    if (!aligned(scales, 2 * ng)) return KVQ_ERR_ALIGN;
  }
  return KVQ_OK;
}

static int check_plan(const kvq_layout& L, int32_t batch, int32_t n_q, const kvq_plan_t* plan) {
  if (!plan) return KVQ_ERR_NULL;
  if (plan->n_splits < 1 || plan->n_splits > kMaxSplits) return KVQ_ERR_SHAPE;
  if (plan->chunk < kTile || plan->chunk % kTile) return KVQ_ERR_SHAPE;
  if (plan->ws_bytes < workspace_bytes(batch, n_q, plan->n_splits, L.head_dim)) return KVQ_ERR_WORKSPACE;
  return KVQ_OK;
}

static int check_heads(const kvq_layout& L, int32_t batch, int32_t n_q) {
  if (batch < 0 || n_q < 1) return KVQ_ERR_SHAPE;
  if (batch > 65535 || (int64_t)batch * n_q > INT_MAX / 8) return KVQ_ERR_UNSUPPORTED;  // grid limits
  if (n_q % L.n_kv_heads) return KVQ_ERR_SHAPE;
  return KVQ_OK;
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

}  // namespace kvq

using namespace kvq;

extern "C" {

int kvq_version(void) { return (0 << 16) | (1 << 8) | 0; }

const char* kvq_status_string(int s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_NULL: return "null pointer (a required buffer or an int8 store's scales)";
    case KVQ_ERR_SHAPE: return "inconsistent shape or stride";
    case KVQ_ERR_UNSUPPORTED: return "unsupported head_dim, scale group, dtype or extent";
    case KVQ_ERR_ALIGN: return "misaligned pointer or stride";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_HIP: return "HIP runtime error at launch";
    case KVQ_ERR_MISMATCH: return "cache blob does not match the cache layout (store types, scale group, heads)";
    case KVQ_ERR_SCRATCH: return "split partials exceed the library's static scratch (16 MiB)";
    default: return "unknown status";
  }
}

// Key positions per split of the decode partial kernel for l_eff keys, with
// `units` workgroups per split index (sequences x kv heads x 16-row blocks)
// and `rows` (<= 16) query rows per workgroup.
static int64_t decode_split_chunk(const kvq_layout& L, int64_t l_eff, int64_t units, int64_t rows, int32_t n_cu) {
  int64_t chunk;
  if (l_eff < 64) {
    // genie v1.3.0: a single block below 64 positions.
    chunk = round_up(l_eff > 0 ? l_eff : 1, kTile);
  } else {
    // Bytes one position of one kv head costs to read (algorithmic).
    const int64_t kv_pos = kv_bytes_per_pos(L);
    // Partial (m, l, O) bytes one split writes for its query rows.
    const int64_t part = rows * (L.head_dim + 2) * 4;
    // Long splits keep the partial traffic near 1 % of the KV bytes ...
    chunk = ceil_div(part * 100, kv_pos);
    if (chunk < 512) chunk = 512;
    // ... unless that leaves fewer workgroups than compute units; then the
    // chip gets one workgroup per CU. (Measured on single sequences of 32K to
    // 128K positions at head_dim 64 to 256: one workgroup per CU, each with
    // longer splits, beats filling every CU's resident slots, since each
    // workgroup pays its pipeline start and merge once and the reduce reads
    // half as many partials.)
    const int64_t want_wg = n_cu;
    if (units * ceil_div(l_eff, chunk) < want_wg) chunk = ceil_div(units * l_eff, want_wg);
    // A split gets at least one tile per wavefront of its workgroup.
    chunk = round_up(chunk < kMinSplitChunk ? kMinSplitChunk : chunk, kTile);
    const int64_t cap = round_up(l_eff, kTile);
    if (chunk > cap) chunk = cap;
    // The reduce keeps one weight per split in LDS.
    const int64_t min_chunk = round_up(ceil_div(l_eff, kMaxSplits), kTile);
    if (chunk < min_chunk) chunk = min_chunk;
  }
  return chunk;
}

int kvq_plan(const kvq_layout* layout, int32_t batch, int32_t n_q_heads, int32_t max_seq_len,
             int32_t window, int32_t n_cu, kvq_plan_t* out) {
  int st = check_layout(layout);
  if (st) return st;
  if (!out) return KVQ_ERR_NULL;
  const kvq_layout& L = *layout;
  if ((st = check_heads(L, batch, n_q_heads))) return st;
  if (max_seq_len < 0 || window < 0 || n_cu < 1) return KVQ_ERR_SHAPE;

  const int64_t l_eff = effective_len(max_seq_len, window);
  const int64_t G = n_q_heads / L.n_kv_heads;
  const int64_t head_blocks = ceil_div(G, kHeadsPerBlock);
  const int64_t units = (int64_t)(batch > 0 ? batch : 1) * L.n_kv_heads * head_blocks;
  const int64_t chunk = decode_split_chunk(L, l_eff, units, G < kHeadsPerBlock ? G : kHeadsPerBlock, n_cu);
  if (chunk > INT_MAX) return KVQ_ERR_UNSUPPORTED;
  int64_t n_splits = l_eff > 0 ? ceil_div(l_eff, chunk) : 1;
  out->chunk = (int32_t)chunk;
  out->n_splits = (int32_t)n_splits;
  out->ws_bytes = workspace_bytes(batch, n_q_heads, n_splits, L.head_dim);
  return KVQ_OK;
}

int kv_quant_append(const kvq_layout* layout, void* k_store, void* v_store, uint16_t* k_scales,
                    uint16_t* v_scales, const uint16_t* k_new, const uint16_t* v_new,
                    const int32_t* d_start_pos, int32_t batch, int32_t n_tok, void* stream) {
  int st = check_layout(layout);
  if (st) return st;
  const kvq_layout& L = *layout;
  if ((st = check_store_ptrs(L, L.k_dtype, k_store, k_scales))) return st;
  if ((st = check_store_ptrs(L, L.v_dtype, v_store, v_scales))) return st;
  if (!k_new || !v_new || !d_start_pos) return KVQ_ERR_NULL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(d_start_pos, 4)) return KVQ_ERR_ALIGN;
  if (batch < 0 || n_tok < 0) return KVQ_ERR_SHAPE;
  if ((int64_t)batch * n_tok * L.n_kv_heads > (int64_t)INT_MAX / 64) return KVQ_ERR_UNSUPPORTED;
  if (batch == 0 || n_tok == 0) return KVQ_OK;
  return launch_append(L, k_store, v_store, k_scales, v_scales, k_new, v_new, d_start_pos, batch,
                       n_tok, stream);
}

int kv_decode_attn_splitk(const kvq_layout* layout, const void* k_store, const void* v_store,
                          const uint16_t* k_scales, const uint16_t* v_scales, const uint16_t* q,
                          int32_t batch, int32_t n_q_heads, const int32_t* d_seq_lens,
                          int32_t window, float sm_scale, const kvq_plan_t* plan, void* ws,
                          int64_t ws_bytes, void* stream) {
  int st = check_layout(layout);
  if (st) return st;
  const kvq_layout& L = *layout;
  if ((st = check_store_ptrs(L, L.k_dtype, k_store, k_scales))) return st;
  if ((st = check_store_ptrs(L, L.v_dtype, v_store, v_scales))) return st;
  if ((st = check_heads(L, batch, n_q_heads))) return st;
  if ((st = check_plan(L, batch, n_q_heads, plan))) return st;
  if (!q || !d_seq_lens) return KVQ_ERR_NULL;
  if (!aligned(q, 16) || !aligned(d_seq_lens, 4)) return KVQ_ERR_ALIGN;
  if (window < 0) return KVQ_ERR_SHAPE;
  if (!(sm_scale == sm_scale) || sm_scale > 3.0e38f || sm_scale < -3.0e38f) return KVQ_ERR_SHAPE;
  if (!ws) return KVQ_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return KVQ_ERR_ALIGN;
  if (ws_bytes < plan->ws_bytes) return KVQ_ERR_WORKSPACE;
  if (has_q4(L) && !q4_decode_supported(L)) return KVQ_ERR_UNSUPPORTED;
  if (batch == 0) return KVQ_OK;
  if (has_q4(L))
    return launch_partial_q4(L, k_store, v_store, k_scales, v_scales, nullptr, nullptr, q, batch, n_q_heads,
                             d_seq_lens, window, sm_scale, *plan, ws, stream);
  return launch_partial(L, k_store, v_store, k_scales, v_scales, nullptr, nullptr, q, batch, n_q_heads,
                        d_seq_lens, window, sm_scale, *plan, ws, stream);
}

int kv_decode_attn_static(const kvq_layout* layout, const void* k_store, const void* v_store,
                          const uint16_t* k_scales, const uint16_t* v_scales, const uint16_t* q, int32_t batch,
                          int32_t n_q_heads, const int32_t* d_seq_lens, int32_t window, float sm_scale,
                          const kvq_plan_t* plan, uint16_t* out, void* stream) {
  int st = check_layout(layout);
  if (st) return st;
  const kvq_layout& L = *layout;
  if ((st = check_store_ptrs(L, L.k_dtype, k_store, k_scales))) return st;
  if ((st = check_store_ptrs(L, L.v_dtype, v_store, v_scales))) return st;
  if ((st = check_heads(L, batch, n_q_heads))) return st;
  if (!plan) return KVQ_ERR_NULL;
  if (plan->n_splits < 1 || plan->n_splits > kMaxSplits) return KVQ_ERR_SHAPE;
  if (plan->chunk < kTile || plan->chunk % kTile) return KVQ_ERR_SHAPE;
  if (workspace_bytes(batch, n_q_heads, plan->n_splits, L.head_dim) > kStaticScratchBytes) return KVQ_ERR_SCRATCH;
  if (!q || !d_seq_lens || !out) return KVQ_ERR_NULL;
  if (!aligned(q, 16) || !aligned(d_seq_lens, 4) || !aligned(out, 16)) return KVQ_ERR_ALIGN;
  if (window < 0) return KVQ_ERR_SHAPE;
  if (!(sm_scale == sm_scale) || sm_scale > 3.0e38f || sm_scale < -3.0e38f) return KVQ_ERR_SHAPE;
  if (has_q4(L) && !q4_decode_supported(L)) return KVQ_ERR_UNSUPPORTED;
  if (batch == 0) return KVQ_OK;
  void* ws = nullptr;
  if ((st = static_scratch(&ws))) return st;
  st = has_q4(L) ? launch_partial_q4(L, k_store, v_store, k_scales, v_scales, nullptr, nullptr, q, batch, n_q_heads,
                                     d_seq_lens, window, sm_scale, *plan, ws, stream)
                 : launch_partial(L, k_store, v_store, k_scales, v_scales, nullptr, nullptr, q, batch, n_q_heads,
                                  d_seq_lens, window, sm_scale, *plan, ws, stream);
  if (st) return st;
  return launch_reduce(L, ws, batch, n_q_heads, *plan, out, stream);
}

int kv_append_decode_splitk(const kvq_layout* layout, void* k_store, void* v_store, uint16_t* k_scales,
                            uint16_t* v_scales, const uint16_t* k_new, const uint16_t* v_new,
                            const uint16_t* q, int32_t batch, int32_t n_q_heads,
                            const int32_t* d_seq_lens, int32_t window, float sm_scale,
                            const kvq_plan_t* plan, void* ws, int64_t ws_bytes, void* stream) {
  int st = check_layout(layout);
  if (st) return st;
  const kvq_layout& L = *layout;
  if ((st = check_store_ptrs(L, L.k_dtype, k_store, k_scales))) return st;
  if ((st = check_store_ptrs(L, L.v_dtype, v_store, v_scales))) return st;
  if ((st = check_heads(L, batch, n_q_heads))) return st;
  if ((st = check_plan(L, batch, n_q_heads, plan))) return st;
  if (!k_new || !v_new || !q || !d_seq_lens) return KVQ_ERR_NULL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(q, 16) || !aligned(d_seq_lens, 4))
    return KVQ_ERR_ALIGN;
  if (window < 0) return KVQ_ERR_SHAPE;
  if (!(sm_scale == sm_scale) || sm_scale > 3.0e38f || sm_scale < -3.0e38f) return KVQ_ERR_SHAPE;
  if (!ws) return KVQ_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return KVQ_ERR_ALIGN;
  if (ws_bytes < plan->ws_bytes) return KVQ_ERR_WORKSPACE;
  if (has_q4(L) && !q4_decode_supported(L)) return KVQ_ERR_UNSUPPORTED;
  if (batch == 0) return KVQ_OK;
  if (has_q4(L))
    return launch_partial_q4(L, k_store, v_store, k_scales, v_scales, k_new, v_new, q, batch, n_q_heads,
                             d_seq_lens, window, sm_scale, *plan, ws, stream);
  return launch_partial(L, k_store, v_store, k_scales, v_scales, k_new, v_new, q, batch, n_q_heads,
                        d_seq_lens, window, sm_scale, *plan, ws, stream);
}

int kvq_decode_launches(const kvq_layout* layout, int32_t batch, int32_t n_q_heads, const kvq_plan_t* plan,
                        int32_t* launches) {
  int st = check_layout(layout);
  if (st) return st;
  const kvq_layout& L = *layout;
  if ((st = check_heads(L, batch, n_q_heads))) return st;
  if ((st = check_plan(L, batch, n_q_heads, plan))) return st;
  if (!launches) return KVQ_ERR_NULL;
  *launches = batch == 0 ? 0 : (!has_q4(L) && one_launch_ok(L, batch, n_q_heads, *plan) ? 1 : 2);
  return KVQ_OK;
}

int kv_decode_attn(const kvq_layout* layout, void* k_store, void* v_store, uint16_t* k_scales, uint16_t* v_scales,
                   const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q, int32_t batch,
                   int32_t n_q_heads, const int32_t* d_seq_lens, int32_t window, float sm_scale,
                   const kvq_plan_t* plan, void* ws, int64_t ws_bytes, uint32_t* d_arrive, uint16_t* out,
                   void* stream) {
  int st = check_layout(layout);
  if (st) return st;
  const kvq_layout& L = *layout;
  if ((st = check_store_ptrs(L, L.k_dtype, k_store, k_scales))) return st;
  if ((st = check_store_ptrs(L, L.v_dtype, v_store, v_scales))) return st;
  if ((st = check_heads(L, batch, n_q_heads))) return st;
  if ((st = check_plan(L, batch, n_q_heads, plan))) return st;
  if ((k_new == nullptr) != (v_new == nullptr)) return KVQ_ERR_NULL;
  if (!q || !d_seq_lens || !out || !d_arrive) return KVQ_ERR_NULL;
  if ((k_new && (!aligned(k_new, 16) || !aligned(v_new, 16))) || !aligned(q, 16) || !aligned(d_seq_lens, 4) ||
      !aligned(out, 16) || !aligned(d_arrive, 4))
    return KVQ_ERR_ALIGN;
  if (window < 0) return KVQ_ERR_SHAPE;
  if (!(sm_scale == sm_scale) || sm_scale > 3.0e38f || sm_scale < -3.0e38f) return KVQ_ERR_SHAPE;
  if (!ws) return KVQ_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return KVQ_ERR_ALIGN;
  if (ws_bytes < plan->ws_bytes) return KVQ_ERR_WORKSPACE;
  if (has_q4(L) && !q4_decode_supported(L)) return KVQ_ERR_UNSUPPORTED;
  if (batch == 0) return KVQ_OK;
  if (!has_q4(L) && one_launch_ok(L, batch, n_q_heads, *plan))
    return launch_partial(L, k_store, v_store, k_scales, v_scales, k_new, v_new, q, batch, n_q_heads, d_seq_lens,
                          window, sm_scale, *plan, ws, stream, out, d_arrive);
  if (has_q4(L))
    st = launch_partial_q4(L, k_store, v_store, k_scales, v_scales, k_new, v_new, q, batch, n_q_heads, d_seq_lens,
                           window, sm_scale, *plan, ws, stream);
  else
    st = launch_partial(L, k_store, v_store, k_scales, v_scales, k_new, v_new, q, batch, n_q_heads, d_seq_lens,
                        window, sm_scale, *plan, ws, stream);
  if (st) return st;
  return launch_reduce(L, ws, batch, n_q_heads, *plan, out, stream);
}

int kvq_plan_chunk(const kvq_layout* layout, int32_t batch, int32_t n_tok, int32_t n_q_heads,
                   int32_t max_seq_len, int32_t window, int32_t n_cu, kvq_plan_t* out) {
  int st = check_layout(layout);
  if (st) return st;
  if (!out) return KVQ_ERR_NULL;
  const kvq_layout& L = *layout;
  if ((st = check_heads(L, batch, n_q_heads))) return st;
  if (n_tok < 0 || max_seq_len < 0 || window < 0 || n_cu < 1) return KVQ_ERR_SHAPE;
  const int64_t G = n_q_heads / L.n_kv_heads;
  // Keys one workgroup may walk: the whole prefix, or the window plus the chunk.
  const int64_t l_eff = window > 0 ? std::min<int64_t>(max_seq_len, (int64_t)window + n_tok) : max_seq_len;
  if (chunk_as_rows(L, n_tok, G)) {  // the decode partial kernel and its split rule
    const int64_t rows = std::max<int64_t>(1, (int64_t)n_tok * G);
    const int64_t per_wg = has_q4(L) ? kHeadsPerBlock : chunk_rows_per_block(L, n_tok, G);
    const int64_t units = (int64_t)(batch > 0 ? batch : 1) * L.n_kv_heads * ceil_div(rows, per_wg);
    const int64_t chunk = decode_split_chunk(L, l_eff, units, std::min(rows, per_wg), n_cu);
    const int64_t n_splits = l_eff > 0 ? ceil_div(l_eff, chunk) : 1;
    if (n_splits > kMaxSplits || chunk > INT_MAX) return KVQ_ERR_UNSUPPORTED;
    out->n_splits = (int32_t)n_splits;
    out->chunk = (int32_t)chunk;
    out->ws_bytes = workspace_bytes((int64_t)batch * n_tok, n_q_heads, n_splits, L.head_dim);
    return KVQ_OK;
  }
  const int64_t units = (int64_t)(batch > 0 ? batch : 1) * L.n_kv_heads * chunk_row_blocks(n_tok > 0 ? n_tok : 1, G, L.head_dim);
  const int64_t want = (int64_t)resident_chunk_wgs_per_cu(L, chunk_rows_per_wg(n_tok > 0 ? n_tok : 1, G, L.head_dim)) * n_cu;
  int64_t n_splits = 1, chunk = round_up(l_eff > 0 ? l_eff : 1, kTile);
  if (units < want && l_eff > kMinSplitChunk) {
    // Few query rows over a long prefix (a verify window): split the keys so
    // that the grid still covers the chip, at least 4 tiles per split.
    n_splits = std::min(ceil_div(want, units), ceil_div(l_eff, kMinSplitChunk));
    chunk = round_up(ceil_div(l_eff, n_splits), kTile);
    n_splits = ceil_div(l_eff, chunk);
  }
  if (n_splits > kMaxSplits || chunk > INT_MAX) return KVQ_ERR_UNSUPPORTED;
  out->n_splits = (int32_t)n_splits;
  out->chunk = (int32_t)chunk;
  out->ws_bytes = workspace_bytes((int64_t)batch * n_tok, n_q_heads, n_splits, L.head_dim);
  return KVQ_OK;
}

int kv_chunk_attn(const kvq_layout* layout, const void* k_store, const void* v_store, const uint16_t* k_scales,
                  const uint16_t* v_scales, const uint16_t* q, int32_t batch, int32_t n_tok, int32_t n_q_heads,
                  const int32_t* d_start_pos, int32_t window, float sm_scale, const kvq_plan_t* plan, void* ws,
                  int64_t ws_bytes, uint16_t* out, void* stream) {
  int st = check_layout(layout);
  if (st) return st;
  const kvq_layout& L = *layout;
  // int8 K and V, the 4-bit layouts of the decode path (q4_0, k8v4), or an
  // fp32 store when the chunk's rows fit the decode kernel's chunk rows
  if (has_q4(L) && !q4_decode_supported(L)) return KVQ_ERR_UNSUPPORTED;
  if ((st = check_store_ptrs(L, L.k_dtype, k_store, k_scales))) return st;
  if ((st = check_store_ptrs(L, L.v_dtype, v_store, v_scales))) return st;
  if ((st = check_heads(L, batch, n_q_heads))) return st;
  if (n_tok < 0) return KVQ_ERR_SHAPE;
  const bool any_fp32 = L.k_dtype == KVQ_STORE_FP32 || L.v_dtype == KVQ_STORE_FP32;
  if (any_fp32 && !chunk_as_rows(L, n_tok, n_q_heads / L.n_kv_heads)) return KVQ_ERR_UNSUPPORTED;
  if (!plan) return KVQ_ERR_NULL;
  if (plan->n_splits < 1 || plan->n_splits > kMaxSplits) return KVQ_ERR_SHAPE;
  if (plan->chunk < kTile || plan->chunk % kTile) return KVQ_ERR_SHAPE;
  // Key positions of a split are 32-bit in the chunk kernels.
  if ((int64_t)plan->n_splits * plan->chunk > (int64_t)INT_MAX) return KVQ_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)batch * n_tok;
  if (rows * n_q_heads > INT_MAX / 8 || (int64_t)L.n_kv_heads * chunk_row_blocks(n_tok, n_q_heads / L.n_kv_heads, L.head_dim) > 65535)
    return KVQ_ERR_UNSUPPORTED;  // grid limits
  if (plan->ws_bytes < workspace_bytes(rows, n_q_heads, plan->n_splits, L.head_dim)) return KVQ_ERR_WORKSPACE;
  if (!q || !d_start_pos || !out) return KVQ_ERR_NULL;
  if (!aligned(q, 16) || !aligned(d_start_pos, 4) || !aligned(out, 16)) return KVQ_ERR_ALIGN;
  if (window < 0) return KVQ_ERR_SHAPE;
  if (!(sm_scale == sm_scale) || sm_scale > 3.0e38f || sm_scale < -3.0e38f) return KVQ_ERR_SHAPE;
  if (!ws) return KVQ_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return KVQ_ERR_ALIGN;
  if (ws_bytes < plan->ws_bytes) return KVQ_ERR_WORKSPACE;
  if (batch == 0 || n_tok == 0) return KVQ_OK;
  if (has_q4(L) && chunk_as_rows(L, n_tok, n_q_heads / L.n_kv_heads))
    st = launch_chunk_rows_q4(L, k_store, v_store, k_scales, v_scales, q, batch, n_tok, n_q_heads, d_start_pos,
                              window, sm_scale, *plan, ws, stream);
  else if (has_q4(L))
    st = launch_chunk_q4(L, k_store, v_store, k_scales, v_scales, q, batch, n_tok, n_q_heads, d_start_pos, window,
                         sm_scale, *plan, ws, stream);
  else if (chunk_as_rows(L, n_tok, n_q_heads / L.n_kv_heads))
    st = launch_chunk_rows(L, k_store, v_store, k_scales, v_scales, q, batch, n_tok, n_q_heads, d_start_pos, window,
                           sm_scale, *plan, ws, stream);
  else
    st = launch_chunk(L, k_store, v_store, k_scales, v_scales, q, batch, n_tok, n_q_heads, d_start_pos, window,
                      sm_scale, *plan, ws, stream);
  if (st) return st;
  // The partial rows are (b, t, hq): the reduce treats batch * n_tok rows of n_q_heads.
  return launch_reduce(L, ws, (int32_t)rows, n_q_heads, *plan, out, stream);
}

int kvq_blob_size(const kvq_layout* layout, int32_t n_pos, int64_t* payload_bytes) {
  int st = check_layout(layout);
  if (st) return st;
  if (!payload_bytes) return KVQ_ERR_NULL;
  if (n_pos < 0) return KVQ_ERR_SHAPE;
  *payload_bytes = blob_payload_bytes(*layout, n_pos);
  return KVQ_OK;
}

static int check_blob_range(const kvq_layout& L, int32_t seq, int32_t pos0, int32_t n_pos) {
  if (seq < 0 || pos0 < 0 || n_pos < 0 || (int64_t)pos0 + n_pos > L.max_ctx) return KVQ_ERR_SHAPE;
  if ((int64_t)n_pos * L.n_kv_heads > INT_MAX / 64) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

int kv_cache_pack(const kvq_layout* layout, const void* k_store, const void* v_store, const uint16_t* k_scales,
                  const uint16_t* v_scales, int32_t seq, int32_t pos0, int32_t n_pos, void* dst,
                  int64_t dst_bytes, kvq_blob_header* header, void* stream) {
  int st = check_layout(layout);
  if (st) return st;
  const kvq_layout& L = *layout;
  if ((st = check_store_ptrs(L, L.k_dtype, k_store, k_scales))) return st;
  if ((st = check_store_ptrs(L, L.v_dtype, v_store, v_scales))) return st;
  if (!dst || !header) return KVQ_ERR_NULL;
  if (!aligned(dst, 16)) return KVQ_ERR_ALIGN;
  if ((st = check_blob_range(L, seq, pos0, n_pos))) return st;
  const int64_t bytes = blob_payload_bytes(L, n_pos);
  if (dst_bytes < bytes) return KVQ_ERR_WORKSPACE;
  *header = kvq_blob_header{KVQ_BLOB_MAGIC, KVQ_BLOB_VERSION, L.n_kv_heads, L.head_dim, L.k_dtype, L.v_dtype,
                            L.scale_group, n_pos, bytes};
  if (n_pos == 0) return KVQ_OK;
  return launch_blob(L, const_cast<void*>(k_store), const_cast<void*>(v_store), const_cast<uint16_t*>(k_scales),
                     const_cast<uint16_t*>(v_scales), seq, pos0, n_pos, dst, false, stream);
}

int kv_cache_unpack(const kvq_layout* layout, void* k_store, void* v_store, uint16_t* k_scales, uint16_t* v_scales,
                    int32_t seq, int32_t pos0, const kvq_blob_header* header, const void* src, int64_t src_bytes,
                    void* stream) {
  int st = check_layout(layout);
  if (st) return st;
  const kvq_layout& L = *layout;
  if ((st = check_store_ptrs(L, L.k_dtype, k_store, k_scales))) return st;
  if ((st = check_store_ptrs(L, L.v_dtype, v_store, v_scales))) return st;
  if (!src || !header) return KVQ_ERR_NULL;
  if (!aligned(src, 16)) return KVQ_ERR_ALIGN;
  const kvq_blob_header& h = *header;
  if (h.magic != KVQ_BLOB_MAGIC || h.version != KVQ_BLOB_VERSION || h.n_kv_heads != L.n_kv_heads ||
      h.head_dim != L.head_dim || h.k_dtype != L.k_dtype || h.v_dtype != L.v_dtype ||
      h.scale_group != L.scale_group || h.n_pos < 0 || h.payload_bytes != blob_payload_bytes(L, h.n_pos))
    return KVQ_ERR_MISMATCH;
  if ((st = check_blob_range(L, seq, pos0, h.n_pos))) return st;
  if (src_bytes < h.payload_bytes) return KVQ_ERR_WORKSPACE;
  if (h.n_pos == 0) return KVQ_OK;
  return launch_blob(L, k_store, v_store, k_scales, v_scales, seq, pos0, h.n_pos, const_cast<void*>(src), true,
                     stream);
}

int kvq_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t n_cu, void* stream) {
  if (!buf || !sink) return KVQ_ERR_NULL;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return KVQ_ERR_ALIGN;
  if (bytes < 0 || bytes % 16 || n_cu < 1) return KVQ_ERR_SHAPE;
  if (bytes == 0) return KVQ_OK;
  return launch_stream(buf, bytes, sink, n_cu, stream);
}

int kv_decode_reduce(const kvq_layout* layout, const void* ws, int64_t ws_bytes,
                     const int32_t* d_seq_lens, int32_t batch, int32_t n_q_heads, int32_t window,
                     const kvq_plan_t* plan, uint16_t* out, void* stream) {
  int st = check_layout(layout);
  if (st) return st;
  const kvq_layout& L = *layout;
  if ((st = check_heads(L, batch, n_q_heads))) return st;
  if ((st = check_plan(L, batch, n_q_heads, plan))) return st;
  if (!d_seq_lens || !out) return KVQ_ERR_NULL;
  if (!aligned(d_seq_lens, 4) || !aligned(out, 16)) return KVQ_ERR_ALIGN;
  if (window < 0) return KVQ_ERR_SHAPE;
  if (!ws) return KVQ_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return KVQ_ERR_ALIGN;
  if (ws_bytes < plan->ws_bytes) return KVQ_ERR_WORKSPACE;
  if (batch == 0) return KVQ_OK;
  return launch_reduce(L, ws, batch, n_q_heads, *plan, out, stream);
}

}  // extern "C"
