// kv_quant_append: quantize new K/V rows into the cache.
//
// genie-ai-runtime v0.1.0-alpha.12, "Path I series" #64: per-head conversion
// with scale capture (one scale per position and kv head). Strata PR 2698,
// "What it does": each 64-value group shares an FP16 scale, its absmax / 127;
// k8v32 / k32v8 quantize only one of the stores.
//
// Work mapping: each lane owns 4 consecutive elements of a row, so a row of
// head_dim values spans head_dim/4 lanes (16, 32 or 64) and a wavefront carries
// 4, 2 or 1 rows. A 64-value scale group is 16 lanes; a per-row group is the
// whole row. The group absmax is a butterfly max over those lanes.
//
// Arithmetic: quantize4 (kvq_device.h), bit-exact with the CPU definition.
//
// A q4 store (head_dim 256, Strata PR 2698 "Not in this PR"): the row's
// wavefront rotates it (fwht256) and quantizes each 32-value block to Q4_0
// (q4_quantize, kvq_q4.h); lanes 8k .. 8k+3 write block k's 16 bytes and lane
// 8k its fp16 scale.
#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_q4.h"

namespace kvq {

struct AppendStore {
  void* store;
  uint16_t* scales;
  const uint16_t* src;
  int32_t dtype;  // KVQ_STORE_*
  int32_t pad_;
};

struct AppendArgs {
  AppendStore st[2];  // [0] = K, [1] = V
  const int32_t* start_pos;
  int64_t s_seq, s_pos, s_head;
  int64_t ss_seq, ss_pos, ss_head;
  int64_t max_ctx;
  int32_t n_kv, n_tok, rows;  // rows = batch * n_tok * n_kv
  int32_t group_lanes;        // lanes sharing one scale (power of two)
};

template <int D>
__global__ __launch_bounds__(256) void kvq_append_kernel(AppendArgs a) {
  constexpr int TPR = D / 4;      // lanes per row
  constexpr int RPB = 256 / TPR;  // rows per block
  const AppendStore S = a.st[blockIdx.y];
  const int lr = threadIdx.x % TPR;
  const int row = blockIdx.x * RPB + threadIdx.x / TPR;
  // Rows, and so scale groups, never straddle this exit: whole groups leave together.
  if (row >= a.rows) return;
  const int h = row % a.n_kv;
  const int t = (row / a.n_kv) % a.n_tok;
  const int b = row / (a.n_kv * a.n_tok);
  // The row's values and its position are fetched together (neither waits for
  // the other).
  const u32x2 raw = *reinterpret_cast<const u32x2*>(S.src + (int64_t)row * D + 4 * lr);
  const int64_t pos = (int64_t)a.start_pos[b] + t;
  if (pos < 0 || pos >= a.max_ctx) return;

  const uint32_t hb[4] = {raw.x & 0xffffu, raw.x >> 16, raw.y & 0xffffu, raw.y >> 16};
  const int64_t row_off = b * a.s_seq + pos * a.s_pos + h * a.s_head;

  if (S.dtype == KVQ_STORE_Q4) {
    if constexpr (D == 256) {  // one row per wavefront (TPR == 64)
      float y[4] = {h_bits_to_f32(hb[0]), h_bits_to_f32(hb[1]), h_bits_to_f32(hb[2]), h_bits_to_f32(hb[3])};
      fwht256(y, lr);
      uint16_t scale_bits;
      const uint32_t packed = q4_quantize(y, lr, &scale_bits);
      if ((lr & 7) < 4)
        *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(S.store) + row_off / 2 + 16 * (lr >> 3) + 4 * (lr & 7)) =
            packed;
      if ((lr & 7) == 0) S.scales[b * a.ss_seq + pos * a.ss_pos + h * a.ss_head + (lr >> 3)] = scale_bits;
    }
    return;
  }
  if (S.dtype == KVQ_STORE_FP32) {
    // fp32 store: the fp16 values widened exactly.
    float4 v = {h_bits_to_f32(hb[0]), h_bits_to_f32(hb[1]), h_bits_to_f32(hb[2]), h_bits_to_f32(hb[3])};
    *reinterpret_cast<float4*>(static_cast<float*>(S.store) + row_off + 4 * lr) = v;
    return;
  }

  uint16_t scale_bits;  // a scale group is 16 lanes (64 values) or the whole row
  const uint32_t packed = a.group_lanes == 16 ? quantize4<16>(hb, &scale_bits) : quantize4<TPR>(hb, &scale_bits);
  *reinterpret_cast<uint32_t*>(static_cast<int8_t*>(S.store) + row_off + 4 * lr) = packed;
  if (lr % a.group_lanes == 0) {
    const int64_t soff = b * a.ss_seq + pos * a.ss_pos + h * a.ss_head + lr / a.group_lanes;
    S.scales[soff] = scale_bits;
  }
}

// ---- int8 and fp32 stores: 8 values per lane ---------------------------------------
// Lane l of a wavefront owns values 8 (l % LPR) .. +7 of row l / LPR, LPR = D / 8
// lanes per row (32, 16, 8): one 16-byte load per lane, RW = 64 / LPR rows per
// wavefront. A workgroup (4 wavefronts) covers 4 RW consecutive tokens of one
// kv head and one sequence, so the token and head of a row come from the grid
// (no division per lane). The group absmax and the codes: group_max and code_of
// (kvq_device.h).

struct Append8Args {
  AppendStore st[2];  // [0] = K, [1] = V
  const int32_t* start_pos;
  int64_t s_seq, s_pos, s_head;
  int64_t ss_seq, ss_pos, ss_head;
  int64_t max_ctx;
  int32_t n_kv, n_tok;
};

template <int D, bool G64>
__global__ __launch_bounds__(256) void kvq_append8_kernel(Append8Args a) {
  constexpr int LPR = D / 8;               // lanes per row
  constexpr int RW = 64 / LPR;             // rows per wavefront
  constexpr int GL = G64 ? 8 : LPR;        // lanes per scale group
  const AppendStore S = a.st[blockIdx.y];
  const int b = blockIdx.z;
  const int h = blockIdx.x % a.n_kv;       // uniform: scalar arithmetic
  const int tb = blockIdx.x / a.n_kv;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int t = (tb * 4 + wv) * RW + lane / LPR;
  const int lr = lane % LPR;
  const bool live = t < a.n_tok;
  u32x4 raw = {0u, 0u, 0u, 0u};
  if (live) raw = *reinterpret_cast<const u32x4*>(S.src + (((int64_t)b * a.n_tok + t) * a.n_kv + h) * D + 8 * lr);
  const int64_t pos = (int64_t)a.start_pos[b] + t;
  const bool store = live && pos >= 0 && pos < a.max_ctx;  // rows outside the cache are dropped
  const int64_t row_off = b * a.s_seq + pos * a.s_pos + h * a.s_head;
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = h_bits_to_f32((raw[e >> 1] >> (16 * (e & 1))) & 0xffffu);

  if (S.dtype == KVQ_STORE_FP32) {  // the fp16 values widened exactly
    if (store) {
      float4* dst = reinterpret_cast<float4*>(static_cast<float*>(S.store) + row_off + 8 * lr);
      dst[0] = make_float4(x[0], x[1], x[2], x[3]);
      dst[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
    return;
  }
  // absmax on the fp16 bit patterns (exact), over the group's lanes
  uint32_t amax = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) amax = max(amax, max(raw[k] & 0x7fffu, (raw[k] >> 16) & 0x7fffu));
  amax = group_max<GL>(amax);
  const f16 scale_h = (f16)(h_bits_to_f32(amax) / 127.0f);  // fp32 IEEE division, then fp16 RNE
  const float s = (float)scale_h;
  const float rs = __builtin_amdgcn_rcpf(s);
  uint32_t w[2] = {0u, 0u};
  if (s > 0.0f) {
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e >> 2] |= ((uint32_t)code_of(x[e], s, rs) & 0xffu) << (8 * (e & 3));
  }
  if (store) {
    *reinterpret_cast<u32x2*>(static_cast<int8_t*>(S.store) + row_off + 8 * lr) = (u32x2){w[0], w[1]};
    if (lr % GL == 0) S.scales[b * a.ss_seq + pos * a.ss_pos + h * a.ss_head + lr / GL] = __builtin_bit_cast(uint16_t, scale_h);
  }
}

template <int D>
static void launch_append8_t(const Append8Args& a, bool g64, dim3 grid, hipStream_t s) {
  if (g64) hipLaunchKernelGGL((kvq_append8_kernel<D, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((kvq_append8_kernel<D, false>), grid, dim3(256), 0, s, a);
}

int launch_append(const kvq_layout& L, void* k_store, void* v_store, uint16_t* k_scales,
                  uint16_t* v_scales, const uint16_t* k_new, const uint16_t* v_new,
                  const int32_t* d_start_pos, int32_t batch, int32_t n_tok, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!has_q4(L)) {
    Append8Args a{};
    a.st[0] = {k_store, k_scales, k_new, L.k_dtype, 0};
    a.st[1] = {v_store, v_scales, v_new, L.v_dtype, 0};
    a.start_pos = d_start_pos;
    a.s_seq = L.s_seq;
    a.s_pos = L.s_pos;
    a.s_head = L.s_head;
    a.ss_seq = L.ss_seq;
    a.ss_pos = L.ss_pos;
    a.ss_head = L.ss_head;
    a.max_ctx = L.max_ctx;
    a.n_kv = L.n_kv_heads;
    a.n_tok = n_tok;
    const int tok_per_wg = 4 * (64 / (L.head_dim / 8));
    const dim3 grid(L.n_kv_heads * ((n_tok + tok_per_wg - 1) / tok_per_wg), 2, batch);
    const bool g64 = L.scale_group == 64 && L.head_dim != 64;
    switch (L.head_dim) {
      case 64: launch_append8_t<64>(a, g64, grid, s); break;
      case 128: launch_append8_t<128>(a, g64, grid, s); break;
      case 256: launch_append8_t<256>(a, g64, grid, s); break;
      default: return KVQ_ERR_UNSUPPORTED;
    }
    return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
  }
  // Layouts with a q4 store: one row per wavefront (the rotation spans it).
  AppendArgs a{};
  a.st[0] = {k_store, k_scales, k_new, L.k_dtype, 0};
  a.st[1] = {v_store, v_scales, v_new, L.v_dtype, 0};
  a.start_pos = d_start_pos;
  a.s_seq = L.s_seq;
  a.s_pos = L.s_pos;
  a.s_head = L.s_head;
  a.ss_seq = L.ss_seq;
  a.ss_pos = L.ss_pos;
  a.ss_head = L.ss_head;
  a.max_ctx = L.max_ctx;
  a.n_kv = L.n_kv_heads;
  a.n_tok = n_tok;
  a.rows = batch * n_tok * L.n_kv_heads;
  const int tpr = L.head_dim / 4;
  a.group_lanes = (L.scale_group == 64) ? 16 : tpr;
  const int rpb = 256 / tpr;
  dim3 grid((a.rows + rpb - 1) / rpb, 2);
  switch (L.head_dim) {
    case 64: hipLaunchKernelGGL(kvq_append_kernel<64>, grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(kvq_append_kernel<128>, grid, dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(kvq_append_kernel<256>, grid, dim3(256), 0, s, a); break;
    default: return KVQ_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace kvq
