// kv_decode_reduce: combine the split partials of kv_decode_attn_splitk.
//
// genie-ai-runtime releases, v1.3.0 "split-K decode attention": a reduce kernel
// combines the per-split online-softmax partials of each head. Strata PR 2698
// notes the merge cost grows with context, so the merge is spread wide: one
// workgroup per (sequence, query head, 64-dim slice).
//
// For (b, hq) over its splits s:
//   M = max_s m_s;  w_s = 2^(m_s - M);  out = sum_s w_s O_s / sum_s w_s l_s
// (m_s is in the log2 domain, O_s unnormalized), rounded to fp16 (RNE). The
// partial kernel records every split, an empty one as (m, l) = (-inf, 0) with
// its O left unwritten, so this kernel needs no context lengths: a split with
// m = -inf contributes nothing and its O is never used in arithmetic. A head
// whose splits are all empty (context length 0) gets an all-zero row.
//
// Latency, not bandwidth, bounds this kernel (a few MB in total), so each lane
// issues all loads of a batch of splits at once and folds them into a running
// (max, sum, output) triple; the 16 lanes that share a 4-dim column then merge
// their triples through LDS.
#include <math.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

struct ReduceArgs {
  const float* ws_o;
  const float* ws_ml;
  uint16_t* out;
  int32_t n_splits;
};

constexpr int kReduceBatch = 16;  // splits per lane per round of loads (256 splits: one round)

template <int D>
__global__ __launch_bounds__(256) void kvq_reduce_kernel(ReduceArgs a) {
  const int bh = blockIdx.x;     // b * n_q + hq
  const int slice = blockIdx.y;  // 64-dim slice
  const int tid = threadIdx.x;
  const int sp = tid >> 4;       // split phase 0..15: splits sp, sp + 16, ...
  const int d4 = tid & 15;       // 4-dim column of the slice
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml) + (int64_t)bh * a.n_splits;
  const float* O = a.ws_o + (int64_t)bh * a.n_splits * D + slice * 64 + 4 * d4;

  float m_run = -INFINITY, l_run = 0.0f;
  float4 o_run = {0.f, 0.f, 0.f, 0.f};
  for (int base = sp; base < a.n_splits; base += 16 * kReduceBatch) {
    float2 v[kReduceBatch];
    float4 o[kReduceBatch];
#pragma unroll
    for (int k = 0; k < kReduceBatch; ++k) {
      const int s = base + 16 * k;
      v[k] = make_float2(-INFINITY, 0.0f);
      o[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (s < a.n_splits) {
        v[k] = ml[s];
        o[k] = *reinterpret_cast<const float4*>(O + (int64_t)s * D);
      }
    }
    float bm = m_run;
#pragma unroll
    for (int k = 0; k < kReduceBatch; ++k) bm = fmaxf(bm, v[k].x);
    if (bm == -INFINITY) continue;  // nothing recorded yet
    const float r = m_run == -INFINITY ? 0.0f : exp2f(m_run - bm);
    l_run *= r;
    o_run.x *= r;
    o_run.y *= r;
    o_run.z *= r;
    o_run.w *= r;
    m_run = bm;
#pragma unroll
    for (int k = 0; k < kReduceBatch; ++k) {
      if (v[k].x != -INFINITY) {
        const float w = exp2f(v[k].x - bm);
        l_run = fmaf(w, v[k].y, l_run);
        o_run.x = fmaf(w, o[k].x, o_run.x);
        o_run.y = fmaf(w, o[k].y, o_run.y);
        o_run.z = fmaf(w, o[k].z, o_run.z);
        o_run.w = fmaf(w, o[k].w, o_run.w);
      }
    }
  }

  __shared__ float4 part_o[16][16];
  __shared__ float part_m[16][16];
  __shared__ float part_l[16][16];
  part_o[sp][d4] = o_run;
  part_m[sp][d4] = m_run;
  part_l[sp][d4] = l_run;
  __syncthreads();
  if (tid < 16) {
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < 16; ++k) M = fmaxf(M, part_m[k][tid]);
    float4 t = {0.f, 0.f, 0.f, 0.f};
    float l = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float mk = part_m[k][tid];
        if (mk != -INFINITY) {
          const float w = exp2f(mk - M);
          const float4 u = part_o[k][tid];
          l = fmaf(w, part_l[k][tid], l);
          t.x = fmaf(w, u.x, t.x);
          t.y = fmaf(w, u.y, t.y);
          t.z = fmaf(w, u.z, t.z);
          t.w = fmaf(w, u.w, t.w);
        }
      }
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const f16 r0 = (f16)(t.x * inv), r1 = (f16)(t.y * inv), r2 = (f16)(t.z * inv), r3 = (f16)(t.w * inv);
    u32x2 pk = {(uint32_t)__builtin_bit_cast(uint16_t, r0) | ((uint32_t)__builtin_bit_cast(uint16_t, r1) << 16),
                (uint32_t)__builtin_bit_cast(uint16_t, r2) | ((uint32_t)__builtin_bit_cast(uint16_t, r3) << 16)};
    *reinterpret_cast<u32x2*>(a.out + (int64_t)bh * D + slice * 64 + 4 * tid) = pk;
  }
}

int launch_reduce(const kvq_layout& L, const void* ws, int32_t batch, int32_t n_q_heads,
                  const kvq_plan_t& plan, uint16_t* out, void* stream) {
  ReduceArgs a{};
  const int64_t rows = (int64_t)batch * n_q_heads * plan.n_splits;
  a.ws_o = static_cast<const float*>(ws);
  a.ws_ml = static_cast<const float*>(ws) + rows * L.head_dim;
  a.out = out;
  a.n_splits = plan.n_splits;
  dim3 grid(batch * n_q_heads, L.head_dim / 64);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (L.head_dim) {
    case 64: hipLaunchKernelGGL(kvq_reduce_kernel<64>, grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(kvq_reduce_kernel<128>, grid, dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(kvq_reduce_kernel<256>, grid, dim3(256), 0, s, a); break;
    default: return KVQ_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace kvq
