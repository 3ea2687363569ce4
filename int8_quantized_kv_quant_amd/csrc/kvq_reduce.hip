// kv_decode_reduce: combine the split partials of kv_decode_attn_splitk.
//
// genie-ai-runtime releases, v1.3.0 "split-K decode attention": a reduce kernel
// combines the per-split online-softmax partials of each head. Strata PR 2698
// notes the merge cost grows with context, so the merge is spread wide: one
// workgroup per (sequence, query head, 64-dim slice), its 256 lanes reading
// 16 splits x 64 dims per step with 128-bit loads.
//
// For (b, hq) with valid splits s (those whose range starts inside the context):
//   M = max_s m_s;  w_s = 2^(m_s - M);  out = sum_s w_s O_s / sum_s w_s l_s
// (m_s is in the log2 domain, O_s unnormalized), rounded to fp16 (RNE).
#include <math.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

struct ReduceArgs {
  const float* ws_o;
  const float* ws_ml;
  const int32_t* seq_lens;
  uint16_t* out;
  int32_t n_q, n_splits, chunk, window, max_ctx;
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int D>
__global__ __launch_bounds__(256) void kvq_reduce_kernel(ReduceArgs a) {
  const int bh = blockIdx.x;     // b * n_q + hq
  const int slice = blockIdx.y;  // 64-dim slice
  const int b = bh / a.n_q;
  const int tid = threadIdx.x;
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_ctx ? a.max_ctx : L);
  const int lo = a.window > 0 ? max(0, L - a.window) : 0;
  const int n_valid = L > lo ? (int)min((int64_t)a.n_splits, ((int64_t)(L - lo) + a.chunk - 1) / a.chunk) : 0;
  uint16_t* out = a.out + (int64_t)bh * D + slice * 64;
  if (n_valid == 0) {
    if (tid < 64) out[tid] = 0;
    return;
  }
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml) + (int64_t)bh * a.n_splits;
  const float* O = a.ws_o + (int64_t)bh * a.n_splits * D + slice * 64;

  __shared__ float wts[kMaxSplits];
  __shared__ float red[4];
  __shared__ float4 part[16][16];

  float mx = -INFINITY;
  for (int s = tid; s < n_valid; s += 256) mx = fmaxf(mx, ml[s].x);
  mx = wave_max(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float ls = 0.0f;
  for (int s = tid; s < n_valid; s += 256) {
    const float2 v = ml[s];
    const float w = v.x == -INFINITY ? 0.0f : exp2f(v.x - M);
    wts[s] = w;
    ls += w * v.y;
  }
  ls = wave_sum(ls);
  if ((tid & 63) == 0) red[tid >> 6] = ls;
  __syncthreads();
  const float Lsum = (red[0] + red[1]) + (red[2] + red[3]);

  const int sp = tid >> 4;  // split phase 0..15
  const int d4 = tid & 15;  // 4-dim column of the slice
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = sp; s < n_valid; s += 16) {
    const float w = wts[s];
    const float4 v = *reinterpret_cast<const float4*>(O + (int64_t)s * D + 4 * d4);
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
  }
  part[sp][d4] = acc;
  __syncthreads();
  if (tid < 16) {
    float4 t = part[0][tid];
#pragma unroll
    for (int k = 1; k < 16; ++k) {
      const float4 u = part[k][tid];
      t.x += u.x;
      t.y += u.y;
      t.z += u.z;
      t.w += u.w;
    }
    const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
    const f16 r0 = (f16)(t.x * inv), r1 = (f16)(t.y * inv), r2 = (f16)(t.z * inv), r3 = (f16)(t.w * inv);
    u32x2 pk = {(uint32_t)__builtin_bit_cast(uint16_t, r0) | ((uint32_t)__builtin_bit_cast(uint16_t, r1) << 16),
                (uint32_t)__builtin_bit_cast(uint16_t, r2) | ((uint32_t)__builtin_bit_cast(uint16_t, r3) << 16)};
    *reinterpret_cast<u32x2*>(out + 4 * tid) = pk;
  }
}

int launch_reduce(const kvq_layout& L, const void* ws, const int32_t* d_seq_lens, int32_t batch,
                  int32_t n_q_heads, int32_t window, const kvq_plan_t& plan, uint16_t* out,
                  void* stream) {
  ReduceArgs a{};
  const int64_t rows = (int64_t)batch * n_q_heads * plan.n_splits;
  a.ws_o = static_cast<const float*>(ws);
  a.ws_ml = static_cast<const float*>(ws) + rows * L.head_dim;
  a.seq_lens = d_seq_lens;
  a.out = out;
  a.n_q = n_q_heads;
  a.n_splits = plan.n_splits;
  a.chunk = plan.chunk;
  a.window = window;
  a.max_ctx = L.max_ctx > 0x7fffffff ? 0x7fffffff : (int32_t)L.max_ctx;
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
