// kv_decode_reduce: combine the split partials of kv_decode_attn_splitk.
//
// genie-ai-runtime releases, v1.3.0 "split-K decode attention": a reduce kernel
// combines the per-split online-softmax partials of each head. Strata PR 2698
// notes the merge cost grows with context, so the merge is spread wide: one
// workgroup per (sequence, query head, slice of 16, 32 or 64 dims).
//
// For (b, hq) over its splits s:
//   M = max_s m_s;  w_s = 2^(m_s - M);  out = sum_s w_s O_s / sum_s w_s l_s
// (m_s is in the log2 domain, O_s unnormalized), rounded to fp16 (RNE). The
// partial kernel records every split, an empty one as (m, l) = (-inf, 0) with
// its O left unwritten, so this kernel needs no context lengths: a split with
// m = -inf contributes nothing and its O is never used in arithmetic. A head
// whose splits are all empty (context length 0) gets an all-zero row.
//
// Latency, not bandwidth, bounds this kernel (a few MB in total, and at batch
// 1 only n_q_heads rows), so the work is spread over many lanes: a workgroup
// covers SLICE dims of one (b, hq) row; lane (column c, split phase p) folds the
// splits p, p + P, ... of its 4-dim column into a running (max, sum, output)
// triple, issuing a batch of loads at once; the P phases of a column are P
// consecutive lanes of one wavefront: they take the column's maximum, rescale
// their own triple to it and add up (sum, output) by butterflies of
// register-only lane exchanges (DPP moves and permlane swaps: no LDS, no
// barrier, no exponential per level). Narrow slices give small batches many
// workgroups.
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

constexpr int kReduceBatch = 8;  // splits per lane per round of loads

struct Triple {
  float m, l;
  float4 o;
};

// Maximum and sum over the P consecutive lanes (16, 32 or 64) of a group:
// every lane of the group gets the result (each level adds the same two
// operands on both sides of the exchange, so the lanes agree bit for bit).
template <int P>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (P >= 64) {
    const float2 t = lane_pair<32>(x);
    x = fmaxf(t.x, t.y);
  }
  if constexpr (P >= 32) {
    const float2 t = lane_pair<16>(x);
    x = fmaxf(t.x, t.y);
  }
  x = fmaxf(x, lane_xor<8>(x));
  x = fmaxf(x, lane_xor<4>(x));
  x = fmaxf(x, lane_xor<2>(x));
  return fmaxf(x, lane_xor<1>(x));
}
template <int P>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (P >= 64) {
    const float2 t = lane_pair<32>(x);
    x = t.x + t.y;
  }
  if constexpr (P >= 32) {
    const float2 t = lane_pair<16>(x);
    x = t.x + t.y;
  }
  x = x + lane_xor<8>(x);
  x = x + lane_xor<4>(x);
  x = x + lane_xor<2>(x);
  return x + lane_xor<1>(x);
}

template <int D, int SLICE>
__global__ __launch_bounds__(256) void kvq_reduce_kernel(ReduceArgs a) {
  constexpr int C = SLICE / 4;  // 4-dim columns per workgroup
  constexpr int P = 256 / C;    // split phases per column (16, 32 or 64 lanes)
  const int bh = blockIdx.x;    // b * n_q + hq
  const int slice = blockIdx.y;
  const int tid = threadIdx.x;
  const int p = tid % P;
  const int c = tid / P;
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml) + (int64_t)bh * a.n_splits;
  const float* O = a.ws_o + (int64_t)bh * a.n_splits * D + slice * SLICE + 4 * c;

  Triple run = {-INFINITY, 0.0f, make_float4(0.f, 0.f, 0.f, 0.f)};
  for (int base = p; base < a.n_splits; base += P * kReduceBatch) {
    float2 v[kReduceBatch];
    float4 o[kReduceBatch];
#pragma unroll
    for (int k = 0; k < kReduceBatch; ++k) {
      const int s = base + P * k;
      v[k] = make_float2(-INFINITY, 0.0f);
      o[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (s < a.n_splits) {
        v[k] = ml[s];
        o[k] = *reinterpret_cast<const float4*>(O + (int64_t)s * D);
      }
    }
    float bm = run.m;
#pragma unroll
    for (int k = 0; k < kReduceBatch; ++k) bm = fmaxf(bm, v[k].x);
    if (bm == -INFINITY) continue;  // nothing recorded yet
    // An empty split (m = -inf) has its O row unwritten: it must not enter the
    // arithmetic, so it is skipped rather than weighted by 0.
    const float r = run.m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(run.m - bm);
    run.l *= r;
    run.o.x *= r;
    run.o.y *= r;
    run.o.z *= r;
    run.o.w *= r;
    run.m = bm;
#pragma unroll
    for (int k = 0; k < kReduceBatch; ++k) {
      if (v[k].x != -INFINITY) {
        const float w = __builtin_amdgcn_exp2f(v[k].x - bm);
        run.l = fmaf(w, v[k].y, run.l);
        run.o.x = fmaf(w, o[k].x, run.o.x);
        run.o.y = fmaf(w, o[k].y, run.o.y);
        run.o.z = fmaf(w, o[k].z, run.o.z);
        run.o.w = fmaf(w, o[k].w, run.o.w);
      }
    }
  }

  // The column's maximum over its P lanes, every lane's triple rescaled to it
  // (an empty lane, m = -inf, contributes 0), then the sums.
  const float M = group_max<P>(run.m);
  const float w = run.m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(run.m - M);
  run.l = group_sum<P>(w * run.l);
  run.o.x = group_sum<P>(w * run.o.x);
  run.o.y = group_sum<P>(w * run.o.y);
  run.o.z = group_sum<P>(w * run.o.z);
  run.o.w = group_sum<P>(w * run.o.w);
  if (p == 0) {
    const float inv = run.l > 0.0f ? 1.0f / run.l : 0.0f;
    const f16 r0 = (f16)(run.o.x * inv), r1 = (f16)(run.o.y * inv), r2 = (f16)(run.o.z * inv),
              r3 = (f16)(run.o.w * inv);
    u32x2 pk = {(uint32_t)__builtin_bit_cast(uint16_t, r0) | ((uint32_t)__builtin_bit_cast(uint16_t, r1) << 16),
                (uint32_t)__builtin_bit_cast(uint16_t, r2) | ((uint32_t)__builtin_bit_cast(uint16_t, r3) << 16)};
    *reinterpret_cast<u32x2*>(a.out + (int64_t)bh * D + slice * SLICE + 4 * c) = pk;
  }
}

// Few splits (n_splits <= P, P = 1, 2 or 4): a workgroup covers whole rows,
// lane (row, 4-dim column, split phase p) loads split p of its column, and the
// P phases (consecutive lanes) combine as in kvq_reduce_kernel. With one split
// this is the normalization out = O / l, one float4 per lane.
template <int D, int P>
__global__ __launch_bounds__(256) void kvq_reduce_few_kernel(ReduceArgs a, int64_t rows) {
  constexpr int C = D / 4;            // 4-dim columns per row
  constexpr int R = 256 / (C * P);    // rows per workgroup
  static_assert(R >= 1 && R * C * P == 256, "reduce tiling");
  const int tid = threadIdx.x;
  const int p = tid % P;
  const int c = (tid / P) % C;
  const int64_t bh = (int64_t)blockIdx.x * R + tid / (P * C);
  if (bh >= rows) return;  // whole P-groups leave together, so the butterfly below stays closed
  Triple run = {-INFINITY, 0.0f, make_float4(0.f, 0.f, 0.f, 0.f)};
  if (p < a.n_splits) {
    const float2 v = reinterpret_cast<const float2*>(a.ws_ml)[bh * a.n_splits + p];
    if (v.x != -INFINITY) {  // an empty split's O row was never written
      run.m = v.x;
      run.l = v.y;
      run.o = *reinterpret_cast<const float4*>(a.ws_o + (bh * a.n_splits + p) * D + 4 * c);
    }
  }
  if constexpr (P > 1) {  // the P phases: max, rescale, sums (as in kvq_reduce_kernel)
    float M = fmaxf(run.m, lane_xor<1>(run.m));
    if constexpr (P > 2) M = fmaxf(M, lane_xor<2>(M));
    const float w = run.m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(run.m - M);
    float r[5] = {w * run.l, w * run.o.x, w * run.o.y, w * run.o.z, w * run.o.w};
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      r[k] = r[k] + lane_xor<1>(r[k]);
      if constexpr (P > 2) r[k] = r[k] + lane_xor<2>(r[k]);
    }
    run.l = r[0];
    run.o = make_float4(r[1], r[2], r[3], r[4]);
  }
  if (p == 0) {
    // out = O / l with O and l taken at the same reference
    const float inv = run.l > 0.0f ? 1.0f / run.l : 0.0f;
    const f16 r0 = (f16)(run.o.x * inv), r1 = (f16)(run.o.y * inv), r2 = (f16)(run.o.z * inv),
              r3 = (f16)(run.o.w * inv);
    u32x2 pk = {(uint32_t)__builtin_bit_cast(uint16_t, r0) | ((uint32_t)__builtin_bit_cast(uint16_t, r1) << 16),
                (uint32_t)__builtin_bit_cast(uint16_t, r2) | ((uint32_t)__builtin_bit_cast(uint16_t, r3) << 16)};
    *reinterpret_cast<u32x2*>(a.out + bh * D + 4 * c) = pk;
  }
}

template <int D>
static void launch_reduce_d(const ReduceArgs& a, int64_t rows, hipStream_t s) {
  // One to four splits: whole rows per workgroup.
  if (a.n_splits <= 4) {
    const int P = a.n_splits == 1 ? 1 : (a.n_splits == 2 ? 2 : 4);
    const int64_t R = 256 / ((D / 4) * P);
    const dim3 grid((unsigned)((rows + R - 1) / R));
    if (P == 1) hipLaunchKernelGGL((kvq_reduce_few_kernel<D, 1>), grid, dim3(256), 0, s, a, rows);
    else if (P == 2) hipLaunchKernelGGL((kvq_reduce_few_kernel<D, 2>), grid, dim3(256), 0, s, a, rows);
    else hipLaunchKernelGGL((kvq_reduce_few_kernel<D, 4>), grid, dim3(256), 0, s, a, rows);
    return;
  }
  // Narrower slices (more split phases per column) when there are few (b, hq)
  // rows and more than one split per lane at 16 phases, so that the grid still
  // spreads over the chip and each lane waits on few loads; with at most 16
  // splits the longer butterfly of a narrow slice would cost more than it saves.
  if (a.n_splits <= 16 || rows * (D / 64) >= 256) {
    hipLaunchKernelGGL((kvq_reduce_kernel<D, 64>), dim3(rows, D / 64), dim3(256), 0, s, a);
  } else if (rows * (D / 32) >= 256) {
    hipLaunchKernelGGL((kvq_reduce_kernel<D, 32>), dim3(rows, D / 32), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((kvq_reduce_kernel<D, 16>), dim3(rows, D / 16), dim3(256), 0, s, a);
  }
}

int launch_reduce(const kvq_layout& L, const void* ws, int32_t batch, int32_t n_q_heads,
                  const kvq_plan_t& plan, uint16_t* out, void* stream) {
  ReduceArgs a{};
  const int64_t bh = (int64_t)batch * n_q_heads;
  const int64_t rows = bh * plan.n_splits;
  a.ws_o = static_cast<const float*>(ws);
  a.ws_ml = static_cast<const float*>(ws) + rows * L.head_dim;
  a.out = out;
  a.n_splits = plan.n_splits;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (L.head_dim) {
    case 64: launch_reduce_d<64>(a, bh, s); break;
    case 128: launch_reduce_d<128>(a, bh, s); break;
    case 256: launch_reduce_d<256>(a, bh, s); break;
    default: return KVQ_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace kvq
