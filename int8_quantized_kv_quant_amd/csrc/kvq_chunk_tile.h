// Pieces shared by the chunk-attention kernels (int8 and 4-bit stores): the
// transposed fp16 value tile and the per-row online softmax of the O^T layout.
#pragma once

#include <math.h>

#include "kvq_device.h"
#include "kvq_tile.h"

namespace kvq {

constexpr int kChunkStages = 3;

// The fp16 value tile of the chunk kernel is stored transposed: row d holds the
// 32 positions of dim d, position p at slot vt_slot(p), so that the P.V
// contraction index 8*q4 + e (position kpos(e, q4)) is contiguous per lane.
__device__ __forceinline__ int vt_slot(int p) { return 8 * ((p & 15) >> 2) + 4 * (p >> 4) + (p & 3); }
// Bytes per dim row: 32 fp16 and 16 bytes of padding, so that the rows four
// apart that one conversion store writes (and the 16 consecutive rows one
// operand read covers) fall on distinct LDS banks.
constexpr int kVtPitch = 80;

// Accumulators of one block of 16 query rows in the O^T layout: lane (c16, q4)
// holds O^T[dim 16*mt + 4*q4 + i][row c16], i.e. only values of its own row.
template <int D>
struct RowAcc {
  f32x4 o[D / 16];
  f32x4 l;       // the row sum (all four elements equal)
  float m_ref;   // lazily raised reference max of the row (log2 domain)
};

// Online-softmax update of one tile's scores for the lane's own row; returns
// P (fp16) in the B-operand layout of O^T += V_hat^T . P^T.
template <int D>
__device__ __forceinline__ f16x8 row_softmax(const float (&z)[2][4], RowAcc<D>& acc) {
  float tmax = z[0][0];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, z[ct][i]);
  tmax = max_xor16_xor32(tmax);
  const bool need = tmax > acc.m_ref + kTau;
  if (__any(need)) {
    const float m_new = need ? tmax : acc.m_ref;
    const float alpha = need ? __builtin_amdgcn_exp2f(acc.m_ref - m_new) : 1.0f;
    acc.m_ref = m_new;
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) acc.o[mt] *= alpha;
    acc.l *= alpha;
  }
  const float mu = acc.m_ref == -INFINITY ? 0.0f : acc.m_ref;
  f16x8 pa;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) pa[4 * ct + i] = (f16)__builtin_amdgcn_exp2f(z[ct][i] - mu);
  return pa;
}

}  // namespace kvq
