// Device helpers of the 4-bit stores: the 256-point Walsh-Hadamard rotation of
// one row held by a whole wavefront (4 values per lane) and the Q4_0 block
// quantizer of the rotated row.
//
// Strata PR 2698, "Not in this PR": q4_0 and k8v4 use a Hadamard rotation over
// head_dim 256 with Q4_0 blocks; K is rotated together with the queries, V is
// rotated and the output rotated back. Q4_0 is the published 4-bit block
// format: 32 values share one fp16 scale d = (value of largest magnitude) / -8,
// codes q = min(15, trunc(x / d + 8.5)) stand for (q - 8) * d.
#pragma once

#include "kvq_device.h"

namespace kvq {

// One butterfly stage of fwht256 between lanes l and l ^ M (elements 4M
// apart): the lower element keeps a + b, the upper one a - b, each as
// fma(+-1, b, a) or fma(+-1, own, partner) with an exact product, so it rounds
// exactly as the sum or the difference.
template <int M>
__device__ __forceinline__ void fwht_stage(float (&v)[4], int lane) {
  const float sgn = (lane & M) ? -1.0f : 1.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if constexpr (M < 16) {
      v[k] = fmaf(sgn, v[k], lane_xor<M>(v[k]));
    } else {
      const float2 ab = lane_pair<M>(v[k]);  // (a, b): the lower and the upper lane's value
      v[k] = fmaf(sgn, ab.y, ab.x);
    }
  }
}

// y = H x / 16 for the 256 values of one row, lane l holding elements
// 4l .. 4l+3 in v[0..3] (all 64 lanes of the wavefront take part). fp32
// butterflies (a, b) -> (a + b, a - b) over index pairs at distance 1, 2, 4,
// ..., 128, in that order, then * 1/16 (exact): every step is one correctly
// rounded fp32 addition or subtraction, so the result does not depend on how
// the pairs are assigned to lanes. The lane exchanges are DPP moves and
// permlane swaps (registers only).
__device__ __forceinline__ void fwht256(float (&v)[4], int lane) {
#pragma clang fp contract(off)
  float a = v[0] + v[1], b = v[0] - v[1], c = v[2] + v[3], d = v[2] - v[3];
  v[0] = a + c;
  v[2] = a - c;
  v[1] = b + d;
  v[3] = b - d;
  fwht_stage<1>(v, lane);
  fwht_stage<2>(v, lane);
  fwht_stage<4>(v, lane);
  fwht_stage<8>(v, lane);
  fwht_stage<16>(v, lane);
  fwht_stage<32>(v, lane);
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] *= 0.0625f;
}

// Q4_0 quantization of a rotated row held as by fwht256: lanes 8k .. 8k+7 hold
// block k (32 values). Returns, for lanes with (lane & 7) < 4, the dword of
// the block's bytes 4 * (lane & 7) .. +3 (byte j = code j | code (j+16) << 4);
// *scale_bits gets the block's fp16 scale (every lane of the block) and, if
// given, *own the lane's 4 codes (byte k = code of y[k]).
//   m: the value of largest magnitude, the first one on ties;
//   d = m * -0.125 (= m / -8, exact), r = 1/d correctly rounded (0 if d = 0);
//   q = min(15, trunc(fp32(fp32(y * r) + 8.5))), no fused multiply-add.
__device__ __forceinline__ uint32_t q4_quantize(const float (&y)[4], int lane, uint16_t* scale_bits,
                                                uint32_t* own = nullptr) {
#pragma clang fp contract(off)  // y * r and + 8.5 are two roundings, as in the published quantizer
  const int lb = lane & 7;
  float am = fabsf(y[0]), m = y[0];
  int idx = 4 * lb;
#pragma unroll
  for (int k = 1; k < 4; ++k)
    if (fabsf(y[k]) > am) {
      am = fabsf(y[k]);
      m = y[k];
      idx = 4 * lb + k;
    }
  auto take = [&](float pam, float pm, int pidx) {
    if (pam > am || (pam == am && pidx < idx)) {
      am = pam;
      m = pm;
      idx = pidx;
    }
  };
  take(lane_xor<1>(am), lane_xor<1>(m), lane_xor<1>(idx));
  take(lane_xor<2>(am), lane_xor<2>(m), lane_xor<2>(idx));
  take(lane_xor<4>(am), lane_xor<4>(m), lane_xor<4>(idx));
  const float d = m * -0.125f;
  const float r = d != 0.0f ? __fdiv_rn(1.0f, d) : 0.0f;
  uint32_t codes = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float t = y[k] * r + 8.5f;  // not contracted (pragma above)
    codes |= (uint32_t)min(15, (int)t) << (8 * k);
  }
  *scale_bits = __builtin_bit_cast(uint16_t, (f16)d);
  if (own) *own = codes;
  const uint32_t hi = lane_xor_u32<4>(codes);  // codes of values 16 + 4 * (lane & 3) + k
  return codes | (hi << 4);
}

}  // namespace kvq
