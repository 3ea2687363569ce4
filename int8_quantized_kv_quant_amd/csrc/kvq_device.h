// Device helpers for the gfx950 kernels of libkvq: vector types, bounds-checked
// buffer loads and the int8 -> fp16 operand construction used by the MFMA path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Resource word 3 of a raw (stride 0) buffer on gfx9-class GPUs: 32-bit data
// format, bounds checked against num_records.
constexpr uint32_t kBufWord3 = 0x00020000u;
// A byte offset that is outside every buffer this library builds (their
// num_records never exceed INT_MAX): loads from it return zeros.
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kBufWord3);
}

__device__ __forceinline__ u32x4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ u32x2 ld64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t ld32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}

__device__ __forceinline__ f16x2 as_h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ uint32_t as_u32(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ float h_bits_to_f32(uint32_t bits) {
  return (float)__builtin_bit_cast(f16, (uint16_t)bits);
}

// int8 codes -> fp16 without arithmetic. A code c (two's complement byte) XOR
// 0x80 is the unsigned byte c + 128; placing 0x64 above it gives the fp16 bit
// pattern of 1024 + (c + 128) = 1152 + c, exact for every byte value.
constexpr uint32_t kCodeFlip = 0x80808080u;
constexpr float kCodeBias = 1152.0f;
// Bytes 0 and 1 of a flipped dword as two biased fp16 values.
__device__ __forceinline__ uint32_t biased_h2_lo(uint32_t flipped) {
  return __builtin_amdgcn_perm(0x64646464u, flipped, 0x04010400u);
}
// Bytes 2 and 3 of a flipped dword as two biased fp16 values.
__device__ __forceinline__ uint32_t biased_h2_hi(uint32_t flipped) {
  return __builtin_amdgcn_perm(0x64646464u, flipped, 0x04030402u);
}
// Interleave bytes 0,1 (sel01) or 2,3 (sel23) of two dwords: [b.x, a.x, b.y, a.y].
__device__ __forceinline__ uint32_t zip_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(a, b, 0x05010400u);
}
__device__ __forceinline__ uint32_t zip_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(a, b, 0x07030602u);
}

// Eight biased fp16 values (1152 + code) from two dwords of codes.
__device__ __forceinline__ f16x8 codes8_biased(uint32_t d0, uint32_t d1) {
  d0 ^= kCodeFlip;
  d1 ^= kCodeFlip;
  u32x4 r = {biased_h2_lo(d0), biased_h2_hi(d0), biased_h2_lo(d1), biased_h2_hi(d1)};
  return __builtin_bit_cast(f16x8, r);
}

// Eight fp16 values from eight fp32 values that are exactly representable in
// fp16 (the fp32 store holds widened fp16 data), so truncation is exact.
__device__ __forceinline__ f16x8 f32x8_to_f16x8(u32x4 a, u32x4 b) {
  auto cv = [](uint32_t x, uint32_t y) {
    return as_u32(__builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(__builtin_bit_cast(float, x),
                                                                      __builtin_bit_cast(float, y))));
  };
  u32x4 r = {cv(a.x, a.y), cv(a.z, a.w), cv(b.x, b.y), cv(b.z, b.w)};
  return __builtin_bit_cast(f16x8, r);
}

// ---- cross-lane exchanges in registers (no LDS round trip) -----------------------
// The value of lane l ^ M (M = 1, 2, 4, 8) by DPP moves, each a gather from
// one lane: quad permutations give l ^ 1, l ^ 2 and l ^ 3, the half-row mirror
// l ^ 7 (within 8 lanes) and the row mirror l ^ 15 (within 16); l ^ 4 is
// (l ^ 7) ^ 3 and l ^ 8 is (l ^ 15) ^ 7.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
template <int M>
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t x) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8, "DPP lane exchange");
  if constexpr (M == 1) return dpp_u32<0xB1>(x);        // quad_perm [1,0,3,2]
  else if constexpr (M == 2) return dpp_u32<0x4E>(x);   // quad_perm [2,3,0,1]
  else if constexpr (M == 4) return dpp_u32<0x1B>(dpp_u32<0x141>(x));  // half-row mirror, quad_perm [3,2,1,0]
  else return dpp_u32<0x141>(dpp_u32<0x140>(x));        // row mirror, half-row mirror
}
template <int M>
__device__ __forceinline__ float lane_xor(float x) {
  return __builtin_bit_cast(float, lane_xor_u32<M>(__builtin_bit_cast(uint32_t, x)));
}
template <int M>
__device__ __forceinline__ int lane_xor(int x) {
  return (int)lane_xor_u32<M>((uint32_t)x);
}
// The values of both lanes of the pair (l, l ^ M), M = 16 or 32, the lower
// lane's (bit M clear) in .x: v_permlane16_swap / v_permlane32_swap with x in
// both operands exchange the odd 16-lane rows (upper 32 lanes) of the first
// with the even rows (lower 32 lanes) of the second, so the first result holds
// the lower lane's value and the second the upper lane's, in both lanes.
template <int M>
__device__ __forceinline__ float2 lane_pair(float x) {
  static_assert(M == 16 || M == 32, "permlane swap distance");
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  uint32_t lo, hi;
  if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    lo = r[0];
    hi = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    lo = r[0];
    hi = r[1];
  }
  return make_float2(__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi));
}

__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Maximum of x over aligned groups of GL consecutive lanes (GL = 8, 16, 32 or
// 64), every lane of a group receiving it: DPP quad permutes (lanes ^ 1, ^ 2),
// the half-row and row mirrors (lanes 7 - i within 8, 15 - i within 16), then
// v_permlane16_swap / v_permlane32_swap for lanes ^ 16 and ^ 32.
template <int GL>
__device__ __forceinline__ uint32_t group_max(uint32_t x) {
  static_assert(GL == 8 || GL == 16 || GL == 32 || GL == 64, "scale group lanes");
  x = max(x, dpp_u32<0xB1>(x));   // quad_perm [1,0,3,2]
  x = max(x, dpp_u32<0x4E>(x));   // quad_perm [2,3,0,1]
  x = max(x, dpp_u32<0x141>(x));  // row_half_mirror
  if constexpr (GL >= 16) x = max(x, dpp_u32<0x140>(x));  // row_mirror
  if constexpr (GL >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = max((uint32_t)r[0], (uint32_t)r[1]);
  }
  if constexpr (GL >= 64) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    x = max((uint32_t)r[0], (uint32_t)r[1]);
  }
  return x;
}

// Code of x (fp16 value, widened) for the fp16 scale s > 0 with rs = rcp(s)
// (within 1 ulp): clamp(round-half-even(x / s), -127, 127), exactly as a
// correctly rounded division followed by rint. For fp16 x and s the exact
// quotient q is either a half-integer or at least 2^-13 away from every
// half-integer, while t = x * rs is within 3e-7 |q| (< 6e-5 for |q| <= 190,
// the largest quotient a subnormal scale allows) of q: so rint(t) is the
// correctly rounded code except at exact ties, where it may land on the odd
// neighbour. The residual r = x - c s (exact: c s has at most 19 significant
// bits and |r| <= 1.5 s) is then +-s/2, and the tie goes to the even code.
__device__ __forceinline__ int code_of(float x, float s, float rs) {
  float c = __builtin_rintf(x * rs);
  const float r = fmaf(-c, s, x);
  if (fabsf(r) == 0.5f * s && ((int)c & 1)) c += r > 0.0f ? 1.0f : -1.0f;
  return (int)fminf(fmaxf(c, -127.0f), 127.0f);
}

// Quantizer of one group of values spread over GL consecutive lanes (groups
// aligned to GL), 4 fp16 values (bit patterns hb) per lane. Strata PR 2698,
// "What it does": the FP16 scale of a group is its absmax / 127; each value
// becomes the int8 code of x / scale.
//   absmax: exact, on the fp16 bit patterns (for finite values the ordering
//           of |x| is the integer ordering of the bits with the sign cleared);
//   scale = fp16_rne(absmax / 127.0f), the division correctly rounded in fp32;
//   code  = clamp(rint(x / scale), -127, 127) as a correctly rounded fp32
//           division would give it (x and scale are fp16, so that quotient
//           rounds to the same integer as the exact one, ties to even),
//           computed by code_of; 0 where scale == 0.
// Every lane of a group must be active. Returns the 4 codes packed
// little-endian; *scale_bits gets the fp16 scale.
template <int GL>
__device__ __forceinline__ uint32_t quantize4(const uint32_t (&hb)[4], uint16_t* scale_bits) {
  uint32_t amax = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) amax = max(amax, hb[e] & 0x7fffu);
  amax = group_max<GL>(amax);
  const f16 scale_h = (f16)(h_bits_to_f32(amax) / 127.0f);  // fp32 IEEE division, then fp16 RNE
  const float s = (float)scale_h;
  const float rs = __builtin_amdgcn_rcpf(s);
  uint32_t packed = 0;
  if (s > 0.0f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) packed |= ((uint32_t)code_of(h_bits_to_f32(hb[e]), s, rs) & 0xffu) << (8 * e);
  }
  *scale_bits = __builtin_bit_cast(uint16_t, scale_h);
  return packed;
}

}  // namespace kvq
