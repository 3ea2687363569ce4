// Per-tile building blocks of the kernels that read 4-bit stores (the split-K
// decode partials and chunk attention, head_dim 256): the LDS stage layout and
// its direct-to-LDS loads, and the key operands and scores for q4 keys and for
// the int8 keys of k8v4.
//
// Strata PR 2698, "Not in this PR": q4_0 (K and V) and k8v4 (V only) hold
// Q4_0 blocks of rows rotated by the 256-point Hadamard transform.
#pragma once

#include <math.h>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_tile.h"

namespace kvq {

// Stage of one wavefront (bytes): K codes, V codes (128 bytes per q4 row),
// K scale rows, V scale rows. Code rows hold their 16-byte chunk c at slot
// c ^ swz(r); a scale region is 1 KiB for 16-byte rows (a 64-lane
// direct-to-LDS load writes 16 bytes per lane, lanes past row 31 zeros). The
// decode kernel splits the q4 K scale region into two 512-byte halves filled
// by 32 lanes each, for tiles of even and odd index.
template <bool KQ4, bool KG64>
struct Q4Stage {
  static constexpr int D = 256;
  static constexpr int KRB = KQ4 ? D / 2 : D;  // bytes per K row
  static constexpr int VRB = D / 2;
  static constexpr int KNG = KQ4 ? D / kQ4Block : (KG64 ? D / 64 : 1);  // K scales per row
  static constexpr int KSB = 2 * KNG;
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = 32 * KRB;
  static constexpr int KS_OFF = V_OFF + 32 * VRB;
  static constexpr int KS_SPITCH = KSB >= 4 ? KSB : 4;
  static constexpr int KS_BYTES = KQ4 ? 1024 : 256;
  static constexpr int VS_OFF = KS_OFF + KS_BYTES;
  static constexpr int BYTES = VS_OFF + 1024;
  static constexpr int NK = 32 * KRB / 1024 + 1;  // direct-to-LDS loads of a K half
  static constexpr int NV = 32 * VRB / 1024 + 1;  // of a V half
};

// Rows per 256-byte LDS line = 16 / CH; consecutive such row groups get
// distinct chunk slots, so 16 rows read at one chunk hit 16 distinct banks.
template <int CH>
__device__ __forceinline__ int swz(int r) {
  constexpr int SH = CH == 16 ? 0 : (CH == 8 ? 1 : 2);
  return (r >> SH) & (CH - 1);
}

// Direct-to-LDS loads of a 32-row code tile with ROWB bytes per row at byte
// `lds` (rows >= nvalid read as zeros: out-of-range lane offset), with the
// non-temporal cache policy when NT.
template <int ROWB, bool NT = false>
__device__ __forceinline__ void issue_codes(uint32_t lds, const u32x4& rs, uint32_t soff, int nvalid, uint32_t row,
                                            int lane) {
  constexpr int CH = ROWB / 16;
  constexpr int NI = 32 * ROWB / 1024;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int slot = 64 * i + lane;
    const int r = slot / CH;
    const int c = (slot % CH) ^ swz<CH>(r);
    dma<16, NT>(rs, lds + 1024 * i, (nvalid >= kTile || r < nvalid) ? (uint32_t)r * row + 16 * c : kOOB, soff);
  }
}

// Direct-to-LDS load of the scale rows (SB bytes each) of a 32-row tile.
// HALF32 (16-byte rows only): lanes 32..63 write nothing, so the load fills
// exactly 512 bytes.
template <int SB, bool NT = false, bool HALF32 = false>
__device__ __forceinline__ void issue_scales(uint32_t lds, const u32x4& rs, uint32_t soff, int nvalid, uint32_t srow,
                                             int lane) {
  const int nv = nvalid < kTile ? nvalid : kTile;
  if constexpr (SB == 16 && HALF32) {
    if (lane < 32) dma<16, NT>(rs, lds, lane < nv ? (uint32_t)lane * srow : kOOB, soff);
  } else if constexpr (SB == 16) {  // lane l = row l, 16 bytes at 16 l
    dma<16, NT>(rs, lds, lane < nv ? (uint32_t)lane * srow : kOOB, soff);
  } else if constexpr (SB == 8) {  // two lanes per row, 8 bytes at 8 r
    const int r = lane >> 1;
    dma<4, NT>(rs, lds, r < nv ? (uint32_t)r * srow + 4 * (lane & 1) : kOOB, soff);
  } else {  // one 2-byte scale per row, at 4 r
    static_assert(SB == 2, "scale row size");
    dma<2, NT>(rs, lds, lane < nv ? (uint32_t)lane * srow : kOOB, soff);
  }
}

// Fill the K half (HALF = 0) or the V half (HALF = 1) of a stage with the tile
// at position p0. The half's previous contents were read by this wavefront:
// those LDS reads complete before new data can land. For q4 keys the scale
// rows go to the 512-byte half `kpar` of the K scale region.
template <bool KQ4, bool KG64, int HALF>
__device__ __forceinline__ void issue_half(uint8_t* st, const u32x4& rs, const u32x4& srs, int p0, int nvalid,
                                           uint32_t row, uint32_t srow, int lane, int kpar = 0) {
  using T = Q4Stage<KQ4, KG64>;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const uint32_t base = lds_addr_of(st);
  const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)p0 * row);
  const uint32_t ssoff = __builtin_amdgcn_readfirstlane((uint32_t)p0 * srow);
  if constexpr (HALF == 0) {
    issue_codes<T::KRB, kNtCodes>(base + T::K_OFF, rs, soff, nvalid, row, lane);
    if constexpr (KQ4)
      issue_scales<T::KSB, kNtScales, true>(base + T::KS_OFF + 512 * kpar, srs, ssoff, nvalid, srow, lane);
    else
      issue_scales<T::KSB, kNtScales>(base + T::KS_OFF, srs, ssoff, nvalid, srow, lane);
  } else {
    issue_codes<T::VRB, kNtCodes>(base + T::V_OFF, rs, soff, nvalid, row, lane);
    issue_scales<16, kNtScales>(base + T::VS_OFF, srs, ssoff, nvalid, srow, lane);
  }
}

// ---- keys ---------------------------------------------------------------------------
// Two codes (bytes 0, 1 or 2, 3 of a dword of code bytes) as the fp16
// subnormals code * 2^-24 (exact: the matrix cores take subnormal inputs).
__device__ __forceinline__ uint32_t sub_h2_lo(uint32_t w) { return __builtin_amdgcn_perm(0u, w, 0x0c010c00u); }
__device__ __forceinline__ uint32_t sub_h2_hi(uint32_t w) { return __builtin_amdgcn_perm(0u, w, 0x0c030c02u); }

// q4 K codes of one tile for lane (c16, q4): k[ct][j] = bytes 8 (q4 & 1) .. +7
// of block j of row 16 ct + c16 (dims 32 j + 8 q4 .. +7 after the nibble
// select). The tile's scale rows stay in LDS until its scores are taken.
struct KQ4Regs {
  u32x2 k[2][8];
};

template <bool KG64>
__device__ __forceinline__ void read_k_q4(KQ4Regs& t, const uint8_t* __restrict__ st, int c16, int q4) {
  using T = Q4Stage<true, KG64>;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int r = 16 * ct + c16;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      t.k[ct][j] = *reinterpret_cast<const u32x2*>(st + T::K_OFF + r * T::KRB + 16 * (j ^ swz<8>(r)) + 8 * (q4 & 1));
  }
}

constexpr uint32_t kQ4NegBias = 0xE408E408u;  // fp16 pair (-1032, -1032)

// Query operands of scores_q4 for lane (c16, q4), loaded once per split: for
// block j the rotated query's dims 32 j + 8 q4 .. +7 of row c16 as hi and lo
// fp16 terms (the dims 16..31 of each block, lanes q4 = 2, 3, divided by 16),
// and, in the lanes q4 = 0, the row's 8 block sums as hi and lo terms (zero in
// the other lanes).
struct Q4Query {
  f16x8 h[8], l[8];
  f16x8 sh, sl;
};

// qh, ql: LDS rows of the hi and lo terms (+ 64 j for block j, lane's q4
// offset included); sh, sl: LDS block sums of row c16.
__device__ __forceinline__ void load_q4_query(Q4Query& q, const uint8_t* qh, const uint8_t* ql, const uint8_t* sh,
                                              const uint8_t* sl, int q4) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    q.h[j] = *reinterpret_cast<const f16x8*>(qh + 64 * j);
    q.l[j] = *reinterpret_cast<const f16x8*>(ql + 64 * j);
  }
  const f16x8 fz = {};
  q.sh = q4 == 0 ? *reinterpret_cast<const f16x8*>(sh) : fz;
  q.sl = q4 == 0 ? *reinterpret_cast<const f16x8*>(sl) : fz;
}

// Exact scores of a q4 K tile: z[ct][i] for positions x = 16 ct + 4 q4 + i of
// query row c16 (log2 domain); positions outside [vlo, vhi) get -inf.
//   ks       the tile's 32 scale rows (16 bytes: the 8 block scales, fp16) in LDS;
//   qy       the query operands (Q4Query);
//   c2s      sm_scale * log2(e) * 2^24.
// The lanes q4 = 0, 1 take the low nibbles (code q) of their bytes and the
// lanes q4 = 2, 3 the high ones in place (16 q), both as the fp16 subnormals
// of the masked byte times 2^-24, so that with the /16 of their query dims
// every product is exactly code * q_d * 2^-24. Block j gives
// a_j = 2^-24 * sum_d code_d q_d (fp32 sums); one MFMA pair per C-tile gives
// c = sum_j d_j Q_j over the row scales (k slots 0..7 of the lanes q4 = 0) and
// the block sums, and
//   z = c2s * (sum_j d_j a_j - 8 * 2^-24 * c)  =  c2 * sum_j d_j sum_d (code_d - 8) q_d,
// the dequantized key (code - 8) * d taken without rounding.
__device__ __forceinline__ void scores_q4(const KQ4Regs& t, int vlo, int vhi, float (&z)[2][4],
                                          const uint8_t* __restrict__ ks, const Q4Query& qy, float c2s, int c16,
                                          int q4) {
  const uint32_t mask = q4 >= 2 ? 0xF0F0F0F0u : 0x0F0F0F0Fu;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 zz[2];
  u32x4 ps[2][4];  // the 8 block scales of row 16 ct + 4 q4 + i: the position of score z[ct][i]
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const f16x8 own = *reinterpret_cast<const f16x8*>(ks + (16 * ct + c16) * 16);  // A: row c16's scales
    f32x4 c = mfma16(own, qy.sh, zero);
    c = mfma16(own, qy.sl, c);
#pragma unroll
    for (int i = 0; i < 4; ++i) zz[ct][i] = c[i] * (-8.0f / 16777216.0f);
#pragma unroll
    for (int i = 0; i < 4; ++i) ps[ct][i] = *reinterpret_cast<const u32x4*>(ks + (16 * ct + 4 * q4 + i) * 16);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const uint32_t w0 = t.k[ct][j].x & mask;
      const uint32_t w1 = t.k[ct][j].y & mask;
      const u32x4 a4 = {sub_h2_lo(w0), sub_h2_hi(w0), sub_h2_lo(w1), sub_h2_hi(w1)};  // (masked byte) * 2^-24
      f32x4 a = mfma16(__builtin_bit_cast(f16x8, a4), qy.h[j], zero);
      a = mfma16(__builtin_bit_cast(f16x8, a4), qy.l[j], a);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t sw = ps[ct][i][j >> 1];
        const f16 d = __builtin_bit_cast(f16x2, sw)[j & 1];
        zz[ct][i] = fmaf(a[i], (float)d, zz[ct][i]);
      }
    }
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int x = 16 * ct + 4 * q4 + i;
      z[ct][i] = (x >= vlo && x < vhi) ? zz[ct][i] * c2s : -INFINITY;
    }
}

// int8 K operands (k8v4) from this stage layout, as stage_read_k reads them.
template <bool KG64>
__device__ __forceinline__ void read_k_i8(KRegs<Shape<256, true, true, KG64>>& t, const uint8_t* __restrict__ st,
                                          int c16, int q4) {
  using S = Shape<256, true, true, KG64>;
  using T = Q4Stage<false, KG64>;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int r = 16 * ct + c16;
#pragma unroll
    for (int j = 0; j < S::NJ; ++j)
      t.k[ct][j][0] = *reinterpret_cast<const u32x4*>(st + T::K_OFF + r * 256 + 16 * ((4 * j + q4) ^ swz<16>(r)));
    const uint8_t* ksp = st + T::KS_OFF + (16 * ct + 4 * q4) * T::KS_SPITCH;
    if constexpr (KG64) {  // 8-byte rows
      const u32x4 a = *reinterpret_cast<const u32x4*>(ksp);
      const u32x4 b = *reinterpret_cast<const u32x4*>(ksp + 16);
      t.ks[ct][0][0] = a.x; t.ks[ct][0][1] = a.y;
      t.ks[ct][1][0] = a.z; t.ks[ct][1][1] = a.w;
      t.ks[ct][2][0] = b.x; t.ks[ct][2][1] = b.y;
      t.ks[ct][3][0] = b.z; t.ks[ct][3][1] = b.w;
    } else {  // one 2-byte scale per row, rows 4 bytes apart
      const u32x4 a = *reinterpret_cast<const u32x4*>(ksp);
      t.ks[ct][0][0] = a.x & 0xffffu;
      t.ks[ct][1][0] = a.y & 0xffffu;
      t.ks[ct][2][0] = a.z & 0xffffu;
      t.ks[ct][3][0] = a.w & 0xffffu;
    }
  }
}

// Scores of an int8 K tile (k8v4): as the int8 kernel's, with the bias
// correction added after each MFMA instead of preloaded into its accumulator
// (one register per group instead of four). masked = false (wavefront-
// uniform): every position of the tile inside [vlo, vhi), no mask.
template <bool KG64>
__device__ __forceinline__ void scores_i8(const KRegs<Shape<256, true, true, KG64>>& t, int vlo, int vhi,
                                          float (&z)[2][4], const f16x8 (&qv)[4][2], const float (&corr)[KG64 ? 4 : 1],
                                          float c2, int q4, bool masked = true) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    f32x4 zz = zero;
    if constexpr (KG64) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 c = t.k[ct][j][0];
        f32x4 a = mfma16(codes8_biased(c.x, c.y), qv[j][0], zero);
        a = mfma16(codes8_biased(c.z, c.w), qv[j][1], a);
#pragma unroll
        for (int i = 0; i < 4; ++i) zz[i] = fmaf(a[i] + corr[j], scale_of(t.ks[ct][i], j), zz[i]);
      }
    } else {
      f32x4 a = zero;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 c = t.k[ct][j][0];
        a = mfma16(codes8_biased(c.x, c.y), qv[j][0], a);
        a = mfma16(codes8_biased(c.z, c.w), qv[j][1], a);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) zz[i] = (a[i] + corr[0]) * scale_of(t.ks[ct][i], 0);
    }
    if (masked) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int x = 16 * ct + 4 * q4 + i;
        z[ct][i] = (x >= vlo && x < vhi) ? zz[i] * c2 : -INFINITY;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) z[ct][i] = zz[i] * c2;
    }
  }
}

}  // namespace kvq
