// Per-tile building blocks shared by the split-K decode kernel and the chunk
// attention kernel on gfx950: the operand registers of a 32-position K/V tile,
// the MFMA products S^T = K.Q^T and O += P.V_hat with int8 codes entering as
// exact fp16 values, the base-2 online softmax, and the direct-to-LDS staging
// of code tiles and their scale rows (see kvq_decode.hip for the data flow).
//
// genie-ai-runtime release v0.1.0-alpha.12, "Path I series" #65: keys and
// values are dequantized as code * scale of their (position, kv head); Strata
// PR 2698, "What it does": an FP16 scale for each 64-value group.
#pragma once

#include <math.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr float kTau = 8.0f;
constexpr float kLog2e = 1.4426950408889634f;

// Compile-time shape of one kernel instance.
template <int D_, bool KI8_, bool VI8_, bool G64_>
struct Shape {
  static constexpr int D = D_;
  static constexpr bool KI8 = KI8_, VI8 = VI8_, G64 = G64_;
  static constexpr int NJ = D / 64;          // 64-wide dim blocks per row (2 k-steps each)
  static constexpr int NG = G64 ? NJ : 1;    // scales per row
  static constexpr int SB = 2 * NG;          // scale bytes per row
  static constexpr int NKS = (SB + 3) / 4;   // dwords holding one row's scales
  static constexpr int VB = D / 16;          // V dims per lane per position = PV n-tiles
  static constexpr int KE = KI8 ? 1 : 4;     // element bytes
  static constexpr int VE = VI8 ? 1 : 4;
  static constexpr int KW = KI8 ? 1 : 4;     // u32x4 of K per (C-tile, dim block)
  static constexpr int VW = VB * VE / 4;     // dwords of V per lane per position
  static constexpr int CH = D / 16;          // 16-byte chunks per int8 row
};

// Operand registers of one 32-position tile for one lane, in two halves that
// are never live together in the LDS-staged kernel.
//   k[ct][j]  A operand of S^T: row c16 of C-tile ct, dims 64j + 16*q4 + [0,16)
//   ks[ct][i] the NG fp16 scales of position 16ct + 4*q4 + i (packed)
//   v[e]      B operand of P.V: position kpos(e), dims VB*c16 + [0,VB)
//   vs[e]     fp16 scale of v[e]'s group (low half)
template <class S>
struct KRegs {
  u32x4 k[2][S::NJ][S::KW];
  uint32_t ks[2][4][S::NKS];
};
template <class S>
struct VRegs {
  uint32_t v[8][S::VW];
  uint32_t vs[8];
};

template <class S>
struct WaveAcc {
  f32x4 o[S::VB];
  f32x4 l;
  float m_ref;
};

// Position (within the tile) of element e of a lane's k-slice in P.V: the lane
// of S^T with row group q4 holds positions 4*q4 + i of both 16-row C-tiles.
__device__ __forceinline__ int kpos(int e, int q4) { return e < 4 ? 4 * q4 + e : 12 + 4 * q4 + e; }

__device__ __forceinline__ float scale_of(const uint32_t* packed, int j) {
  const uint32_t w = packed[j >> 1];
  return h_bits_to_f32((j & 1) ? (w >> 16) : (w & 0xffffu));
}

// The query operand (B of S^T = K.Q^T) for lane (head c16, k-group q4) lives in
// LDS, rows padded to break bank conflicts; k-step 2j+u covers dims
// 64j + 16*q4 + 8u + [0, 8). `qp` points at the lane's row + 32*q4 bytes.
// Every LDS pointer that the tile loop reads through is a __restrict__
// parameter: the alias scopes this gives the reads let the compiler wait only
// for the LDS stage being read, not for the stage that is still loading.
template <class S>
struct QOperand {
  static constexpr int ROW = 2 * S::D + 16;  // bytes per padded head row
};
__device__ __forceinline__ f16x8 q_get(const uint8_t* __restrict__ qp, int j, int u) {
  return *reinterpret_cast<const f16x8*>(qp + 128 * j + 16 * u);
}

// K half of a tile: the scaled, masked scores z (log2 domain) of the 32
// positions x 16 query rows of S^T = K.Q^T; lane (c16, q4) gets positions
// 16*ct + 4*q4 + i of query row c16. Positions x of the tile with
// vlo <= x < vhi keep their score, the others get -inf (vlo, vhi may differ
// per lane: per query row). masked = false (wavefront-uniform) skips the
// mask when every position of the tile is inside every row's range.
template <class S>
__device__ __forceinline__ void tile_scores_q(const KRegs<S>& t, int vlo, int vhi, float (&z)[2][4],
                                              const f16x8 (&qv)[S::NJ][2], const float (&corr)[S::NG],
                                              float c2, int q4, bool masked = true) {
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    f32x4 zz = {0.f, 0.f, 0.f, 0.f};
    if constexpr (S::KI8 && S::G64) {
#pragma unroll
      for (int j = 0; j < S::NJ; ++j) {
        const u32x4 c = t.k[ct][j][0];
        f32x4 a = mfma16(codes8_biased(c.x, c.y), qv[j][0], (f32x4){corr[j], corr[j], corr[j], corr[j]});
        a = mfma16(codes8_biased(c.z, c.w), qv[j][1], a);
#pragma unroll
        for (int i = 0; i < 4; ++i) zz[i] = fmaf(a[i], scale_of(t.ks[ct][i], j), zz[i]);
      }
    } else if constexpr (S::KI8) {
      f32x4 a = {corr[0], corr[0], corr[0], corr[0]};
#pragma unroll
      for (int j = 0; j < S::NJ; ++j) {
        const u32x4 c = t.k[ct][j][0];
        a = mfma16(codes8_biased(c.x, c.y), qv[j][0], a);
        a = mfma16(codes8_biased(c.z, c.w), qv[j][1], a);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) zz[i] = a[i] * scale_of(t.ks[ct][i], 0);
    } else {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < S::NJ; ++j) {
        a = mfma16(f32x8_to_f16x8(t.k[ct][j][0], t.k[ct][j][S::KW > 1 ? 1 : 0]), qv[j][0], a);
        a = mfma16(f32x8_to_f16x8(t.k[ct][j][S::KW > 2 ? 2 : 0], t.k[ct][j][S::KW > 3 ? 3 : 0]), qv[j][1], a);
      }
      zz = a;
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

// tile_scores_q with the query operands read from LDS (`qb`, see QOperand)
// and positions [vlo, vhi) of the tile kept (per query row). All query
// operand reads are issued before the first MFMA so that their LDS latency is
// paid once per tile.
template <class S>
__device__ __forceinline__ void tile_scores(const KRegs<S>& t, int vlo, int vhi, float (&z)[2][4],
                                            const uint8_t* __restrict__ qb, const float (&corr)[S::NG],
                                            float c2, int q4) {
  f16x8 qv[S::NJ][2];
#pragma unroll
  for (int j = 0; j < S::NJ; ++j) {
    qv[j][0] = q_get(qb, j, 0);
    qv[j][1] = q_get(qb, j, 1);
  }
  __builtin_amdgcn_sched_barrier(0);
  tile_scores_q<S>(t, vlo, vhi, z, qv, corr, c2, q4);
}
// The same with positions [0, nvalid) kept for every query row.
template <class S>
__device__ __forceinline__ void tile_scores(const KRegs<S>& t, int nvalid, float (&z)[2][4],
                                            const uint8_t* __restrict__ qb, const float (&corr)[S::NG],
                                            float c2, int q4) {
  tile_scores<S>(t, 0, nvalid, z, qb, corr, c2, q4);
}

// Maximum over lanes l, l ^ 16 and l ^ 32 without going through LDS:
// v_permlane16_swap exchanges the odd 16-lane rows of its first operand with
// the even rows of its second, v_permlane32_swap the upper 32 lanes of the
// first with the lower 32 of the second. With x in both operands, every lane
// ends up holding its own value and that of its partner lane, one in each.
__device__ __forceinline__ float max_xor16_xor32(float x) {
  float y;
  asm volatile("" : "=v"(y) : "0"(x));  // a second register holding x
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, y), false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  x = fmaxf(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
  asm volatile("" : "=v"(y) : "0"(x));
  const auto u = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, y), false, false);
  const uint32_t u0 = u[0], u1 = u[1];
  return fmaxf(__builtin_bit_cast(float, u0), __builtin_bit_cast(float, u1));
}

// Online-softmax update for one tile's scores; returns the tile's
// probabilities P (fp16) in the A-operand layout of P.V.
template <class S>
__device__ __forceinline__ f16x8 tile_softmax(const float (&z)[2][4], WaveAcc<S>& acc, int q4) {
  // ---- online softmax (base 2) -------------------------------------------------
  float tmax = z[0][0];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, z[ct][i]);
  tmax = max_xor16_xor32(tmax);  // tile max of head c16
  const bool need = tmax > acc.m_ref + kTau;
  if (__any(need)) {
    const float m_new = need ? tmax : acc.m_ref;
    const float alpha = need ? __builtin_amdgcn_exp2f(acc.m_ref - m_new) : 1.0f;
    acc.m_ref = m_new;
    // acc.o / acc.l rows are heads 4*q4 + i; lane h holds head h's alpha.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ai = __shfl(alpha, 4 * q4 + i);
#pragma unroll
      for (int n = 0; n < S::VB; ++n) acc.o[n][i] *= ai;
      acc.l[i] *= ai;
    }
  }
  const float mu = acc.m_ref == -INFINITY ? 0.0f : acc.m_ref;
  f16x8 pa;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) pa[4 * ct + i] = (f16)__builtin_amdgcn_exp2f(z[ct][i] - mu);
  return pa;
}

// V half of a tile: O += P . V_hat ;  l += P . 1. PART 1 and 2 split the work
// in two halves of the output columns (l goes with PART 2), so that a wait can
// sit between them; PART 0 does all of it.
// RB row blocks (acc[0 .. RB)) share every value operand: each dequantized
// operand feeds one MFMA per block.
template <class S, int PART = 0, int RB = 1>
__device__ __forceinline__ void tile_pv_rows(const VRegs<S>& t, const f16x8 (&pa)[RB], WaveAcc<S>* acc) {
  constexpr int W0 = PART == 2 ? S::VW / 2 : 0, W1 = PART == 1 ? S::VW / 2 : S::VW;
  constexpr int N0 = PART == 2 ? S::VB / 2 : 0, N1 = PART == 1 ? S::VB / 2 : S::VB;
  if constexpr (S::VI8) {
    constexpr uint32_t kNegBias = 0xE480E480u;  // fp16 pair (-1152, -1152)
    f16x2 sv[4];
#pragma unroll
    for (int pi = 0; pi < 4; ++pi) sv[pi] = as_h2(__builtin_amdgcn_perm(t.vs[2 * pi + 1], t.vs[2 * pi], 0x05040100u));
#pragma unroll
    for (int w = W0; w < W1; ++w) {
      uint32_t z01[4], z23[4];
#pragma unroll
      for (int pi = 0; pi < 4; ++pi) {
        z01[pi] = zip_lo(t.v[2 * pi + 1][w], t.v[2 * pi][w]) ^ kCodeFlip;
        z23[pi] = zip_hi(t.v[2 * pi + 1][w], t.v[2 * pi][w]) ^ kCodeFlip;
      }
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        u32x4 r;
#pragma unroll
        for (int pi = 0; pi < 4; ++pi) {
          const uint32_t src = bb < 2 ? z01[pi] : z23[pi];
          const uint32_t biased = (bb & 1) ? biased_h2_hi(src) : biased_h2_lo(src);
          const f16x2 c = as_h2(biased) + as_h2(kNegBias);  // exact code
          r[pi] = as_u32(c * sv[pi]);                        // fp16(code * scale)
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          acc[rb].o[4 * w + bb] = mfma16(pa[rb], __builtin_bit_cast(f16x8, r), acc[rb].o[4 * w + bb]);
      }
    }
  } else {
#pragma unroll
    for (int n = N0; n < N1; ++n) {
      u32x4 r;
#pragma unroll
      for (int pi = 0; pi < 4; ++pi)
        r[pi] = as_u32(__builtin_bit_cast(
            f16x2, __builtin_amdgcn_cvt_pkrtz(__builtin_bit_cast(float, t.v[2 * pi][n]),
                                              __builtin_bit_cast(float, t.v[2 * pi + 1][n]))));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[rb].o[n] = mfma16(pa[rb], __builtin_bit_cast(f16x8, r), acc[rb].o[n]);
    }
  }
  if constexpr (PART != 1) {
    const f16x8 ones = {(f16)1, (f16)1, (f16)1, (f16)1, (f16)1, (f16)1, (f16)1, (f16)1};
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb].l = mfma16(pa[rb], ones, acc[rb].l);
  }
}
// One row block.
template <class S, int PART = 0>
__device__ __forceinline__ void tile_pv(const VRegs<S>& t, f16x8 pa, WaveAcc<S>& acc) {
  const f16x8 p1[1] = {pa};
  tile_pv_rows<S, PART, 1>(t, p1, &acc);
}

// ---- LDS staging for int8 K and V --------------------------------------------------
// Stage layout (bytes): K codes [0, 32D), V codes [32D, 64D), K scales
// [64D, 64D+256), V scales [64D+256, 64D+512). Row r of a code tile holds its
// 16-byte chunk c at chunk slot c ^ swz(r). The scales of row r start at
// r * SPITCH: a direct-to-LDS load places lane l's data at l * max(size, 4)
// bytes, so 2-byte scale rows land 4 bytes apart.
template <class S>
struct Stage {
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = 32 * S::D;
  static constexpr int KS_OFF = 64 * S::D;
  static constexpr int VS_OFF = 64 * S::D + 256;
  static constexpr int BYTES = 64 * S::D + 512;
  static constexpr int SPITCH = S::SB >= 4 ? S::SB : 4;
  // Rows per 256 bytes (the LDS bank width) = 16 / CH; spreading consecutive
  // such row groups over distinct chunk slots keeps 16 lanes that read 16
  // different rows at one column on 16 distinct bank groups.
  static __device__ __forceinline__ int swz(int r) {
    constexpr int SH = S::CH == 16 ? 0 : (S::CH == 8 ? 1 : 2);
    return (r >> SH) & (S::CH - 1);
  }
};

typedef __attribute__((address_space(3))) uint8_t* lds_u8_t;

// Direct-to-LDS buffer loads, written as inline asm: the compiler's wait-count
// insertion cannot tell which LDS bytes such a load writes and would make every
// later LDS read wait for all of them, which serialises the two stages. Here
// every wait for these loads is explicit (wait_vm below); the tile loop issues
// no other vector-memory instruction, so counts are exact. Lane l's data lands
// at M0 + l * max(bytes, 4). Writing M0 needs one wait state before the load.
// NT sets the load's non-temporal cache policy (data read once: the caches
// need not keep it).
#define KVQ_DMA_ASM(OP, POLICY)                                                          \
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t" OP " %1, %2, %3 offen" POLICY " lds" \
               :: "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0")
template <int BYTES, bool NT = false>
__device__ __forceinline__ void dma(u32x4 rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  static_assert(BYTES == 16 || BYTES == 4 || BYTES == 2, "direct-to-LDS load size");
  if constexpr (BYTES == 16) {
    if constexpr (NT) KVQ_DMA_ASM("buffer_load_dwordx4", " nt"); else KVQ_DMA_ASM("buffer_load_dwordx4", "");
  } else if constexpr (BYTES == 4) {
    if constexpr (NT) KVQ_DMA_ASM("buffer_load_dword", " nt"); else KVQ_DMA_ASM("buffer_load_dword", "");
  } else {
    if constexpr (NT) KVQ_DMA_ASM("buffer_load_ushort", " nt"); else KVQ_DMA_ASM("buffer_load_ushort", "");
  }
}
#undef KVQ_DMA_ASM

// Cache policy of the decode kernels' KV tile loads. A decode step reads each
// cached position's codes (int8 or 4-bit) once, so they stream with the
// non-temporal policy; the scale rows keep the default one. Measured on the
// 128K-context and the batched shapes, the non-temporal code loads shorten the
// partial kernel by 3-10 % and the same policy on the scale loads lengthens it.
// The chunk kernels keep the default policy: there the workgroups of several
// row blocks read the same key tiles.
constexpr bool kNtCodes = true;
constexpr bool kNtScales = false;

// Wait until at most N vector-memory operations of this wavefront are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// A raw buffer resource as four SGPRs: base, stride 0, size in bytes, flags.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 r = {(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, kBufWord3};
  r.x = __builtin_amdgcn_readfirstlane(r.x);
  r.y = __builtin_amdgcn_readfirstlane(r.y);
  r.z = __builtin_amdgcn_readfirstlane(r.z);
  return r;
}

__device__ __forceinline__ uint32_t lds_addr_of(const uint8_t* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_u8_t)p);
}

// Direct-to-LDS loads that fill one half (K or V) of a stage: a code tile and
// its scale rows.
template <class S>
constexpr int kHalfLoads = 32 * S::D / 1024 + 1;

// Fill the K half (HALF = 0) or the V half (HALF = 1) of a stage with the tile
// at position p0 (nvalid positions of it inside the split).
//
// Bounds: a row the tile does not own gets the out-of-range offset kOOB in its
// lane offset, so it reads as zeros. The lane offset is the only part of the
// address that the buffer range check is sure to cover (the uniform soffset
// may not be), so no row beyond the split is ever fetched from memory; a full
// tile (nvalid >= 32) has no such row and skips the selects.
template <class S, int HALF>
__device__ __forceinline__ void stage_issue(uint8_t* st, const u32x4& rs, const u32x4& srs, int p0, int nvalid,
                                            uint32_t row, uint32_t srow, int lane) {
  using T = Stage<S>;
  constexpr int NI = 32 * S::D / 1024;  // 1 KiB direct-to-LDS loads per code tile
  constexpr int CODE_OFF = HALF == 0 ? T::K_OFF : T::V_OFF;
  constexpr int SCALE_OFF = HALF == 0 ? T::KS_OFF : T::VS_OFF;
  // The half's previous contents were read by this wavefront: make sure those
  // LDS reads have completed before new data can land.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const uint32_t base = lds_addr_of(st);
  const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)p0 * row);
  auto code_off = [&](int i) {
    const int slot = i * 64 + lane;
    const int r = slot / S::CH;
    const int c = (slot % S::CH) ^ T::swz(r);
    return (uint32_t)r * row + 16 * c;
  };
  if (nvalid >= kTile) {
#pragma unroll
    for (int i = 0; i < NI; ++i) dma<16, kNtCodes>(rs, base + CODE_OFF + 1024 * i, code_off(i), soff);
  } else {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = (i * 64 + lane) / S::CH;
      dma<16, kNtCodes>(rs, base + CODE_OFF + 1024 * i, r < nvalid ? code_off(i) : kOOB, soff);
    }
  }
  const uint32_t ssoff = __builtin_amdgcn_readfirstlane((uint32_t)p0 * srow);
  const int nv = nvalid < kTile ? nvalid : kTile;
  if constexpr (S::SB >= 4) {
    constexpr int PER = S::SB / 4;  // dwords per row
    const int r = lane / PER;
    const uint32_t voff = r < nv ? (uint32_t)r * srow + 4 * (lane % PER) : kOOB;
    dma<4, kNtScales>(srs, base + SCALE_OFF, voff, ssoff);
  } else {  // lane l = row l, written at byte 4l (see SPITCH); rows 32..63 read as 0
    const uint32_t voff = lane < nv ? (uint32_t)lane * srow : kOOB;
    dma<2, kNtScales>(srs, base + SCALE_OFF, voff, ssoff);
  }
}

template <class S>
__device__ __forceinline__ void stage_read_k(KRegs<S>& t, const uint8_t* __restrict__ st, int c16, int q4) {
  using T = Stage<S>;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int r = 16 * ct + c16;
#pragma unroll
    for (int j = 0; j < S::NJ; ++j) {
      const int slot = (4 * j + q4) ^ T::swz(r);
      t.k[ct][j][0] = *reinterpret_cast<const u32x4*>(st + T::K_OFF + r * S::D + 16 * slot);
    }
    const uint8_t* ksp = st + T::KS_OFF + (16 * ct + 4 * q4) * T::SPITCH;
    if constexpr (S::SB == 8) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(ksp);
      const u32x4 b = *reinterpret_cast<const u32x4*>(ksp + 16);
      t.ks[ct][0][0] = a.x; t.ks[ct][0][S::NKS - 1] = a.y;
      t.ks[ct][1][0] = a.z; t.ks[ct][1][S::NKS - 1] = a.w;
      t.ks[ct][2][0] = b.x; t.ks[ct][2][S::NKS - 1] = b.y;
      t.ks[ct][3][0] = b.z; t.ks[ct][3][S::NKS - 1] = b.w;
    } else if constexpr (S::SB == 4) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(ksp);
      t.ks[ct][0][0] = a.x;
      t.ks[ct][1][0] = a.y;
      t.ks[ct][2][0] = a.z;
      t.ks[ct][3][0] = a.w;
    } else {  // one 2-byte scale per row, rows 4 bytes apart
      const u32x4 a = *reinterpret_cast<const u32x4*>(ksp);
      t.ks[ct][0][0] = a.x & 0xffffu;
      t.ks[ct][1][0] = a.y & 0xffffu;
      t.ks[ct][2][0] = a.z & 0xffffu;
      t.ks[ct][3][0] = a.w & 0xffffu;
    }
  }
}

template <class S>
__device__ __forceinline__ void stage_read_v(VRegs<S>& t, const uint8_t* __restrict__ st, int c16, int q4) {
  using T = Stage<S>;
  const int byte = S::VB * c16;
  const int grp = S::G64 ? byte / 64 : 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int r = kpos(e, q4);
    const uint8_t* p = st + T::V_OFF + r * S::D + 16 * ((byte / 16) ^ T::swz(r)) + (byte % 16);
    if constexpr (S::VW == 4) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(p);
      t.v[e][0] = v.x;
      t.v[e][1] = v.y;
      t.v[e][2] = v.z;
      t.v[e][3] = v.w;
    } else if constexpr (S::VW == 2) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(p);
      t.v[e][0] = v.x;
      t.v[e][S::VW - 1] = v.y;
    } else {
      t.v[e][0] = *reinterpret_cast<const uint32_t*>(p);
    }
    t.vs[e] = *reinterpret_cast<const uint16_t*>(st + T::VS_OFF + r * T::SPITCH + 2 * grp);
  }
}


// ---- LDS staging for an fp32 store (the fp32 side of k8v32 / k32v8) ----------------
// One 32-position tile of fp32 rows: row r's 16-byte chunk c (dims 4c..4c+3)
// sits at byte r * 4D + 16 * F32Stage::slot(r, c). The permutation of a row's
// chunks is chosen for the MFMA-layout reads, which fetch 16 bytes per lane:
//   K (S^T's A operand): 16 lanes read chunk c of rows r .. r + 15, so the low
//     four chunk bits are XOR-ed with the row's;
//   V (P.V's B operand): 16 lanes read one row at chunks NC*c16 + m, NC = the
//     chunks per lane (D / 64), so the low log2(NC) bits are XOR-ed with bits
//     4-5 (chunks 16 apart hit the same banks).
// Both maps only change bits below the ones they depend on, so each is its own
// inverse: the direct-to-LDS loads fetch chunk slot(r, c) into slot c.
template <class S, bool IS_K>
struct F32Stage {
  static constexpr int CH = S::D / 4;  // 16-byte chunks per fp32 row
  static constexpr int NC = S::D / 64;  // chunks of V per lane per position
  static constexpr int BYTES = 32 * S::D * 4;
  static constexpr int LOADS = BYTES / 1024;  // 1 KiB direct-to-LDS loads per tile
  static __device__ __forceinline__ int slot(int r, int c) {
    if constexpr (IS_K) return c ^ (r & 15);
    else return c ^ ((c >> 4) & (NC - 1));
  }
};

// Load the fp32 tile at p0 (positions >= nvalid read as zeros) into a stage.
template <class S, bool IS_K>
__device__ __forceinline__ void f32stage_issue(uint8_t* st, const u32x4& rs, int p0, int nvalid, uint32_t row,
                                               int lane) {
  using T = F32Stage<S, IS_K>;
  // this wavefront's LDS reads of the stage's previous tile have completed
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const uint32_t base = lds_addr_of(st);
  const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)p0 * row);
#pragma unroll
  for (int i = 0; i < T::LOADS; ++i) {
    const int sl = i * 64 + lane;
    const int r = sl / T::CH;
    const uint32_t off = r < nvalid ? (uint32_t)r * row + 16 * T::slot(r, sl % T::CH) : kOOB;
    dma<16, kNtCodes>(rs, base + 1024 * i, off, soff);
  }
}

template <class S>
__device__ __forceinline__ void f32stage_read_k(KRegs<S>& t, const uint8_t* __restrict__ st, int c16, int q4) {
  using T = F32Stage<S, true>;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int r = 16 * ct + c16;
#pragma unroll
    for (int j = 0; j < S::NJ; ++j)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        t.k[ct][j][m] = *reinterpret_cast<const u32x4*>(st + r * 4 * S::D + 16 * T::slot(r, 16 * j + 4 * q4 + m));
  }
}

template <class S>
__device__ __forceinline__ void f32stage_read_v(VRegs<S>& t, const uint8_t* __restrict__ st, int c16, int q4) {
  using T = F32Stage<S, false>;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int r = kpos(e, q4);
#pragma unroll
    for (int m = 0; m < T::NC; ++m) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(st + r * 4 * S::D + 16 * T::slot(r, T::NC * c16 + m));
      t.v[e][4 * m + 0] = v.x;
      t.v[e][4 * m + 1] = v.y;
      t.v[e][4 * m + 2] = v.z;
      t.v[e][4 * m + 3] = v.w;
    }
  }
}

}  // namespace kvq
