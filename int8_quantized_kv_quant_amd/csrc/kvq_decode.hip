// kv_decode_attn_splitk: split-K partials of single-token decode attention over
// an int8 (or fp32) KV cache, on the gfx950 matrix cores.
//
// genie-ai-runtime releases, v1.3.0 "split-K decode attention": the KV range of
// a head is split over blocks that each form an online-softmax partial, later
// combined by a reduce kernel. v0.1.0-alpha.12 "Path I series" #65: each key and
// value is dequantized as code * scale of its (position, kv head). Strata
// PR 2698 "What it does": one FP16 scale per 64 values; k8v32 / k32v8.
//
// Mapping. One workgroup = (sequence b, kv head, block of up to 16 query heads
// sharing it, split s); its NW wavefronts take 32-position tiles of the split
// round-robin. Per tile a wavefront computes, with v_mfma_f32_16x16x32_f16:
//   S^T (32 positions x 16 heads) = K (codes) . Q^T      (D/16 MFMAs)
//   O   (16 heads x D)           += P (fp16) . V_hat     (D/16 MFMAs)
//   l   (16 heads)               += P . 1                (1 MFMA)
// Query heads beyond the group are zero rows. The GQA group is the MFMA's
// 16-wide dimension, so K and V are read from HBM once per kv head.
//
// Keys. Codes enter the MFMA as 1152 + code (exact fp16, built by byte
// permutes); the 1152 * sum(q) term is removed by starting each accumulator at
// -1152 * sum(q) of its dims. A k-step never mixes two 64-value scale groups, so
// per-group dot products are scaled by their fp16 scale in fp32 afterwards:
//   z = sm_scale * log2(e) * sum_j scale_j * dot_j     (exact dequantization).
// Values. V_hat = fp16(code * scale) per element (one rounding, relative error
// <= 2^-11), so P.V_hat needs no per-position rescaling afterwards.
// Softmax. Base-2 online softmax with a lazily raised reference max: the
// accumulators are rescaled only when a tile's max exceeds the reference by more
// than kTau (then P <= 2^kTau in fp16). The row sum l comes out of the same MFMA
// as O, so out = O / l is a convex combination of the V_hat rows.
// Partial output of a split: per query head its max m (log2 domain), l, and the
// unnormalized O, after merging the wavefronts of the workgroup in LDS.
//
// Bounds. Every K/V/scale load goes through a buffer resource whose size ends
// at the last row of the context, and positions outside the split get an
// out-of-range offset, so they read as zero and are masked out of the softmax.
#include <math.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr float kTau = 8.0f;
constexpr float kLog2e = 1.4426950408889634f;

struct PartialArgs {
  const void* k_store;
  const void* v_store;
  const uint16_t* k_scales;
  const uint16_t* v_scales;
  const uint16_t* q;
  const int32_t* seq_lens;
  float* ws_o;   // [B][Hq][n_splits][D]
  float* ws_ml;  // [B][Hq][n_splits][2]
  int64_t s_seq, s_pos, s_head;
  int64_t ss_seq, ss_pos, ss_head;
  int32_t max_ctx;
  int32_t n_kv, G, n_q, head_blocks;
  int32_t n_splits, chunk, window;
  float c2;  // sm_scale * log2(e)
};

template <int D, bool KI8, bool VI8, bool G64, int NW>
__global__ __launch_bounds__(NW * 64) void kvq_partial_kernel(PartialArgs a) {
  constexpr int NJ = D / 64;            // 64-wide dim blocks per row (2 k-steps each)
  constexpr int NG = G64 ? NJ : 1;      // scales per row
  constexpr int VB = D / 16;            // V elements per lane per position = PV n-tiles
  constexpr int KE = KI8 ? 1 : 4;       // K element bytes
  constexpr int VE = VI8 ? 1 : 4;       // V element bytes

  const int split = blockIdx.x;
  const int hk = blockIdx.y / a.head_blocks;
  const int hblk = blockIdx.y % a.head_blocks;
  const int b = blockIdx.z;

  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_ctx ? a.max_ctx : L);
  const int lo = a.window > 0 ? max(0, L - a.window) : 0;
  const int64_t start64 = (int64_t)lo + (int64_t)split * a.chunk;
  if (start64 >= L) return;  // empty split: the reduce never reads it
  const int start = (int)start64;
  const int end = (split == a.n_splits - 1) ? L : (int)min((int64_t)L, start64 + a.chunk);

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int c16 = lane & 15;
  const int q4 = lane >> 4;
  const int nh = min(16, a.G - hblk * 16);
  const int hq0 = hk * a.G + hblk * 16;

  // ---- buffer resources of this (sequence, kv head) slice -------------------
  const uint32_t krow = (uint32_t)(a.s_pos * KE);
  const uint32_t vrow = (uint32_t)(a.s_pos * VE);
  const uint32_t srow = (uint32_t)(a.ss_pos * 2);
  const int64_t st_off = (int64_t)b * a.s_seq + (int64_t)hk * a.s_head;
  const int64_t sc_off = (int64_t)b * a.ss_seq + (int64_t)hk * a.ss_head;
  const auto krs = make_rsrc(static_cast<const char*>(a.k_store) + st_off * KE,
                             (uint32_t)(((int64_t)(L - 1) * a.s_pos + D) * KE));
  const auto vrs = make_rsrc(static_cast<const char*>(a.v_store) + st_off * VE,
                             (uint32_t)(((int64_t)(L - 1) * a.s_pos + D) * VE));
  const uint32_t sc_bytes = (uint32_t)(((int64_t)(L - 1) * a.ss_pos + NG) * 2);
  const auto ksrs = make_rsrc(KI8 ? static_cast<const void*>(a.k_scales + sc_off) : nullptr, KI8 ? sc_bytes : 0u);
  const auto vsrs = make_rsrc(VI8 ? static_cast<const void*>(a.v_scales + sc_off) : nullptr, VI8 ? sc_bytes : 0u);

  // ---- query operand (B of S^T = K.Q^T): lane = (head c16, k-group q4) -------
  // k-step 2j+u of the contraction covers dims 64j + 16*q4 + 8u + [0, 8).
  f16x8 qb[NJ][2];
  float qsum[NJ];
  {
    const bool has = c16 < nh;
    const uint16_t* qp = a.q + ((int64_t)b * a.n_q + hq0 + (has ? c16 : 0)) * D + 16 * q4;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      u32x4 x0 = {0, 0, 0, 0}, x1 = {0, 0, 0, 0};
      if (has) {
        x0 = *reinterpret_cast<const u32x4*>(qp + 64 * j);
        x1 = *reinterpret_cast<const u32x4*>(qp + 64 * j + 8);
      }
      qb[j][0] = __builtin_bit_cast(f16x8, x0);
      qb[j][1] = __builtin_bit_cast(f16x8, x1);
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += (float)qb[j][0][e] + (float)qb[j][1][e];
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      qsum[j] = s;  // sum of q over the 64 dims of block j, for head c16
    }
  }
  // Accumulator start values that cancel the +1152 code bias (per scale group).
  f32x4 cinit[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float s = 0.0f;
    if (G64) {
      s = qsum[g];
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j) s += qsum[j];
    }
    const float v = KI8 ? -kCodeBias * s : 0.0f;
    cinit[g] = (f32x4){v, v, v, v};
  }

  f32x4 acc_o[VB];
#pragma unroll
  for (int t = 0; t < VB; ++t) acc_o[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  f32x4 acc_l = {0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;
  const f16x8 ones = {(f16)1, (f16)1, (f16)1, (f16)1, (f16)1, (f16)1, (f16)1, (f16)1};

  for (int p0 = start + wv * kTile; p0 < end; p0 += NW * kTile) {
    // ---- issue all loads of the tile ----------------------------------------
    // K rows for the A operand: row c16 of C-tile ct is position p0 + 16ct + c16.
    u32x4 kr[2][NJ][KI8 ? 1 : 4];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int pk = p0 + 16 * ct + c16;
      const uint32_t off = pk < end ? (uint32_t)pk * krow : kOOB;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if (KI8) {
          kr[ct][j][0] = ld128(krs, off + 64 * j + 16 * q4);
        } else {
#pragma unroll
          for (int m = 0; m < (KI8 ? 1 : 4); ++m) kr[ct][j][m] = ld128(krs, off + 4 * (64 * j + 16 * q4) + 16 * m);
        }
      }
    }
    // K scales for the C layout: lane (head c16, rows 4*q4+i) -> positions
    // p0 + 16ct + 4q4 + i; all NG scales of the row.
    uint32_t ks[2][4][NG > 1 ? NG / 2 : 1];
    if (KI8) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ps = p0 + 16 * ct + 4 * q4 + i;
          const uint32_t off = ps < end ? (uint32_t)ps * srow : kOOB;
          if (NG == 4) {
            const u32x2 v = ld64(ksrs, off);
            ks[ct][i][0] = v.x;
            ks[ct][i][NG > 1 ? 1 : 0] = v.y;
          } else if (NG == 2) {
            ks[ct][i][0] = ld32(ksrs, off);
          } else {
            ks[ct][i][0] = ld16(ksrs, off);
          }
        }
    }
    // V rows for the B operand of P.V: lane = (dim block c16, k-group q4);
    // element e of the lane's k-slice is position p0 + kpos(e).
    constexpr int VW = (VB * VE) / 4;  // dwords of V per lane per position
    uint32_t vr[8][VW];
    uint32_t vs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int pv = p0 + (e < 4 ? 4 * q4 + e : 16 + 4 * q4 + (e - 4));
      const uint32_t off = pv < end ? (uint32_t)pv * vrow : kOOB;
      const uint32_t base = off + VB * VE * c16;
      if (VW == 1) {
        vr[e][0] = ld32(vrs, base);
      } else if (VW == 2) {
        const u32x2 v = ld64(vrs, base);
        vr[e][0] = v.x;
        vr[e][VW > 1 ? 1 : 0] = v.y;
      } else {
#pragma unroll
        for (int m = 0; m < VW / 4; ++m) {
          const u32x4 v = ld128(vrs, base + 16 * m);
          vr[e][4 * m + 0] = v.x;
          vr[e][4 * m + 1] = v.y;
          vr[e][4 * m + 2] = v.z;
          vr[e][4 * m + 3] = v.w;
        }
      }
      if (VI8) {
        const int grp = G64 ? (VB * c16) / 64 : 0;
        const uint32_t soff = pv < end ? (uint32_t)pv * srow + 2 * grp : kOOB;
        vs[e] = ld16(vsrs, soff);
      }
    }

    // ---- S^T = K . Q^T ------------------------------------------------------
    float z[2][4];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      f32x4 zz = {0.f, 0.f, 0.f, 0.f};
      if (KI8 && G64) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const u32x4 c = kr[ct][j][0];
          f32x4 acc = mfma16(codes8_biased(c.x, c.y), qb[j][0], cinit[j]);
          acc = mfma16(codes8_biased(c.z, c.w), qb[j][1], acc);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t pr = ks[ct][i][j / 2];
            const float sc = h_bits_to_f32((j & 1) ? (pr >> 16) : (pr & 0xffffu));
            zz[i] = fmaf(acc[i], sc, zz[i]);
          }
        }
      } else if (KI8) {
        f32x4 acc = cinit[0];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const u32x4 c = kr[ct][j][0];
          acc = mfma16(codes8_biased(c.x, c.y), qb[j][0], acc);
          acc = mfma16(codes8_biased(c.z, c.w), qb[j][1], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) zz[i] = acc[i] * h_bits_to_f32(ks[ct][i][0] & 0xffffu);
      } else {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          acc = mfma16(f32x8_to_f16x8(kr[ct][j][0], kr[ct][j][KI8 ? 0 : 1]), qb[j][0], acc);
          acc = mfma16(f32x8_to_f16x8(kr[ct][j][KI8 ? 0 : 2], kr[ct][j][KI8 ? 0 : 3]), qb[j][1], acc);
        }
        zz = acc;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ps = p0 + 16 * ct + 4 * q4 + i;
        z[ct][i] = ps < end ? zz[i] * a.c2 : -INFINITY;
      }
    }

    // ---- online softmax (base 2) over the tile --------------------------------
    float tmax = z[0][0];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, z[ct][i]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));  // max over the tile for head c16
    const bool need = tmax > m_ref + kTau;
    if (__any(need)) {
      const float m_new = need ? tmax : m_ref;
      const float alpha = need ? exp2f(m_ref - m_new) : 1.0f;
      m_ref = m_new;
      // acc_o / acc_l rows are heads 4*q4 + i; lane h holds head h's alpha.
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * q4 + i);
#pragma unroll
        for (int t = 0; t < VB; ++t) acc_o[t][i] *= ai;
        acc_l[i] *= ai;
      }
    }
    const float mu = m_ref == -INFINITY ? 0.0f : m_ref;
    f16x8 pa;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) pa[4 * ct + i] = (f16)exp2f(z[ct][i] - mu);

    // ---- O += P . V_hat ;  l += P . 1 --------------------------------------------
    if (VI8) {
      f16x2 sv[4];
      constexpr uint32_t kNegBias = 0xE480E480u;  // fp16 pair (-1152, -1152)
#pragma unroll
      for (int pi = 0; pi < 4; ++pi) sv[pi] = as_h2((vs[2 * pi] & 0xffffu) | (vs[2 * pi + 1] << 16));
#pragma unroll
      for (int w = 0; w < VW; ++w) {
        uint32_t z01[4], z23[4];
#pragma unroll
        for (int pi = 0; pi < 4; ++pi) {
          z01[pi] = zip_lo(vr[2 * pi + 1][w], vr[2 * pi][w]) ^ kCodeFlip;
          z23[pi] = zip_hi(vr[2 * pi + 1][w], vr[2 * pi][w]) ^ kCodeFlip;
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
          acc_o[4 * w + bb] = mfma16(pa, __builtin_bit_cast(f16x8, r), acc_o[4 * w + bb]);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < VB; ++t) {
        u32x4 r;
#pragma unroll
        for (int pi = 0; pi < 4; ++pi)
          r[pi] = as_u32(__builtin_bit_cast(
              f16x2, __builtin_amdgcn_cvt_pkrtz(__builtin_bit_cast(float, vr[2 * pi][t]),
                                                __builtin_bit_cast(float, vr[2 * pi + 1][t]))));
        acc_o[t] = mfma16(pa, __builtin_bit_cast(f16x8, r), acc_o[t]);
      }
    }
    acc_l = mfma16(pa, ones, acc_l);
  }

  // ---- merge the wavefronts of the workgroup -----------------------------------
  __shared__ float sm_m[NW][16];
  __shared__ float sm_l[NW][16];
  __shared__ __attribute__((aligned(16))) float sm_o[16 * D];
  if (q4 == 0) sm_m[wv][c16] = m_ref;
  if (c16 == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sm_l[wv][4 * q4 + i] = acc_l[i];
  }
  __syncthreads();
  float mrow[4], frow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * q4 + i;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < NW; ++k) M = fmaxf(M, sm_m[k][h]);
    mrow[i] = M;
    const float mw = sm_m[wv][h];
    frow[i] = (mw == -INFINITY) ? 0.0f : exp2f(mw - M);
  }
  // O rows of this lane: heads 4*q4+i, dims VB*c16 + t.
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    if (wv == k) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * q4 + i;
        if (h < nh) {
          float* dst = sm_o + h * D + VB * c16;
#pragma unroll
          for (int t4 = 0; t4 < VB / 4; ++t4) {
            float4 v = {acc_o[4 * t4 + 0][i] * frow[i], acc_o[4 * t4 + 1][i] * frow[i],
                        acc_o[4 * t4 + 2][i] * frow[i], acc_o[4 * t4 + 3][i] * frow[i]};
            float4* d4 = reinterpret_cast<float4*>(dst + 4 * t4);
            if (k > 0) {
              const float4 o = *d4;
              v.x += o.x;
              v.y += o.y;
              v.z += o.z;
              v.w += o.w;
            }
            *d4 = v;
          }
        }
      }
    }
    __syncthreads();
  }
  // ---- write the split's partial -----------------------------------------------
  const int64_t row0 = ((int64_t)b * a.n_q + hq0) * a.n_splits + split;
  for (int idx = threadIdx.x; idx < nh * (D / 4); idx += NW * 64) {
    const int h = idx / (D / 4);
    const int d4 = idx % (D / 4);
    const float4 v = reinterpret_cast<const float4*>(sm_o + h * D)[d4];
    reinterpret_cast<float4*>(a.ws_o + (row0 + (int64_t)h * a.n_splits) * D)[d4] = v;
  }
  if (threadIdx.x < nh) {
    const int h = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < NW; ++k) M = fmaxf(M, sm_m[k][h]);
    float l = 0.0f;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const float mk = sm_m[k][h];
      if (mk != -INFINITY) l += sm_l[k][h] * exp2f(mk - M);
    }
    float2* ml = reinterpret_cast<float2*>(a.ws_ml) + row0 + (int64_t)h * a.n_splits;
    *ml = make_float2(M, l);
  }
  (void)mrow;
}

template <int D, bool KI8, bool VI8, bool G64>
static void launch_partial_t(const PartialArgs& a, dim3 grid, hipStream_t s) {
  constexpr int NW = 4;
  hipLaunchKernelGGL((kvq_partial_kernel<D, KI8, VI8, G64, NW>), grid, dim3(NW * 64), 0, s, a);
}

template <int D>
static int dispatch_dtypes(const kvq_layout& L, const PartialArgs& a, dim3 grid, hipStream_t s) {
  const bool ki8 = L.k_dtype == KVQ_STORE_INT8, vi8 = L.v_dtype == KVQ_STORE_INT8;
  const bool g64 = L.scale_group == 64 && L.head_dim != 64;  // at D = 64 both granularities coincide
  if (ki8 && vi8) {
    if (g64) launch_partial_t<D, true, true, true>(a, grid, s);
    else launch_partial_t<D, true, true, false>(a, grid, s);
  } else if (ki8) {
    if (g64) launch_partial_t<D, true, false, true>(a, grid, s);
    else launch_partial_t<D, true, false, false>(a, grid, s);
  } else if (vi8) {
    if (g64) launch_partial_t<D, false, true, true>(a, grid, s);
    else launch_partial_t<D, false, true, false>(a, grid, s);
  } else {
    launch_partial_t<D, false, false, false>(a, grid, s);
  }
  return KVQ_OK;
}

int launch_partial(const kvq_layout& L, const void* k_store, const void* v_store,
                   const uint16_t* k_scales, const uint16_t* v_scales, const uint16_t* q,
                   int32_t batch, int32_t n_q_heads, const int32_t* d_seq_lens, int32_t window,
                   float sm_scale, const kvq_plan_t& plan, void* ws, void* stream) {
  PartialArgs a{};
  a.k_store = k_store;
  a.v_store = v_store;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.q = q;
  a.seq_lens = d_seq_lens;
  const int64_t rows = (int64_t)batch * n_q_heads * plan.n_splits;
  a.ws_o = static_cast<float*>(ws);
  a.ws_ml = static_cast<float*>(ws) + rows * L.head_dim;
  a.s_seq = L.s_seq;
  a.s_pos = L.s_pos;
  a.s_head = L.s_head;
  a.ss_seq = L.ss_seq;
  a.ss_pos = L.ss_pos;
  a.ss_head = L.ss_head;
  a.max_ctx = L.max_ctx > 0x7fffffff ? 0x7fffffff : (int32_t)L.max_ctx;
  a.n_kv = L.n_kv_heads;
  a.G = n_q_heads / L.n_kv_heads;
  a.n_q = n_q_heads;
  a.head_blocks = (a.G + kHeadsPerBlock - 1) / kHeadsPerBlock;
  a.n_splits = plan.n_splits;
  a.chunk = plan.chunk;
  a.window = window;
  a.c2 = sm_scale * kLog2e;
  dim3 grid(plan.n_splits, L.n_kv_heads * a.head_blocks, batch);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int st;
  switch (L.head_dim) {
    case 64: st = dispatch_dtypes<64>(L, a, grid, s); break;
    case 128: st = dispatch_dtypes<128>(L, a, grid, s); break;
    case 256: st = dispatch_dtypes<256>(L, a, grid, s); break;
    default: return KVQ_ERR_UNSUPPORTED;
  }
  if (st) return st;
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace kvq
