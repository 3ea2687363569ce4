// kv_chunk_attn for the 4-bit layouts (q4_0: q4 K and V; k8v4: int8 K, q4 V),
// head_dim 256: attention of a chunk of consecutive query tokens per sequence
// over Q4_0 blocks of rotated rows.
//
// Strata PR 2698, "What it does": the prompt chunk and the verify windows read
// the same cache as decode; "Not in this PR": the 4-bit stores keep rows
// rotated by the 256-point Hadamard transform, the queries are rotated with
// the keys and the output is rotated back.
//
// Mapping, data movement and the causal/window semantics are those of the int8
// chunk kernel (kvq_chunk.hip): one workgroup = (sequence, kv head, 64 query
// rows t * G + h, key split); every wavefront walks every 32-position tile of
// a three-stage direct-to-LDS ring whose loads are spread over the
// wavefronts; the value tile is dequantized once per workgroup into a
// transposed fp16 tile; O^T += V_hat^T . P^T leaves each lane with values of
// its own query row. The 4-bit parts:
//   query   a lane's 64 query values (dims 32 j + 8 q4 + e of its row, the
//           operand of block j) are rotated in registers before any score:
//           the butterflies over e and j run inside the lane, those over q4
//           between the four lanes of the row (q4 keys only; k8v4 keys use
//           the unrotated query and the int8 kernel's operands);
//   keys    exact scores: the codes enter the MFMA as the fp16 subnormals
//           code * 2^-24, one MFMA per Q4_0 block and per half of the query
//           (the rotated query is carried as hi + lo fp16 terms), each block's
//           product scaled by its fp16 scale in fp32, and the -8 offset of the
//           codes taken by one more MFMA per 16 positions (the positions'
//           block scales times the query's block sums);
//   values  nibbles of 4 dims x 8 positions per lane to fp16((q - 8) * d);
//   output  each lane's 64 output values of its row are rotated back in
//           registers (dims 16 mt + 4 q4 + i: butterflies over i and mt
//           inside the lane, over q4 between lanes) before they are stored.
#include <math.h>

#include "kvq_chunk_tile.h"
#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_q4.h"
#include "kvq_q4_tile.h"
#include "kvq_tile.h"

namespace kvq {

struct ChunkQ4Args {
  const void* k_store;
  const void* v_store;
  const uint16_t* k_scales;
  const uint16_t* v_scales;
  const uint16_t* q;          // fp16 [B][T][Hq][D]
  const int32_t* start_pos;   // [B]: position of token 0
  float* ws_o;                // [B*T][Hq][n_splits][D]
  float* ws_ml;               // [B*T][Hq][n_splits][2]
  int64_t s_seq, s_pos, s_head;     // element strides (a q4 element is half a byte)
  int64_t ss_seq, ss_pos, ss_head;  // fp16 scale strides
  int32_t max_ctx;
  int32_t n_kv, G, n_q, T, row_blocks;
  int32_t n_splits, chunk, window;
  float c2;  // sm_scale * log2(e)
};

// Butterfly (a, b) -> (a + b, a - b) of two registers of one lane.
__device__ __forceinline__ void bfly(float& a, float& b) {
  const float s = a + b, d = a - b;
  a = s;
  b = d;
}

// Butterfly between lane l and lane l ^ m (the lane with bit m clear keeps the
// sum), for every value of the lane.
template <int N>
__device__ __forceinline__ void bfly_lanes(float (&x)[N], int lane, int m) {
  const float sgn = (lane & m) ? -1.0f : 1.0f;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const float p = __shfl_xor(x[k], m);
    x[k] = fmaf(sgn, x[k], p);
  }
}

// Rotation y = H x / 16 of the query row held by the four lanes c16 + 16 q4:
// x[8 j + e] = dim 32 j + 8 q4 + e. Index bits 0-2 are e, 3-4 are q4 (lanes
// 16 and 32 apart), 5-7 are j.
__device__ __forceinline__ void rotate_query_row(float (&x)[64], int lane) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int k = 0; k < 64; ++k)
      if ((k & h) == 0) bfly(x[k], x[k + h]);
  bfly_lanes(x, lane, 16);
  bfly_lanes(x, lane, 32);
#pragma unroll
  for (int h = 8; h < 64; h <<= 1)
#pragma unroll
    for (int k = 0; k < 64; ++k)
      if ((k & h) == 0) bfly(x[k], x[k + h]);
#pragma unroll
  for (int k = 0; k < 64; ++k) x[k] *= 0.0625f;
}

// Rotation back of the output row held as acc.o[mt][i] = dim 16 mt + 4 q4 + i
// by the four lanes of the row: bits 0-1 are i, 2-3 are q4, 4-7 are mt.
__device__ __forceinline__ void rotate_output_row(RowAcc<256>& acc, int lane) {
  float x[64];
#pragma unroll
  for (int mt = 0; mt < 16; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[4 * mt + i] = acc.o[mt][i];
#pragma unroll
  for (int h = 1; h < 64; h <<= 1)
#pragma unroll
    for (int k = 0; k < 64; ++k)
      if ((k & h) == 0) bfly(x[k], x[k + h]);  // h = 1, 2 (i) and 4 .. 32 (mt)
  bfly_lanes(x, lane, 16);
  bfly_lanes(x, lane, 32);
#pragma unroll
  for (int mt = 0; mt < 16; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc.o[mt][i] = x[4 * mt + i] * 0.0625f;
}

// fp16 element j of 8 packed values, widened.
__device__ __forceinline__ float half8(const u32x4& w, int j) {
  const uint32_t d = w[j >> 1];
  return h_bits_to_f32((j & 1) ? (d >> 16) : (d & 0xffffu));
}

// Exact scores of a q4 key tile read straight from stage `st`: z[ct][i] for
// positions x = 16 ct + 4 q4 + i of the lane's row (log2 domain), positions
// outside [vlo, vhi) at -inf. qh[j] + ql[j] = the rotated query's dims
// 32 j + 8 q4 .. +7; sh_q + sl_q = its 8 block sums in k slots 0..7 of the
// lanes with q4 = 0 (zeros elsewhere); c2s = sm_scale * log2(e) * 2^24.
//   z = 2^24 sum_b d_b sum_d (code_d * 2^-24) q_d  -  8 sum_b d_b Q_b
template <bool KG64>
__device__ __forceinline__ void scores_q4_exact(const uint8_t* __restrict__ st, int vlo, int vhi, float (&z)[2][4],
                                                const f16x8 (&qh)[8], const f16x8 (&ql)[8], f16x8 sh_q, f16x8 sl_q,
                                                float c2s, int c16, int q4) {
  using T = Q4Stage<true, KG64>;
  const uint32_t sh = 4u * (uint32_t)(q4 >> 1);
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int r = 16 * ct + c16;
    const f16x8 own = *reinterpret_cast<const f16x8*>(st + T::KS_OFF + r * 16);  // scale row of row r
    f32x4 c = mfma16(own, sh_q, zero);
    c = mfma16(own, sl_q, c);
    u32x4 sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = *reinterpret_cast<const u32x4*>(st + T::KS_OFF + (16 * ct + 4 * q4 + i) * 16);
    f32x4 zz;
#pragma unroll
    for (int i = 0; i < 4; ++i) zz[i] = c[i] * (-8.0f / 16777216.0f);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const u32x2 k = *reinterpret_cast<const u32x2*>(st + T::K_OFF + r * T::KRB + 16 * (j ^ swz<8>(r)) + 8 * (q4 & 1));
      const uint32_t w0 = (k.x >> sh) & 0x0F0F0F0Fu;
      const uint32_t w1 = (k.y >> sh) & 0x0F0F0F0Fu;
      const u32x4 a4 = {sub_h2_lo(w0), sub_h2_hi(w0), sub_h2_lo(w1), sub_h2_hi(w1)};  // code * 2^-24
      f32x4 a = mfma16(__builtin_bit_cast(f16x8, a4), qh[j], zero);
      a = mfma16(__builtin_bit_cast(f16x8, a4), ql[j], a);
#pragma unroll
      for (int i = 0; i < 4; ++i) zz[i] = fmaf(a[i], half8(sc[i], j), zz[i]);
      if ((j & 1) == 1) __builtin_amdgcn_sched_barrier(0);  // two blocks' products live at a time
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int x = 16 * ct + 4 * q4 + i;
      z[ct][i] = (x >= vlo && x < vhi) ? zz[i] * c2s : -INFINITY;
    }
  }
}

// This wavefront's quarter of the q4 value tile in stage `st`, dequantized to
// fp16((q - 8) * d) and stored transposed (as the int8 chunk kernel's
// convert_v): lane (dim quad d0, slot block qb) converts 4 dims x 8 positions.
template <bool KQ4, bool KG64>
__device__ __forceinline__ void convert_v_q4(const uint8_t* __restrict__ st, uint8_t* __restrict__ vt, int wv,
                                             int lane) {
  using T = Q4Stage<KQ4, KG64>;
  const int qb = lane & 3;
  const int d0 = 4 * (wv * 16 + (lane >> 2));
  const int blk = d0 >> 5;              // Q4_0 block of the four dims
  const int byte = d0 & 15;             // their bytes in the block
  const uint32_t sh = (d0 & 16) >> 2;   // dims 16..31 of a block: high nibbles
  uint32_t v01[8], v23[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int r = kpos(e, qb);
    const uint32_t raw = *reinterpret_cast<const uint32_t*>(st + T::V_OFF + r * T::VRB + 16 * (blk ^ swz<8>(r)) + byte);
    const uint32_t codes = (raw >> sh) & 0x0F0F0F0Fu;
    const uint32_t sb = *reinterpret_cast<const uint16_t*>(st + T::VS_OFF + r * 16 + 2 * blk);
    const f16x2 s2 = as_h2(sb | (sb << 16));
    v01[e] = as_u32((as_h2(biased_h2_lo(codes)) + as_h2(kQ4NegBias)) * s2);
    v23[e] = as_u32((as_h2(biased_h2_hi(codes)) + as_h2(kQ4NegBias)) * s2);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t* src = k < 2 ? v01 : v23;
    const uint32_t sel = (k & 1) ? 0x07060302u : 0x05040100u;
    u32x4 w;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) w[e2] = __builtin_amdgcn_perm(src[2 * e2 + 1], src[2 * e2], sel);
    *reinterpret_cast<u32x4*>(vt + (d0 + k) * kVtPitch + 16 * qb) = w;
  }
}

template <bool KQ4, bool KG64>
__global__ __launch_bounds__(kChunkWaves * 64, 2) void kvq_chunk_q4_kernel(ChunkQ4Args a) {
  constexpr int D = 256;
  constexpr int NW = kChunkWaves;
  constexpr int ROWS = 16 * NW;
  using T = Q4Stage<KQ4, KG64>;
  using SK = Shape<256, true, true, KG64>;  // int8 keys (k8v4)
  constexpr int NIK = 32 * T::KRB / 1024;   // 1 KiB code loads of a key tile
  constexpr int NIV = 32 * T::VRB / 1024;   // of a value tile
  constexpr int NL = NIK + NIV + 2;         // direct-to-LDS loads per tile
  __shared__ __attribute__((aligned(16))) uint8_t lds_st[kChunkStages][T::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_vt[D * kVtPitch];

  const int split = blockIdx.x;
  const int hk = blockIdx.y / a.row_blocks;
  const int rblk = blockIdx.y % a.row_blocks;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;
  const int q4 = lane >> 4;
  const int G = a.G;

  // ---- rows of the workgroup and the keys they may see (as the int8 kernel)
  const int fr0 = rblk * ROWS;
  const int t_first = fr0 / G;
  const int t_last = min(a.T - 1, (fr0 + ROWS - 1) / G);
  int s0 = a.start_pos[b];
  s0 = s0 < 0 ? 0 : (s0 > a.max_ctx ? a.max_ctx : s0);
  const int hi_all = min(s0 + t_last + 1, a.max_ctx);
  const int lo_all = a.window > 0 ? max(0, s0 + t_first + 1 - a.window) : 0;
  // split * chunk in 64 bits: the split's first key may lie far past hi_all
  const int64_t start64 = (int64_t)lo_all + (int64_t)split * a.chunk;
  const int start = (int)min(start64, (int64_t)hi_all);
  const int end = (split == a.n_splits - 1) ? hi_all : (int)min((int64_t)hi_all, start64 + a.chunk);

  const int fr = fr0 + 16 * wv + c16;  // the lane's flat row t * G + h
  const int tok = fr / G;
  const bool valid = tok < a.T;
  const int64_t id = valid ? (((int64_t)b * a.T + tok) * a.n_q + hk * G + fr % G) * a.n_splits + split : -1;
  float2* const ml = reinterpret_cast<float2*>(a.ws_ml);
  if (start >= end) {  // nothing to attend in this split: empty partials
    if (q4 == 0 && id >= 0) ml[id] = make_float2(-INFINITY, 0.0f);
    return;
  }
  const int P = s0 + tok;
  const int vhi = (valid && P < a.max_ctx) ? P + 1 : 0;
  const int vlo = a.window > 0 ? max(0, P + 1 - a.window) : 0;

  // ---- the lane's query operands, in registers (loaded and used before any
  // direct-to-LDS load, so the compiler's wait for them covers nothing else)
  const uint16_t* qrow = a.q + (((int64_t)b * a.T + (valid ? tok : 0)) * a.n_q + hk * G + fr % G) * D;
  f16x8 qv[8], qlo[8];   // q4 keys: block j = rotated dims 32 j + 8 q4 .. +7, as hi + lo fp16
  f16x8 sq_hi = {}, sq_lo = {};  // q4 keys: the rotated block sums (k slots 0..7 of q4 = 0 lanes)
  f16x8 qi[4][2];        // int8 keys: dims 64 j + 16 q4 + 8 u .. +7
  float corr[SK::NG];
  if constexpr (KQ4) {
    float x[64];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (valid) v = *reinterpret_cast<const u32x4*>(qrow + 32 * j + 8 * q4);
      const f16x8 h = __builtin_bit_cast(f16x8, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[8 * j + e] = (float)h[e];
    }
    rotate_query_row(x, lane);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float sum = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const f16 h = (f16)x[8 * j + e];
        qv[j][e] = h;
        qlo[j][e] = (f16)(x[8 * j + e] - (float)h);
        sum += x[8 * j + e];
      }
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      const f16 hi = (f16)sum;
      sq_hi[j] = q4 == 0 ? hi : (f16)0.0f;
      sq_lo[j] = q4 == 0 ? (f16)(sum - (float)hi) : (f16)0.0f;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (valid) v = *reinterpret_cast<const u32x4*>(qrow + 64 * j + 16 * q4 + 8 * u);
        qi[j][u] = __builtin_bit_cast(f16x8, v);
      }
    float qsum[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += (float)qi[j][0][e] + (float)qi[j][1][e];
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      qsum[j] = s;
    }
#pragma unroll
    for (int g = 0; g < SK::NG; ++g)
      corr[g] = -kCodeBias * (KG64 ? qsum[g] : qsum[0] + qsum[1] + qsum[2] + qsum[3]);
  }

  // ---- key tiles: buffer resources of this (sequence, kv head) slice
  const int64_t st_off = (int64_t)b * a.s_seq + (int64_t)hk * a.s_head;  // elements
  const int64_t sc_off = (int64_t)b * a.ss_seq + (int64_t)hk * a.ss_head;
  const int64_t last = (int64_t)(hi_all - 1) * a.s_pos + D;
  const uint32_t krow = (uint32_t)(KQ4 ? a.s_pos / 2 : a.s_pos);
  const uint32_t vrow = (uint32_t)(a.s_pos / 2);
  const uint32_t srow = (uint32_t)(a.ss_pos * 2);
  const u32x4 krw = rsrc_words(static_cast<const char*>(a.k_store) + (KQ4 ? st_off / 2 : st_off),
                               (uint32_t)(KQ4 ? last / 2 : last));
  const u32x4 vrw = rsrc_words(static_cast<const char*>(a.v_store) + st_off / 2, (uint32_t)(last / 2));
  const u32x4 ksrw = rsrc_words(a.k_scales + sc_off, (uint32_t)(((int64_t)(hi_all - 1) * a.ss_pos + T::KNG) * 2));
  const u32x4 vsrw = rsrc_words(a.v_scales + sc_off, (uint32_t)(((int64_t)(hi_all - 1) * a.ss_pos + D / kQ4Block) * 2));

  // Load i of a tile: K code chunks, V code chunks, K scale rows, V scale rows.
  auto issue_one = [&](int i, uint32_t base, uint32_t ksoff, uint32_t vsoff, uint32_t ssoff, int nvalid) {
    if (i < NIK + NIV) {
      const bool k = i < NIK;
      const int ci = k ? i : i - NIK;
      const int ch = (k ? T::KRB : T::VRB) / 16;
      const int slot = ci * 64 + lane;
      const int r = slot / ch;
      const int c = (slot % ch) ^ (k && !KQ4 ? swz<16>(r) : swz<8>(r));
      const uint32_t voff = r < nvalid ? (uint32_t)r * (k ? krow : vrow) + 16 * c : kOOB;
      dma<16>(k ? krw : vrw, base + (k ? T::K_OFF : T::V_OFF) + 1024 * ci, voff, k ? ksoff : vsoff);
    } else if (i == NIK + NIV) {
      issue_scales<T::KSB>(base + T::KS_OFF, ksrw, ssoff, nvalid, srow, lane);
    } else {
      issue_scales<16>(base + T::VS_OFF, vsrw, ssoff, nvalid, srow, lane);
    }
  };
  auto issue_role = [&](const int w, uint32_t base, uint32_t ksoff, uint32_t vsoff, uint32_t ssoff, int nvalid) {
#pragma unroll
    for (int k = 0; k < (NL + NW - 1) / NW; ++k)
      if (w + NW * k < NL) issue_one(w + NW * k, base, ksoff, vsoff, ssoff, nvalid);
  };
  auto issue_tile = [&](int stage, int p0) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int nvalid = min(kTile, end - p0);
    const uint32_t base = lds_addr_of(&lds_st[stage][0]);
    const uint32_t ksoff = __builtin_amdgcn_readfirstlane((uint32_t)p0 * krow);
    const uint32_t vsoff = __builtin_amdgcn_readfirstlane((uint32_t)p0 * vrow);
    const uint32_t ssoff = __builtin_amdgcn_readfirstlane((uint32_t)p0 * srow);
    switch (wv) {
      case 0: issue_role(0, base, ksoff, vsoff, ssoff, nvalid); break;
      case 1: issue_role(1, base, ksoff, vsoff, ssoff, nvalid); break;
      case 2: issue_role(2, base, ksoff, vsoff, ssoff, nvalid); break;
      default: issue_role(3, base, ksoff, vsoff, ssoff, nvalid); break;
    }
  };
  static_assert(NW == 4, "issue_tile assigns four wavefront roles");
  auto wait_all_but_next = [&]() {
    if (wv < NL % NW) wait_vm<NL / NW + 1>();
    else wait_vm<NL / NW>();
  };

  RowAcc<D> acc;
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt) acc.o[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  acc.l = (f32x4){0.f, 0.f, 0.f, 0.f};
  acc.m_ref = -INFINITY;
  const f16x8 ones = {(f16)1, (f16)1, (f16)1, (f16)1, (f16)1, (f16)1, (f16)1, (f16)1};

  const int n_tiles = (end - start + kTile - 1) / kTile;
  issue_tile(0, start);
  if (n_tiles > 1) issue_tile(1, start + kTile);
  for (int t = 0; t < n_tiles; ++t) {
    if (t + 1 < n_tiles) wait_all_but_next();  // own share of tile t landed; tile t+1 may still load
    else wait_vm<0>();
    // Every wavefront's share of tile t is in LDS, and every wavefront is done
    // with tile t-1 (its stage, which the tile t+2 loads reuse, and the value tile).
    asm volatile("s_barrier" ::: "memory");
    if (t + 2 < n_tiles) issue_tile((t + 2) % kChunkStages, start + (t + 2) * kTile);
    const uint8_t* st = &lds_st[t % kChunkStages][0];
    const int p0 = start + t * kTile;
    convert_v_q4<KQ4, KG64>(st, lds_vt, wv, lane);
    float z[2][4];
    if constexpr (KQ4) {
      scores_q4_exact<KG64>(st, max(vlo, p0) - p0, min(vhi, end) - p0, z, qv, qlo, sq_hi, sq_lo,
                            a.c2 * 16777216.0f, c16, q4);
    } else {
      KRegs<SK> tk;
      read_k_i8<KG64>(tk, st, c16, q4);
      scores_i8<KG64>(tk, max(vlo, p0) - p0, min(vhi, end) - p0, z, qi, corr, a.c2, q4);
    }
    const f16x8 pa = row_softmax<D>(z, acc);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // the value tile is complete
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) {
      const f16x8 v = *reinterpret_cast<const f16x8*>(lds_vt + (16 * mt + c16) * kVtPitch + 16 * q4);
      acc.o[mt] = mfma16(v, pa, acc.o[mt]);
    }
    acc.l = mfma16(ones, pa, acc.l);
  }

  // ---- the lane's row back to the original basis, then its partials: lane
  // (c16, q4) writes dims 16 mt + 4 q4 + [0, 4), lanes q4 = 0 the (max, sum)
  rotate_output_row(acc, lane);
  if (id >= 0) {
    float* o = a.ws_o + id * D + 4 * q4;
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt)
      *reinterpret_cast<float4*>(o + 16 * mt) = make_float4(acc.o[mt][0], acc.o[mt][1], acc.o[mt][2], acc.o[mt][3]);
    if (q4 == 0) ml[id] = make_float2(acc.m_ref, acc.l[0]);
  }
}

int launch_chunk_q4(const kvq_layout& L, const void* k_store, const void* v_store, const uint16_t* k_scales,
                    const uint16_t* v_scales, const uint16_t* q, int32_t batch, int32_t n_tok, int32_t n_q_heads,
                    const int32_t* d_start_pos, int32_t window, float sm_scale, const kvq_plan_t& plan, void* ws,
                    void* stream) {
  if (L.head_dim != 256 || !q4_decode_supported(L)) return KVQ_ERR_UNSUPPORTED;
  ChunkQ4Args a{};
  a.k_store = k_store;
  a.v_store = v_store;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.q = q;
  a.start_pos = d_start_pos;
  const int64_t rows = (int64_t)batch * n_tok * n_q_heads * plan.n_splits;
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
  a.T = n_tok;
  a.row_blocks = chunk_row_blocks(n_tok, a.G, L.head_dim);
  a.n_splits = plan.n_splits;
  a.chunk = plan.chunk;
  a.window = window;
  a.c2 = sm_scale * kLog2e;
  const dim3 grid(plan.n_splits, L.n_kv_heads * a.row_blocks, batch);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (L.k_dtype == KVQ_STORE_Q4)
    hipLaunchKernelGGL((kvq_chunk_q4_kernel<true, false>), grid, dim3(kChunkWaves * 64), 0, s, a);
  else if (L.scale_group == 64)
    hipLaunchKernelGGL((kvq_chunk_q4_kernel<false, true>), grid, dim3(kChunkWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL((kvq_chunk_q4_kernel<false, false>), grid, dim3(kChunkWaves * 64), 0, s, a);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace kvq
