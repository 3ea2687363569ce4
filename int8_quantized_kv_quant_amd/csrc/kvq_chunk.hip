// kv_chunk_attn: attention of a chunk of consecutive query tokens per sequence
// (a prompt chunk, or the few tokens of a verify window) over the int8 KV
// cache, on the gfx950 matrix cores.
//
// Strata PR 2698, "What it does": the prompt chunk and the verify windows read
// the same int8 cache as decode, dequantized on the fly. genie-ai-runtime
// release v0.1.0-alpha.11, "--int8-kv triage": the batched prefill attention
// must read the INT8 cache with its per-(position, kv head) scales, not fall
// back to one decode call per token. genie v1.3.0 "split-K decode attention":
// online-softmax partials per key range, combined by a reduce.
//
// Semantics. Token t of sequence b sits at position P = start_b + t (its own K
// and V rows are already in the cache) and attends to the keys lo <= p <= P,
// lo = max(0, P + 1 - window) for window > 0: causal inside the chunk.
//
// Mapping. One workgroup = (sequence b, kv head, block of 64 query rows, key
// split). Query rows are the (token, head) pairs of the chunk that share the
// kv head, flattened as row = t * G + h; each of the 4 wavefronts owns 16 of
// them as the 16-wide side of the MFMA, with its query operands in registers.
// Every wavefront walks every 32-position key tile of the split, so one tile
// staged in LDS feeds 64 query rows. Per tile and wavefront, exactly as in the
// decode kernel: S^T = K.Q^T (codes as exact fp16, per-group fp32 scaling),
// base-2 online softmax with a per-row causal/window mask, O += P.V_hat.
//
// Data movement. Key tiles go HBM -> LDS through a ring of three stages with
// direct-to-LDS loads; the loads of one tile are spread over the four
// wavefronts, and one barrier per tile publishes a landed tile to all of them
// while the next two tiles are in flight. The workgroup's keys end at the last
// position its tokens may see, so no tile above the diagonal is loaded.
//
// Output. Each wavefront writes the (max, sum, O) partials of its own rows in
// the decode layout, for rows (b, t, hq) in place of (b, hq); the reduce kernel
// combines the splits into fp16.
#include <math.h>

#include "kvq_chunk_tile.h"
#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_tile.h"

namespace kvq {

struct ChunkArgs {
  const void* k_store;
  const void* v_store;
  const uint16_t* k_scales;
  const uint16_t* v_scales;
  const uint16_t* q;          // fp16 [B][T][Hq][D]
  const int32_t* start_pos;   // [B]: position of token 0
  float* ws_o;                // [B*T][Hq][n_splits][D]
  float* ws_ml;               // [B*T][Hq][n_splits][2]
  int64_t s_seq, s_pos, s_head;
  int64_t ss_seq, ss_pos, ss_head;
  int32_t max_ctx;
  int32_t n_kv, G, n_q, T, row_blocks;
  int32_t n_splits, chunk, window;
  float c2;  // sm_scale * log2(e)
  uint32_t ws_bytes;  // partial region bytes when one buffer resource covers it (write-through stores), else 0
};

// This wavefront's quarter of the value tile in stage `st`, dequantized to
// fp16(code * scale) (the decode kernel's rounding) and stored transposed:
// lane (dim quad, slot block qb) converts 4 dims x 8 positions. The slot block
// is the fast lane index, so the 16 lanes of one LDS pass store to 16 distinct
// 16-byte bank groups (rows 80 bytes apart) and read 16 distinct dwords.
template <class S, int NW>
__device__ __forceinline__ void convert_v(const uint8_t* __restrict__ st, uint8_t* __restrict__ vt, int wv, int lane) {
  using ST = Stage<S>;
  constexpr int QPW = S::D / 4 / NW;  // dim quads per wavefront
  if (lane >= 4 * QPW) return;
  const int qb = lane & 3;
  const int d0 = 4 * (wv * QPW + (lane >> 2));
  const int grp = S::G64 ? d0 / 64 : 0;
  constexpr uint32_t kNegBias = 0xE480E480u;  // fp16 pair (-1152, -1152)
  uint32_t v01[8], v23[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int r = kpos(e, qb);
    const uint32_t codes =
        *reinterpret_cast<const uint32_t*>(st + ST::V_OFF + r * S::D + 16 * ((d0 / 16) ^ ST::swz(r)) + (d0 % 16));
    const uint32_t sb = *reinterpret_cast<const uint16_t*>(st + ST::VS_OFF + r * ST::SPITCH + 2 * grp);
    const f16x2 s2 = as_h2(sb | (sb << 16));
    const uint32_t fl = codes ^ kCodeFlip;
    v01[e] = as_u32((as_h2(biased_h2_lo(fl)) + as_h2(kNegBias)) * s2);
    v23[e] = as_u32((as_h2(biased_h2_hi(fl)) + as_h2(kNegBias)) * s2);
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

template <int D, bool G64, int RB>
__global__ __launch_bounds__(kChunkWaves * 64) void kvq_chunk_kernel(ChunkArgs a) {
  using S = Shape<D, true, true, G64>;
  using ST = Stage<S>;
  constexpr int NI = 32 * D / 1024;  // 1 KiB code loads per half tile
  constexpr int NL = 2 * NI + 2;     // direct-to-LDS loads per tile (codes + scale rows)
  constexpr int NW = kChunkWaves;
  constexpr int ROWS = 16 * RB * NW;  // query rows of the workgroup
  __shared__ __attribute__((aligned(16))) uint8_t lds_st[kChunkStages][ST::BYTES];
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

  // ---- rows of the workgroup and the keys they may see ------------------------
  const int fr0 = rblk * ROWS;                         // first flat row (t * G + h)
  const int t_first = fr0 / G;
  const int t_last = min(a.T - 1, (fr0 + ROWS - 1) / G);
  int s0 = a.start_pos[b];
  s0 = s0 < 0 ? 0 : (s0 > a.max_ctx ? a.max_ctx : s0);
  // Keys [lo_all, hi_all): up to the last token's own position (tokens that
  // would sit at or beyond max_ctx see nothing).
  const int hi_all = min(s0 + t_last + 1, a.max_ctx);
  const int lo_all = a.window > 0 ? max(0, s0 + t_first + 1 - a.window) : 0;
  // split * chunk in 64 bits: the split's first key may lie far past hi_all
  const int64_t start64 = (int64_t)lo_all + (int64_t)split * a.chunk;
  const int start = (int)min(start64, (int64_t)hi_all);
  const int end = (split == a.n_splits - 1) ? hi_all : (int)min((int64_t)hi_all, start64 + a.chunk);

  // Row block rb of this wavefront: flat rows fr0 + 16 * (RB * wv + rb) + c16.
  // The lane's row is the S^T column c16 and the O^T column c16.
  auto flat_row = [&](int rb) { return fr0 + 16 * (RB * wv + rb) + c16; };
  auto row_id = [&](int rb) -> int64_t {  // partial row of the lane's row in block rb, or -1
    const int fr = flat_row(rb);
    const int t = fr / G;
    if (t >= a.T) return -1;
    return (((int64_t)b * a.T + t) * a.n_q + hk * G + fr % G) * a.n_splits + split;
  };

  float2* const ml = reinterpret_cast<float2*>(a.ws_ml);
  // Partials written through the L2 (device-scope store bits) when one buffer
  // resource covers them, as the decode partial kernel writes its own: the
  // launch then ends without their write-back (for the chunk kernel the
  // measured difference stays within the ~1 % run-to-run spread of the
  // 2048-token prompt chunk).
  const auto wsr = make_rsrc(a.ws_o, a.ws_bytes);
  const uint32_t ml_base = (uint32_t)((a.ws_ml - a.ws_o) * 4);
  auto put_ml = [&](int64_t id, float2 v) {
    if (a.ws_bytes) __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), wsr, (int)(ml_base + id * 8), 0, 16);
    else ml[id] = v;
  };
  if (start >= end) {  // nothing to attend in this split: empty partials
    if (q4 == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int64_t id = row_id(rb);
        if (id >= 0) put_ml(id, make_float2(-INFINITY, 0.0f));
      }
    }
    return;
  }

  // ---- query operands of the lane's rows, in registers (loaded and used before
  // any direct-to-LDS load, so the compiler's wait for them covers nothing else)
  f16x8 qv[RB][S::NJ][2];
  float corr[RB][S::NG];
  int vlo[RB], vhi[RB];  // keys [vlo, vhi) of the lane's row in block rb
  bool has_row[RB];      // the lane's row in block rb is a token of the chunk
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int fr = flat_row(rb);
    const int t = fr / G;
    const bool valid = t < a.T;
    has_row[rb] = valid;
    const int P = s0 + t;
    vhi[rb] = (valid && P < a.max_ctx) ? P + 1 : 0;
    vlo[rb] = a.window > 0 ? max(0, P + 1 - a.window) : 0;
    const uint16_t* qrow = a.q + (((int64_t)b * a.T + t) * a.n_q + hk * G + fr % G) * D;
#pragma unroll
    for (int j = 0; j < S::NJ; ++j)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (valid) v = *reinterpret_cast<const u32x4*>(qrow + 64 * j + 16 * q4 + 8 * u);
        qv[rb][j][u] = __builtin_bit_cast(f16x8, v);
      }
    float qsum[S::NJ];
#pragma unroll
    for (int j = 0; j < S::NJ; ++j) {
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += (float)qv[rb][j][0][e] + (float)qv[rb][j][1][e];
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      qsum[j] = s;
    }
#pragma unroll
    for (int g = 0; g < S::NG; ++g) {
      float t2 = 0.0f;
      if (G64) {
        t2 = qsum[g];
      } else {
#pragma unroll
        for (int j = 0; j < S::NJ; ++j) t2 += qsum[j];
      }
      corr[rb][g] = -kCodeBias * t2;
    }
  }

  // The keys every row of this wavefront keeps, [lo_all_w, hi_all_w)
  // (wavefront-uniform): a tile inside it needs no mask. Rows past the chunk
  // are written nowhere and do not count; a token at or past max_ctx (no key
  // at all) does, so its wavefront always masks.
  int row_lo = 0, row_hi = 0x7fffffff;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    if (has_row[rb]) {
      row_lo = max(row_lo, vlo[rb]);
      row_hi = min(row_hi, vhi[rb]);
    }
  row_lo = max(row_lo, lane_xor<8>(row_lo));
  row_lo = max(row_lo, lane_xor<4>(row_lo));
  row_lo = max(row_lo, lane_xor<2>(row_lo));
  row_lo = max(row_lo, lane_xor<1>(row_lo));
  row_hi = min(row_hi, lane_xor<8>(row_hi));
  row_hi = min(row_hi, lane_xor<4>(row_hi));
  row_hi = min(row_hi, lane_xor<2>(row_hi));
  row_hi = min(row_hi, lane_xor<1>(row_hi));
  const int lo_all_w = __builtin_amdgcn_readfirstlane(row_lo);  // the 16 rows of lanes 0-15 (q4 lanes repeat them)
  const int hi_all_w = __builtin_amdgcn_readfirstlane(row_hi);

  // ---- key tiles: buffer resources of this (sequence, kv head) slice ----------
  const uint32_t row = (uint32_t)a.s_pos;
  const uint32_t srow = (uint32_t)(a.ss_pos * 2);
  const int64_t st_off = (int64_t)b * a.s_seq + (int64_t)hk * a.s_head;
  const int64_t sc_off = (int64_t)b * a.ss_seq + (int64_t)hk * a.ss_head;
  const u32x4 krw = rsrc_words(static_cast<const char*>(a.k_store) + st_off, (uint32_t)((int64_t)(hi_all - 1) * a.s_pos + D));
  const u32x4 vrw = rsrc_words(static_cast<const char*>(a.v_store) + st_off, (uint32_t)((int64_t)(hi_all - 1) * a.s_pos + D));
  const uint32_t sc_bytes = (uint32_t)(((int64_t)(hi_all - 1) * a.ss_pos + S::NG) * 2);
  const u32x4 ksrw = rsrc_words(a.k_scales + sc_off, sc_bytes);
  const u32x4 vsrw = rsrc_words(a.v_scales + sc_off, sc_bytes);

  // The NL loads of the tile at p0 into stage `stage`, spread over the
  // wavefronts (wavefront w issues loads w, w + NW, ..., a compile-time set):
  // K codes, V codes, K scale rows, V scale rows, in the decode kernel's stage
  // layout. Rows beyond the split read as zeros through an out-of-range lane
  // offset.
  auto issue_one = [&](int i, uint32_t base, uint32_t soff, uint32_t ssoff, int nvalid) {
    if (i < 2 * NI) {
      const int ci = i < NI ? i : i - NI;
      const int slot = ci * 64 + lane;
      const int r = slot / S::CH;
      const int c = (slot % S::CH) ^ ST::swz(r);
      const uint32_t voff = r < nvalid ? (uint32_t)r * row + 16 * c : kOOB;
      dma<16>(i < NI ? krw : vrw, base + (i < NI ? ST::K_OFF : ST::V_OFF) + 1024 * ci, voff, soff);
    } else {
      const uint32_t dst = base + (i == 2 * NI ? ST::KS_OFF : ST::VS_OFF);
      if constexpr (S::SB >= 4) {
        constexpr int PER = S::SB / 4;  // dwords per row
        const int r = lane / PER;
        dma<4>(i == 2 * NI ? ksrw : vsrw, dst, r < nvalid ? (uint32_t)r * srow + 4 * (lane % PER) : kOOB, ssoff);
      } else {  // lane l = row l, written at byte 4l; rows 32..63 read as zero
        dma<2>(i == 2 * NI ? ksrw : vsrw, dst, lane < nvalid ? (uint32_t)lane * srow : kOOB, ssoff);
      }
    }
  };
  // Role w: loads w, w + NW, ... With w a constant in each case below, the
  // unrolled indices are constants and every branch above folds away.
  auto issue_role = [&](const int w, uint32_t base, uint32_t soff, uint32_t ssoff, int nvalid) {
#pragma unroll
    for (int k = 0; k < (NL + NW - 1) / NW; ++k)
      if (w + NW * k < NL) issue_one(w + NW * k, base, soff, ssoff, nvalid);
  };
  auto issue_tile = [&](int stage, int p0) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int nvalid = min(kTile, end - p0);
    const uint32_t base = lds_addr_of(&lds_st[stage][0]);
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)p0 * row);
    const uint32_t ssoff = __builtin_amdgcn_readfirstlane((uint32_t)p0 * srow);
    switch (wv) {
      case 0: issue_role(0, base, soff, ssoff, nvalid); break;
      case 1: issue_role(1, base, soff, ssoff, nvalid); break;
      case 2: issue_role(2, base, soff, ssoff, nvalid); break;
      default: issue_role(3, base, soff, ssoff, nvalid); break;
    }
  };
  static_assert(NW == 4, "issue_tile assigns four wavefront roles");
  // Loads this wavefront issues per tile (NL spread round-robin over NW).
  auto wait_all_but_next = [&]() {
    if (wv < NL % NW) wait_vm<NL / NW + 1>();
    else wait_vm<NL / NW>();
  };

  RowAcc<D> acc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) acc[rb].o[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    acc[rb].l = (f32x4){0.f, 0.f, 0.f, 0.f};
    acc[rb].m_ref = -INFINITY;
  }
  const f16x8 ones = {(f16)1, (f16)1, (f16)1, (f16)1, (f16)1, (f16)1, (f16)1, (f16)1};

  const int n_tiles = (end - start + kTile - 1) / kTile;
  issue_tile(0, start);
  if (n_tiles > 1) issue_tile(1, start + kTile);
  for (int t = 0; t < n_tiles; ++t) {
    if (t + 1 < n_tiles) wait_all_but_next();  // own share of tile t landed; tile t+1 may still load
    else wait_vm<0>();
    // Every wavefront's share of tile t is in LDS, and every wavefront is done
    // with tile t-1 (its stage, which the tile t+2 loads reuse, and the value
    // tile, which is rewritten next).
    asm volatile("s_barrier" ::: "memory");
    if (t + 2 < n_tiles) issue_tile((t + 2) % kChunkStages, start + (t + 2) * kTile);
    const uint8_t* st = &lds_st[t % kChunkStages][0];
    const int p0 = start + t * kTile;
    convert_v<S, NW>(st, lds_vt, wv, lane);
    // Scores and softmax of the wavefront's rows while the value tile fills.
    KRegs<S> tk;
    stage_read_k<S>(tk, st, c16, q4);
    f16x8 pa[RB];
    const bool masked = !(p0 >= lo_all_w && p0 + kTile <= min(hi_all_w, end));
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float z[2][4];
      tile_scores_q<S>(tk, max(vlo[rb], p0) - p0, min(vhi[rb], end) - p0, z, qv[rb], corr[rb], a.c2, q4, masked);
      pa[rb] = row_softmax<D>(z, acc[rb]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // the value tile is complete
    // O^T (dims x rows) += V_hat^T (dims x 32 positions) . P^T; A operand: 8
    // positions of one dim, contiguous in the transposed tile.
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) {
      const f16x8 v = *reinterpret_cast<const f16x8*>(lds_vt + (16 * mt + c16) * kVtPitch + 16 * q4);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[rb].o[mt] = mfma16(v, pa[rb], acc[rb].o[mt]);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb].l = mfma16(ones, pa[rb], acc[rb].l);
  }

  // ---- partials of the wavefront's rows: lane (c16, q4) writes dims
  // 16*mt + 4*q4 + [0, 4) of its row c16, and lanes q4 = 0 its (max, sum) ------
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t id = row_id(rb);
    if (id >= 0) {
      float* o = a.ws_o + id * D + 4 * q4;
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) {
        const float4 v4 = make_float4(acc[rb].o[mt][0], acc[rb].o[mt][1], acc[rb].o[mt][2], acc[rb].o[mt][3]);
        if (a.ws_bytes)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v4), wsr,
                                                 (int)((id * D + 4 * q4 + 16 * mt) * 4), 0, 16);
        else
          *reinterpret_cast<float4*>(o + 16 * mt) = v4;
      }
      if (q4 == 0) put_ml(id, make_float2(acc[rb].m_ref, acc[rb].l[0]));
    }
  }
}

template <int D, int RB>
static void launch_chunk_rb(const kvq_layout& L, const ChunkArgs& a, dim3 grid, hipStream_t s) {
  if (L.scale_group == 64 && L.head_dim != 64)
    hipLaunchKernelGGL((kvq_chunk_kernel<D, true, RB>), grid, dim3(kChunkWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL((kvq_chunk_kernel<D, false, RB>), grid, dim3(kChunkWaves * 64), 0, s, a);
}

template <int D>
static void launch_chunk_d(const kvq_layout& L, const ChunkArgs& a, int rows_per_wg, dim3 grid, hipStream_t s) {
  if (rows_per_wg == 32 * kChunkWaves) launch_chunk_rb<D, 2>(L, a, grid, s);
  else launch_chunk_rb<D, 1>(L, a, grid, s);
}

int launch_chunk(const kvq_layout& L, const void* k_store, const void* v_store, const uint16_t* k_scales,
                 const uint16_t* v_scales, const uint16_t* q, int32_t batch, int32_t n_tok, int32_t n_q_heads,
                 const int32_t* d_start_pos, int32_t window, float sm_scale, const kvq_plan_t& plan, void* ws,
                 void* stream) {
  ChunkArgs a{};
  a.k_store = k_store;
  a.v_store = v_store;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.q = q;
  a.start_pos = d_start_pos;
  const int64_t rows = (int64_t)batch * n_tok * n_q_heads * plan.n_splits;
  a.ws_o = static_cast<float*>(ws);
  a.ws_ml = static_cast<float*>(ws) + rows * L.head_dim;
  if (rows * (L.head_dim + 2) * 4 <= 0x7fffffff) a.ws_bytes = (uint32_t)(rows * (L.head_dim + 2) * 4);
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
  const int rows_per_wg = chunk_rows_per_wg(n_tok, a.G, L.head_dim);
  a.row_blocks = chunk_row_blocks(n_tok, a.G, L.head_dim);
  a.n_splits = plan.n_splits;
  a.chunk = plan.chunk;
  a.window = window;
  a.c2 = sm_scale * 1.4426950408889634f;
  dim3 grid(plan.n_splits, L.n_kv_heads * a.row_blocks, batch);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (L.head_dim) {
    case 64: launch_chunk_d<64>(L, a, rows_per_wg, grid, s); break;
    case 128: launch_chunk_d<128>(L, a, rows_per_wg, grid, s); break;
    case 256: launch_chunk_d<256>(L, a, rows_per_wg, grid, s); break;
    default: return KVQ_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace kvq
