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
};

constexpr int kChunkStages = 3;

template <int D, bool G64>
__global__ __launch_bounds__(kChunkWaves * 64) void kvq_chunk_kernel(ChunkArgs a) {
  using S = Shape<D, true, true, G64>;
  using ST = Stage<S>;
  constexpr int NI = 32 * D / 1024;  // 1 KiB code loads per half tile
  constexpr int NL = 2 * NI + 2;     // direct-to-LDS loads per tile (codes + scale rows)
  constexpr int NW = kChunkWaves;
  __shared__ __attribute__((aligned(16))) uint8_t lds_st[kChunkStages][ST::BYTES];

  const int split = blockIdx.x;
  const int hk = blockIdx.y / a.row_blocks;
  const int rb = blockIdx.y % a.row_blocks;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;
  const int q4 = lane >> 4;
  const int G = a.G;

  // ---- rows of the workgroup and the keys they may see ------------------------
  const int fr0 = rb * kChunkRows;                     // first flat row (t * G + h)
  const int t_first = fr0 / G;
  const int t_last = min(a.T - 1, (fr0 + kChunkRows - 1) / G);
  int s0 = a.start_pos[b];
  s0 = s0 < 0 ? 0 : (s0 > a.max_ctx ? a.max_ctx : s0);
  // Keys [lo_all, hi_all): up to the last token's own position (tokens that
  // would sit at or beyond max_ctx see nothing).
  const int hi_all = min(s0 + t_last + 1, a.max_ctx);
  const int lo_all = a.window > 0 ? max(0, s0 + t_first + 1 - a.window) : 0;
  const int start = lo_all + split * a.chunk;
  const int end = (split == a.n_splits - 1) ? hi_all : min(hi_all, start + a.chunk);

  // This lane's row as the S^T column c16, and as O rows 4*q4 + i.
  const int my_fr = fr0 + wv * 16 + c16;
  const int my_t = my_fr / G;
  const bool my_valid = my_t < a.T;
  const int my_P = s0 + my_t;
  const int my_hi = (my_valid && my_P < a.max_ctx) ? my_P + 1 : 0;  // keys p < my_hi
  const int my_lo = a.window > 0 ? max(0, my_P + 1 - a.window) : 0;
  auto row_id = [&](int r) -> int64_t {  // partial row of wave row r, or -1
    const int fr = fr0 + wv * 16 + r;
    const int t = fr / G;
    if (t >= a.T) return -1;
    return (((int64_t)b * a.T + t) * a.n_q + hk * G + fr % G) * a.n_splits + split;
  };

  float2* const ml = reinterpret_cast<float2*>(a.ws_ml);
  if (start >= end) {  // nothing to attend in this split: empty partials
    if (lane < 16) {
      const int64_t id = row_id(lane);
      if (id >= 0) ml[id] = make_float2(-INFINITY, 0.0f);
    }
    return;
  }

  // ---- query operands of the lane's row, in registers (before any LDS load, so
  // the compiler's wait for them does not include the key tiles) ---------------
  f16x8 qv[S::NJ][2];
  {
    const uint16_t* qrow = a.q + (((int64_t)b * a.T + my_t) * a.n_q + hk * G + my_fr % G) * D;
#pragma unroll
    for (int j = 0; j < S::NJ; ++j)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (my_valid) v = *reinterpret_cast<const u32x4*>(qrow + 64 * j + 16 * q4 + 8 * u);
        qv[j][u] = __builtin_bit_cast(f16x8, v);
      }
  }
  float corr[S::NG];
  {
    float qsum[S::NJ];
#pragma unroll
    for (int j = 0; j < S::NJ; ++j) {
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += (float)qv[j][0][e] + (float)qv[j][1][e];
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      qsum[j] = s;
    }
#pragma unroll
    for (int g = 0; g < S::NG; ++g) {
      float t = 0.0f;
      if (G64) {
        t = qsum[g];
      } else {
#pragma unroll
        for (int j = 0; j < S::NJ; ++j) t += qsum[j];
      }
      corr[g] = -kCodeBias * t;
    }
  }

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

  // Load i of the NL loads of the tile at p0 into stage `st` (wavefront wv
  // issues loads wv, wv + NW, ...): K codes, V codes, K scale rows, V scale
  // rows, laid out as the decode kernel's stage. Rows beyond the split read as
  // zeros through an out-of-range lane offset.
  auto issue_tile = [&](int stage, int p0) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int nvalid = min(kTile, end - p0);
    const uint32_t base = lds_addr_of(&lds_st[stage][0]);
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)p0 * row);
    const uint32_t ssoff = __builtin_amdgcn_readfirstlane((uint32_t)p0 * srow);
    for (int i = wv; i < NL; i += NW) {
      if (i < 2 * NI) {
        const int ci = i < NI ? i : i - NI;
        const int slot = ci * 64 + lane;
        const int r = slot / S::CH;
        const int c = (slot % S::CH) ^ ST::swz(r);
        const uint32_t voff = r < nvalid ? (uint32_t)r * row + 16 * c : kOOB;
        dma<16>(i < NI ? krw : vrw, base + (i < NI ? ST::K_OFF : ST::V_OFF) + 1024 * ci, voff, soff);
      } else {
        const u32x4 srs = i == 2 * NI ? ksrw : vsrw;
        const uint32_t dst = base + (i == 2 * NI ? ST::KS_OFF : ST::VS_OFF);
        if constexpr (S::SB >= 4) {
          constexpr int PER = S::SB / 4;  // dwords per row
          const int r = lane / PER;
          dma<4>(srs, dst, r < nvalid ? (uint32_t)r * srow + 4 * (lane % PER) : kOOB, ssoff);
        } else {  // lane l = row l, written at byte 4l; rows 32..63 read as zero
          dma<2>(srs, dst, lane < nvalid ? (uint32_t)lane * srow : kOOB, ssoff);
        }
      }
    }
  };
  // Loads this wavefront issues per tile (NL spread round-robin over NW).
  auto wait_all_but_next = [&]() {
    if (wv < NL % NW) wait_vm<NL / NW + 1>();
    else wait_vm<NL / NW>();
  };

  WaveAcc<S> acc;
#pragma unroll
  for (int n = 0; n < S::VB; ++n) acc.o[n] = (f32x4){0.f, 0.f, 0.f, 0.f};
  acc.l = (f32x4){0.f, 0.f, 0.f, 0.f};
  acc.m_ref = -INFINITY;

  const int n_tiles = (end - start + kTile - 1) / kTile;
  issue_tile(0, start);
  if (n_tiles > 1) issue_tile(1, start + kTile);
  for (int t = 0; t < n_tiles; ++t) {
    if (t + 1 < n_tiles) wait_all_but_next();  // own share of tile t landed; tile t+1 may still load
    else wait_vm<0>();
    // Every wavefront's share of tile t is in LDS, and every wavefront is done
    // with tile t-1, whose stage the tile t+2 loads now reuse.
    asm volatile("s_barrier" ::: "memory");
    if (t + 2 < n_tiles) issue_tile((t + 2) % kChunkStages, start + (t + 2) * kTile);
    const uint8_t* st = &lds_st[t % kChunkStages][0];
    const int p0 = start + t * kTile;
    KRegs<S> tk;
    stage_read_k<S>(tk, st, c16, q4);
    float z[2][4];
    tile_scores_q<S>(tk, max(my_lo, p0) - p0, min(my_hi, end) - p0, z, qv, corr, a.c2, q4);
    VRegs<S> tv;
    stage_read_v<S>(tv, st, c16, q4);
    const f16x8 pa = tile_softmax<S>(z, acc, q4);
    tile_pv<S>(tv, pa, acc);
  }

  // ---- partials of this wavefront's 16 rows --------------------------------------
  // O rows 4*q4 + i, dims VB*c16 + [0, VB); the max of row r is held by the lanes
  // with c16 = r, its sum by the lanes with q4 = r / 4 (element r % 4).
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t id = row_id(4 * q4 + i);
    if (id >= 0) {
      float* o = a.ws_o + id * D + S::VB * c16;
#pragma unroll
      for (int n4 = 0; n4 < S::VB / 4; ++n4)
        *reinterpret_cast<float4*>(o + 4 * n4) =
            make_float4(acc.o[4 * n4 + 0][i], acc.o[4 * n4 + 1][i], acc.o[4 * n4 + 2][i], acc.o[4 * n4 + 3][i]);
    }
  }
  {
    const int r = c16;
    const int src = 16 * (r >> 2);
    const float l0 = __shfl(acc.l[0], src), l1 = __shfl(acc.l[1], src);
    const float l2 = __shfl(acc.l[2], src), l3 = __shfl(acc.l[3], src);
    const float l = (r & 3) == 0 ? l0 : (r & 3) == 1 ? l1 : (r & 3) == 2 ? l2 : l3;
    if (q4 == 0) {
      const int64_t id = row_id(r);
      if (id >= 0) ml[id] = make_float2(acc.m_ref, l);
    }
  }
}

template <int D>
static void launch_chunk_d(const kvq_layout& L, const ChunkArgs& a, dim3 grid, hipStream_t s) {
  if (L.scale_group == 64 && L.head_dim != 64)
    hipLaunchKernelGGL((kvq_chunk_kernel<D, true>), grid, dim3(kChunkWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL((kvq_chunk_kernel<D, false>), grid, dim3(kChunkWaves * 64), 0, s, a);
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
  a.row_blocks = chunk_row_blocks(n_tok, a.G);
  a.n_splits = plan.n_splits;
  a.chunk = plan.chunk;
  a.window = window;
  a.c2 = sm_scale * 1.4426950408889634f;
  dim3 grid(plan.n_splits, L.n_kv_heads * a.row_blocks, batch);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (L.head_dim) {
    case 64: launch_chunk_d<64>(L, a, grid, s); break;
    case 128: launch_chunk_d<128>(L, a, grid, s); break;
    case 256: launch_chunk_d<256>(L, a, grid, s); break;
    default: return KVQ_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace kvq
