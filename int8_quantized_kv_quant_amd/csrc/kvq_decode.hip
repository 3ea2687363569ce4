// kv_decode_attn_splitk: split-K partials of single-token decode attention over
// an int8 (or fp32) KV cache, on the gfx950 matrix cores.
//
// genie-ai-runtime releases, v1.3.0 "split-K decode attention": the KV range of
// a head is split over blocks that each form an online-softmax partial, later
// combined by a reduce kernel. v0.1.0-alpha.12 "Path I series" #65: each key and
// value is dequantized as code * scale of its (position, kv head). Strata
// PR 2698 "What it does": an FP16 scale for each 64-value group; k8v32 / k32v8.
//
// Mapping. One workgroup = (sequence b, kv head, block of up to 16 query heads
// sharing it, split s). Split s owns the 128-position blocks s, s + S,
// s + 2 S, ... of the attended range, S = min(n_splits, ceil((L - lo) /
// chunk)) (block-cyclic: as many splits as contiguous ranges would use, but
// with one workgroup per compute unit this spreads each XCD's reads over the
// whole context, which shortened the 128K step by ~1.5 us against contiguous
// ranges); wavefront w takes tile w of each block. Per tile a wavefront computes, with
// v_mfma_f32_16x16x32_f16:
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
// Data movement. For int8 K and V the tiles are staged in LDS: each wavefront
// owns one stage with a K half and a V half, each refilled by direct-to-LDS
// buffer loads (no registers held while in flight) as soon as the wavefront has
// copied the half's current tile into registers, so every half is loading the
// next tile for about one tile of compute. Rows land as 16-byte chunks
// XOR-swizzled by row, so the MFMA-layout reads are free of bank conflicts. A
// store with fp32 rows is four times wider per position, so with one int8 and
// one fp32 store (k8v32, k32v8) only the fp32 tile is staged (32 * 4D bytes per
// wavefront) and the int8 operands load straight into a second register set;
// all of tile t + 1's loads are in flight while tile t is computed (measured
// 1.6 us shorter at context 32048 than loading each tile just before its
// use). k32v32 reads both operands straight into registers.
//
// Bounds. Every K/V/scale load goes through a buffer resource whose size ends
// at the last row of the context, and positions outside the split get an
// out-of-range offset, so they read as zero and are masked out of the softmax.
//
// Chunk rows (int8 K and V, the CHUNK instances; Strata PR 2698 "What it
// does": verify windows read the same cache as decode). The rows of a
// workgroup are (token, head) pairs t * G + h of a chunk of T tokens at
// positions start + t, in RB blocks of 16 that share every key and value
// operand (each block its own MFMAs, softmax state and accumulators), each
// row masking keys outside its own causal (and window) range; the partials go
// to rows (b, t, hq) for the same reduce. A verify window of up to 32 rows
// per kv head then reads every key once, with the decode kernel's split over
// the whole chip, where the chunk kernel (64 rows per workgroup sharing each
// tile) would leave most of its wavefronts without rows.
#include <math.h>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_tile.h"

namespace kvq {

struct PartialArgs {
  const void* k_store;
  const void* v_store;
  const uint16_t* k_scales;
  const uint16_t* v_scales;
  // Fused append: the new token's K and V rows, fp16 [B][n_kv][D] (null: none).
  // Row L - 1 of the stores and scales is then written (through the pointers
  // above, which the fused entry point receives writable).
  const uint16_t* k_new;
  const uint16_t* v_new;
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
  // Chunk attention through this kernel (the CHUNK instances): T tokens per
  // sequence at positions start_pos[b] + t; the query rows of a kv head are
  // its (token, head) pairs t * G + h, in blocks of 16 (head_blocks of them),
  // q is fp16 [B][T][n_q][D], and the partial rows are (b, t, hq).
  const int32_t* start_pos;
  int32_t T;
  // One-launch step (the ONE instances): the fp16 output [B][n_q][D] and one
  // arrival counter per (sequence, kv head, head block). ws_bytes: the byte size
  // of the partial region (ws_o then ws_ml) for write-through accesses, or 0
  // when one buffer resource cannot cover it.
  uint16_t* out;
  uint32_t* arrive;
  uint32_t ws_bytes;
  int32_t rows_per_block;  // query heads per head block (<= 16)
};

// Cache policy of the one-launch step's partial stores and loads: device scope
// (sc1), i.e. stores written through the XCD's L2 to memory and loads that miss
// in it. A workgroup on one XCD can then read what a workgroup on another XCD
// wrote once that write has completed, without the write-back and
// invalidation of whole L2 caches that a release/acquire fence pair costs.
constexpr int kWriteThrough = 16;
__device__ __forceinline__ void st128_wt(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, kWriteThrough);
}
__device__ __forceinline__ void st64_wt(__amdgpu_buffer_rsrc_t r, uint32_t off, float2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, (int)off, 0, kWriteThrough);
}
__device__ __forceinline__ float4 ld128_wt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kWriteThrough));
}
__device__ __forceinline__ float2 ld64_wt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kWriteThrough));
}

// ---- operand loads straight from HBM into registers (any store dtype) ----------
// K operands (codes or fp32 rows, and an int8 store's scale rows) of the tile
// at p0; positions at or beyond `end` read as zeros.
template <class S>
__device__ __forceinline__ void load_k_global(KRegs<S>& t, __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t ksrs,
                                              int p0, int end, uint32_t krow, uint32_t srow, int c16, int q4) {
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int pk = p0 + 16 * ct + c16;
    const uint32_t off = pk < end ? (uint32_t)pk * krow : kOOB;
#pragma unroll
    for (int j = 0; j < S::NJ; ++j)
#pragma unroll
      for (int m = 0; m < S::KW; ++m) t.k[ct][j][m] = ld128(krs, off + S::KE * (64 * j + 16 * q4) + 16 * m);
  }
  if constexpr (S::KI8) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ps = p0 + 16 * ct + 4 * q4 + i;
        const uint32_t off = ps < end ? (uint32_t)ps * srow : kOOB;
        if constexpr (S::SB == 8) {
          const u32x2 v = ld64(ksrs, off);
          t.ks[ct][i][0] = v.x;
          t.ks[ct][i][S::NKS - 1] = v.y;
        } else if constexpr (S::SB == 4) {
          t.ks[ct][i][0] = ld32(ksrs, off);
        } else {
          t.ks[ct][i][0] = ld16(ksrs, off);
        }
      }
  }
}

// V operands (codes or fp32 rows, and an int8 store's scales) of the tile at p0.
template <class S>
__device__ __forceinline__ void load_v_global(VRegs<S>& tv, __amdgpu_buffer_rsrc_t vrs, __amdgpu_buffer_rsrc_t vsrs,
                                              int p0, int end, uint32_t vrow, uint32_t srow, int c16, int q4) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int pv = p0 + kpos(e, q4);
    const uint32_t off = pv < end ? (uint32_t)pv * vrow : kOOB;
    const uint32_t base = off + S::VB * S::VE * c16;
    if constexpr (S::VW == 1) {
      tv.v[e][0] = ld32(vrs, base);
    } else if constexpr (S::VW == 2) {
      const u32x2 v = ld64(vrs, base);
      tv.v[e][0] = v.x;
      tv.v[e][S::VW - 1] = v.y;
    } else {
#pragma unroll
      for (int m = 0; m < S::VW / 4; ++m) {
        const u32x4 v = ld128(vrs, base + 16 * m);
        tv.v[e][4 * m + 0] = v.x;
        tv.v[e][4 * m + 1] = v.y;
        tv.v[e][4 * m + 2] = v.z;
        tv.v[e][4 * m + 3] = v.w;
      }
    }
    if constexpr (S::VI8) {
      const int grp = S::G64 ? (S::VB * c16) / 64 : 0;
      tv.vs[e] = ld16(vsrs, pv < end ? (uint32_t)pv * srow + 2 * grp : kOOB);
    }
  }
}

// s_waitcnt vmcnt(0) as the compiler's own wait instruction (expcnt and
// lgkmcnt fields at their maxima): unlike a wait in inline asm, the compiler
// sees it, so it knows every register load issued before it has landed and adds
// no waits of its own for them.
__device__ __forceinline__ void wait_vm0_visible() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Float4 position of float4 f of a merge-slot row. The 16 lanes that write one
// row at a time hold f = 4c + n for c = 0..15: XOR-ing bits 0-1 with bits 4-5
// spreads them over the 16 distinct 16-byte bank groups.
__device__ __forceinline__ int merge_swz(int f) { return f ^ ((f >> 4) & 3); }

// ---- kernel ----------------------------------------------------------------------
template <int D, bool KI8, bool VI8, bool G64, int NW, bool CHUNK = false, int RB = 1, bool ONE = false>
__global__ __launch_bounds__(NW * 64) void kvq_partial_kernel(PartialArgs a) {
  using S = Shape<D, KI8, VI8, G64>;
  constexpr bool kStaged = KI8 && VI8;
  // ONE: the one-launch decode step (kv_decode_attn) over int8 K and V.
  static_assert(!ONE || (kStaged && !CHUNK && RB == 1), "one-launch step: int8 decode only");
  // RB blocks of 16 query rows per workgroup, sharing every key and value
  // operand (chunk rows over int8 K and V only).
  static_assert(RB == 1 || (CHUNK && kStaged && RB == 2), "two row blocks for int8 chunk rows only");
  // One store int8, the other fp32: the fp32 tile is staged in LDS, the int8
  // operands go straight to registers.
  constexpr bool kMix = KI8 != VI8;
  // Lanes of one scale group in the fused append's quantizer (4 values each):
  // 64 values, or the whole row.
  constexpr int kQGL = G64 ? 16 : D / 4;
  static_assert(D % (16 * NW) == 0, "the new position's score: 4-dim steps per lane");
  using FS = F32Stage<S, !KI8>;
  constexpr int STAGE_BYTES = kStaged ? Stage<S>::BYTES : (kMix ? FS::BYTES : 16);
  // One stage per wavefront. After its last tile a wavefront reuses its own
  // stage as its slot of the output merge (16 head rows of D floats, which fit
  // in a stage), so no wavefront waits for another before writing its slot.
  constexpr int SLOT_BYTES = 16 * D * 4;
  constexpr int SLOT_PITCH = (kStaged || kMix) ? STAGE_BYTES : SLOT_BYTES;
  static_assert(!(kStaged || kMix) || SLOT_BYTES <= STAGE_BYTES, "merge slot must fit in a stage");
  constexpr int ST_BYTES = NW * SLOT_PITCH;
  __shared__ __attribute__((aligned(16))) uint8_t lds_st[ST_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_q[16 * RB * QOperand<S>::ROW];
  __shared__ float sm_m[NW][16];
  __shared__ float sm_l[NW][16];
  // The new token's rows when the append is fused ([0] = K, [1] = V): the fp16
  // input (landing place of its direct-to-LDS load), the dequantized values,
  // the codes and scales (for the cache), and the new position's scores.
  __shared__ __attribute__((aligned(16))) uint16_t nw_in[2][D];
  __shared__ __attribute__((aligned(16))) float nw_val[2][D];
  __shared__ __attribute__((aligned(16))) uint32_t nw_code[2][D / 4];
  __shared__ uint16_t nw_scale[2][S::NG];
  __shared__ float nw_z[NW][16];
  __shared__ int sm_last;  // ONE: this workgroup arrived last in its unit

  const int split = blockIdx.x;
  const int hk = blockIdx.y / a.head_blocks;
  const int hblk = blockIdx.y % a.head_blocks;
  const int b = blockIdx.z;

  // Query rows of the workgroup (up to 16 * RB) and the keys [lo, L) they attend.
  // Decode: heads hblk * 16 .. of kv head hk, at context seq_lens[b]. Chunk:
  // flat rows fr0 + r = t * G + h of kv head hk; token t sits at s0 + t and
  // attends [max(0, s0 + t + 1 - window) (window > 0), s0 + t + 1).
  // Query rows per head block: 16, or fewer in the one-launch step
  // (a.rows_per_block), so that a unit's partial stays small.
  const int RPB = ONE ? a.rows_per_block : 16;
  const int fr0 = hblk * RPB * RB;
  const int nh = CHUNK ? min(16 * RB, a.T * a.G - fr0) : min(RPB, a.G - fr0);
  const int hq0 = hk * a.G + fr0;
  const int64_t row0 = ((int64_t)b * a.n_q + hq0) * a.n_splits + split;
  float2* const ml = reinterpret_cast<float2*>(a.ws_ml);
  // Partial row (within ws) of the workgroup's row r < nh.
  auto rowid = [&](int r) -> int64_t {
    if constexpr (CHUNK) {
      const int fr = fr0 + r;
      return (((int64_t)b * a.T + fr / a.G) * a.n_q + hk * a.G + fr % a.G) * a.n_splits + split;
    } else {
      return row0 + (int64_t)r * a.n_splits;
    }
  };
  int L_in, L, lo, s0 = 0;
  if constexpr (CHUNK) {
    s0 = a.start_pos[b];
    s0 = s0 < 0 ? 0 : (s0 > a.max_ctx ? a.max_ctx : s0);
    const int t_first = fr0 / a.G, t_last = min(a.T - 1, (fr0 + nh - 1) / a.G);
    L = (int)min((int64_t)s0 + t_last + 1, (int64_t)a.max_ctx);
    lo = a.window > 0 ? max(0, s0 + t_first + 1 - a.window) : 0;
    L_in = -1;  // no fused append
  } else {
    L_in = a.seq_lens[b];
    L = L_in < 0 ? 0 : (L_in > a.max_ctx ? a.max_ctx : L_in);
    lo = a.window > 0 ? max(0, L - a.window) : 0;
  }
  // Partial stores, written through the L2 to memory whenever one buffer
  // resource covers the workspace (a.ws_bytes != 0). ONE: the last workgroup
  // of the unit, possibly on another XCD, reads them below. Decode: the reduce
  // kernel reads them after this launch, whose end then has fewer dirty L2
  // lines to write back (measured: 64K step 19.4-20.2 -> 18.7-19.0 us, 32K
  // 14.1 -> 13.6-13.9 us, 128K 0.1-0.2 us shorter, the batched and mixed steps
  // unchanged). Chunk rows keep ordinary stores (their verify windows measured
  // no gain).
  const auto wsr = make_rsrc(a.ws_o, a.ws_bytes);
  const uint32_t ml_base = (uint32_t)((a.ws_ml - a.ws_o) * 4);
  const bool wt = ONE || (!CHUNK && a.ws_bytes != 0u);
  auto put_o = [&](int64_t row, int d, float4 v) {
    if (wt) st128_wt(wsr, (uint32_t)((row * D + d) * 4), v);
    else reinterpret_cast<float4*>(a.ws_o + row * D)[d / 4] = v;
  };
  auto put_ml = [&](int64_t row, float2 v) {
    if (wt) st64_wt(wsr, ml_base + (uint32_t)(row * 8), v);
    else ml[row] = v;
  };
  // ONE: after the workgroup's partial stores. Arrival is counted per unit
  // (sequence, kv head, head block) with a device-scope atomic once every lane's
  // write-through stores have completed; the workgroup that brings the count
  // to n_splits resets it to zero for the next call and combines the unit's
  // splits -- as the reduce kernel does: M = max m_s, out = sum 2^(m_s - M) O_s /
  // sum 2^(m_s - M) l_s, fp16 (RNE) -- from loads that miss every cache.
  // No workgroup waits for another, so the launch always drains.
  auto arrive_and_combine = [&]() {
    if constexpr (ONE) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (threadIdx.x == 0) {
        uint32_t* cnt = a.arrive + ((int64_t)b * a.n_kv + hk) * a.head_blocks + hblk;  // < batch * n_q
        const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = old + 1u == (uint32_t)a.n_splits;
        if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm_last = last ? 1 : 0;
      }
      __syncthreads();
      if (!sm_last) return;
      // Every lane takes up to kPairs (head, 4-dim) columns per round and
      // issues all their loads before using any (one memory round trip per
      // round; a unit of up to 8 heads at D = 256 is one round).
      constexpr int kPairs = 2;
      constexpr int K = kOneLaunchMaxSplits;
      for (int base = threadIdx.x; base < nh * (D / 4); base += kPairs * NW * 64) {
        float2 mls[kPairs][K];
        float4 os[kPairs][K];
#pragma unroll
        for (int u = 0; u < kPairs; ++u) {
          const int idx = base + u * NW * 64;
          const int h = idx / (D / 4);
          const int d = 4 * (idx % (D / 4));
          const int64_t hrow = ((int64_t)b * a.n_q + hq0 + h) * a.n_splits;  // split 0 of head h
#pragma unroll
          for (int s = 0; s < K; ++s) {
            // an empty split's O row is unwritten: loaded, but never used
            mls[u][s] = make_float2(-INFINITY, 0.0f);
            os[u][s] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (idx < nh * (D / 4) && s < a.n_splits) {
              mls[u][s] = ld64_wt(wsr, ml_base + (uint32_t)((hrow + s) * 8));
              os[u][s] = ld128_wt(wsr, (uint32_t)(((hrow + s) * D + d) * 4));
            }
          }
        }
#pragma unroll
        for (int u = 0; u < kPairs; ++u) {
          const int idx = base + u * NW * 64;
          if (idx >= nh * (D / 4)) continue;
          const int h = idx / (D / 4);
          const int d = 4 * (idx % (D / 4));
          float M = -INFINITY;
#pragma unroll
          for (int s = 0; s < K; ++s) M = fmaxf(M, mls[u][s].x);
          float l = 0.0f;
          float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
          for (int s = 0; s < K; ++s) {
            if (mls[u][s].x != -INFINITY) {
              const float w = __builtin_amdgcn_exp2f(mls[u][s].x - M);
              l = fmaf(w, mls[u][s].y, l);
              o.x = fmaf(w, os[u][s].x, o.x);
              o.y = fmaf(w, os[u][s].y, o.y);
              o.z = fmaf(w, os[u][s].z, o.z);
              o.w = fmaf(w, os[u][s].w, o.w);
            }
          }
          const float inv = l > 0.0f ? 1.0f / l : 0.0f;
          const f16 r0 = (f16)(o.x * inv), r1 = (f16)(o.y * inv), r2 = (f16)(o.z * inv), r3 = (f16)(o.w * inv);
          const u32x2 pk = {
              (uint32_t)__builtin_bit_cast(uint16_t, r0) | ((uint32_t)__builtin_bit_cast(uint16_t, r1) << 16),
              (uint32_t)__builtin_bit_cast(uint16_t, r2) | ((uint32_t)__builtin_bit_cast(uint16_t, r3) << 16)};
          *reinterpret_cast<u32x2*>(a.out + ((int64_t)b * a.n_q + hq0 + h) * D + d) = pk;
        }
      }
    }
  };

  // Split s takes the blocks s, s + S, s + 2 S, ... of BLK positions of
  // [lo, L) (block-cyclic), S = min(n_splits, ceil((L - lo) / chunk)): as many
  // splits as contiguous ranges of `chunk` positions would use, each reading
  // across the whole context; wavefront w takes tile w of each of its blocks.
  constexpr int BLK = NW * kTile;
  const int n_used = (int)min((int64_t)a.n_splits, ((int64_t)L - lo + a.chunk - 1) / a.chunk);
  const int64_t start64 = (int64_t)lo + (int64_t)split * BLK;
  if (split >= n_used || start64 >= L) {  // empty split: recorded as (m, l) = (-inf, 0), O not written
    if ((int)threadIdx.x < nh) put_ml(rowid(threadIdx.x), make_float2(-INFINITY, 0.0f));
    arrive_and_combine();
    return;
  }
  const int start = (int)start64;
  int end = L;
  // Fused append: the workgroup whose blocks hold position L - 1 takes the new
  // row from the quantizer instead of the cache, and its tiles stop before it.
  const bool own_new = !CHUNK && a.k_new != nullptr && L_in == L && ((L - 1 - lo) / BLK) % n_used == split;
  if (own_new) end = L - 1;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;
  const int q4 = lane >> 4;

  // ---- buffer resources of this (sequence, kv head) slice -------------------
  const uint32_t krow = (uint32_t)(a.s_pos * S::KE);
  const uint32_t vrow = (uint32_t)(a.s_pos * S::VE);
  const uint32_t srow = (uint32_t)(a.ss_pos * 2);
  const int64_t st_off = (int64_t)b * a.s_seq + (int64_t)hk * a.s_head;
  const int64_t sc_off = (int64_t)b * a.ss_seq + (int64_t)hk * a.ss_head;
  const auto krs = make_rsrc(static_cast<const char*>(a.k_store) + st_off * S::KE,
                             (uint32_t)(((int64_t)(L - 1) * a.s_pos + D) * S::KE));
  const auto vrs = make_rsrc(static_cast<const char*>(a.v_store) + st_off * S::VE,
                             (uint32_t)(((int64_t)(L - 1) * a.s_pos + D) * S::VE));
  const uint32_t sc_bytes = (uint32_t)(((int64_t)(L - 1) * a.ss_pos + S::NG) * 2);
  const auto ksrs = make_rsrc(KI8 ? static_cast<const void*>(a.k_scales + sc_off) : nullptr, KI8 ? sc_bytes : 0u);
  const auto vsrs = make_rsrc(VI8 ? static_cast<const void*>(a.v_scales + sc_off) : nullptr, VI8 ? sc_bytes : 0u);

  const int STEP = BLK * n_used;  // from a tile to the same tile of the split's next block
  int p0 = start + wv * kTile;
  // Loads into LDS before the first tile's, counted like them (compiler-visible
  // loads here would make the compiler wait for every load in flight before
  // their first use): the new K (wavefront 0) or V (wavefront 1) row when the
  // append is fused, then 16 / NW query rows per wavefront (rows past nh read
  // as zeros). A query row lands as D consecutive fp16 values at the start of
  // its padded LDS row.
  constexpr int QROWS = 16 * RB / NW;
  KRegs<S> tk;  // int8 operands of the mixed stores' first tile, loaded first
  VRegs<S> tv;
  if constexpr (kMix) {
    if (p0 < end) {
      if constexpr (KI8) load_k_global<S>(tk, krs, ksrs, p0, end, krow, srow, c16, q4);
      else load_v_global<S>(tv, vrs, vsrs, p0, end, vrow, srow, c16, q4);
    }
  }
  if (own_new && wv < 2) {
    const uint16_t* src = (wv == 0 ? a.k_new : a.v_new) + ((int64_t)b * a.n_kv + hk) * D;
    if (lane < D / 8) dma<16>(rsrc_words(src, 2 * D), lds_addr_of(reinterpret_cast<const uint8_t*>(nw_in[wv])),
                              16u * lane, 0u);
  }
  if constexpr (CHUNK) {  // the rows of this block: q [b][t][hk * G + h]
    const u32x4 qrs = rsrc_words(a.q + (int64_t)b * a.T * a.n_q * D, (uint32_t)((int64_t)a.T * a.n_q * D * 2));
#pragma unroll
    for (int i = 0; i < QROWS; ++i) {
      const int r = wv * QROWS + i;
      const int fr = fr0 + r;
      const uint32_t off = (uint32_t)((((int64_t)(fr / a.G) * a.n_q + hk * a.G + fr % a.G) * D) * 2);
      if (lane < D / 8)
        dma<16>(qrs, lds_addr_of(lds_q + r * QOperand<S>::ROW), r < nh ? off + 16 * lane : kOOB, 0u);
    }
  } else {
    const u32x4 qrs = rsrc_words(a.q + ((int64_t)b * a.n_q + hq0) * D, (uint32_t)(nh * D * 2));
#pragma unroll
    for (int i = 0; i < QROWS; ++i) {
      const int r = wv * QROWS + i;
      if (lane < D / 8)
        dma<16>(qrs, lds_addr_of(lds_q + r * QOperand<S>::ROW), r < nh ? (uint32_t)(r * 2 * D + 16 * lane) : kOOB, 0u);
    }
  }
  u32x4 krw = {0, 0, 0, 0}, vrw = krw, ksrw = krw, vsrw = krw;
  if constexpr (kStaged) {  // first tile in flight while the query is prepared
    krw = rsrc_words(static_cast<const char*>(a.k_store) + st_off, (uint32_t)((int64_t)(L - 1) * a.s_pos + D));
    vrw = rsrc_words(static_cast<const char*>(a.v_store) + st_off, (uint32_t)((int64_t)(L - 1) * a.s_pos + D));
    ksrw = rsrc_words(a.k_scales + sc_off, sc_bytes);
    vsrw = rsrc_words(a.v_scales + sc_off, sc_bytes);
    if (p0 < end) {
      stage_issue<S, 0>(lds_st + wv * STAGE_BYTES, krw, ksrw, p0, end - p0, krow, srow, lane);
      stage_issue<S, 1>(lds_st + wv * STAGE_BYTES, vrw, vsrw, p0, end - p0, krow, srow, lane);
    }
  }
  u32x4 frw = {0, 0, 0, 0};  // the fp32 store of the mixed stores
  if constexpr (kMix) {
    frw = KI8 ? rsrc_words(static_cast<const char*>(a.v_store) + st_off * 4, (uint32_t)(((int64_t)(L - 1) * a.s_pos + D) * 4))
              : rsrc_words(static_cast<const char*>(a.k_store) + st_off * 4, (uint32_t)(((int64_t)(L - 1) * a.s_pos + D) * 4));
    if (p0 < end) f32stage_issue<S, !KI8>(lds_st + wv * STAGE_BYTES, frw, p0, end - p0, KI8 ? vrow : krow, lane);
  }

  // ---- this wavefront's LDS loads have landed (the first tile's two halves may
  // still be loading); after the barrier every query row is in LDS.
  if (kStaged && p0 < end) wait_vm<2 * kHalfLoads<S>>();
  else if (kMix && p0 < end) wait_vm<FS::LOADS>();
  else wait_vm<0>();
  if (own_new && wv < 2) {
    const bool i8 = wv == 0 ? KI8 : VI8;
    uint32_t hb[4] = {0, 0, 0, 0};
    if (lane < D / 4) {
      const u32x2 raw = *reinterpret_cast<const u32x2*>(&nw_in[wv][4 * lane]);
      hb[0] = raw.x & 0xffffu; hb[1] = raw.x >> 16; hb[2] = raw.y & 0xffffu; hb[3] = raw.y >> 16;
    }
    float4 val;
    if (i8) {
      uint16_t sb;
      const uint32_t code = quantize4<kQGL>(hb, &sb);  // as kv_quant_append
      const float sc = h_bits_to_f32(sb);
      val = make_float4((float)(int8_t)(code & 0xff) * sc, (float)(int8_t)((code >> 8) & 0xff) * sc,
                        (float)(int8_t)((code >> 16) & 0xff) * sc, (float)(int8_t)(code >> 24) * sc);
      if (lane < D / 4) {
        nw_code[wv][lane] = code;
        if (lane % kQGL == 0) nw_scale[wv][lane / kQGL] = sb;
      }
    } else {  // an fp32 store holds the fp16 value widened
      val = make_float4(h_bits_to_f32(hb[0]), h_bits_to_f32(hb[1]), h_bits_to_f32(hb[2]), h_bits_to_f32(hb[3]));
    }
    if (lane < D / 4) *reinterpret_cast<float4*>(&nw_val[wv][4 * lane]) = val;
  }
  __syncthreads();  // query rows (and the new rows) in LDS
  // ---- fused append: the new row into the cache (one head block writes it).
  // Issued right after the quantization, so that its store latency overlaps
  // the tiles (no workgroup of this launch reads position L - 1 from the
  // cache: its owner takes it from LDS, and the other splits' blocks end
  // before it). The explicit load counts below then over-count by these
  // stores at most, which only makes a wait stricter.
  if (own_new && hblk == 0 && wv < 2 && lane < D / 4) {
    const int64_t r = (int64_t)b * a.s_seq + (int64_t)(L - 1) * a.s_pos + (int64_t)hk * a.s_head;
    const bool i8 = wv == 0 ? KI8 : VI8;
    void* store = const_cast<void*>(wv == 0 ? a.k_store : a.v_store);
    if (i8) {
      reinterpret_cast<uint32_t*>(static_cast<int8_t*>(store) + r)[lane] = nw_code[wv][lane];
      if (lane % kQGL == 0) {
        uint16_t* sc = const_cast<uint16_t*>(wv == 0 ? a.k_scales : a.v_scales);
        sc[(int64_t)b * a.ss_seq + (int64_t)(L - 1) * a.ss_pos + (int64_t)hk * a.ss_head + lane / kQGL] =
            nw_scale[wv][lane / kQGL];
      }
    } else {
      reinterpret_cast<float4*>(static_cast<float*>(store) + r)[lane] =
          *reinterpret_cast<const float4*>(&nw_val[wv][4 * lane]);
    }
  }
  // The lane's query row c16 of row block rb: qb + rb * QB.
  const uint8_t* const qb = lds_q + c16 * QOperand<S>::ROW + 32 * q4;
  constexpr int QB = 16 * QOperand<S>::ROW;

  // ---- per-group sums of q: the accumulator start values -1152 * sum(q) that
  // cancel the +1152 code bias (rows beyond nh are zero).
  float corr[RB][S::NG];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float qsum[S::NJ];
#pragma unroll
    for (int j = 0; j < S::NJ; ++j) {
      const f16x8 h0 = q_get(qb + rb * QB, j, 0), h1 = q_get(qb + rb * QB, j, 1);
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += (float)h0[e] + (float)h1[e];
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      qsum[j] = s;  // sum of q over the 64 dims of block j, for head c16
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
      corr[rb][g] = KI8 ? -kCodeBias * t : 0.0f;
    }
  }
  if (own_new) {
    // Partial scores of the new position for the 16 heads (rows beyond nh are
    // zero), a 1/NW share of the dims per wavefront: lane 4h + r sums dims
    // d0 .. d0 + D / (4 NW) of head h; lds_q row h holds q[h][0..D) as
    // consecutive fp16 values. The merge adds the wavefronts' sums.
    constexpr int DL = D / (4 * NW);
    const int h = lane >> 2, r = lane & 3;
    const int d0 = wv * (D / NW) + r * DL;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(lds_q + h * QOperand<S>::ROW);
    float zs = 0.0f;
#pragma unroll
    for (int d = d0; d < d0 + DL; d += 4) {
      const u32x2 qv = *reinterpret_cast<const u32x2*>(qrow + d);
      const float4 k = *reinterpret_cast<const float4*>(&nw_val[0][d]);
      zs = fmaf(h_bits_to_f32(qv.x & 0xffffu), k.x, zs);
      zs = fmaf(h_bits_to_f32(qv.x >> 16), k.y, zs);
      zs = fmaf(h_bits_to_f32(qv.y & 0xffffu), k.z, zs);
      zs = fmaf(h_bits_to_f32(qv.y >> 16), k.w, zs);
    }
    zs += lane_xor<1>(zs);
    zs += lane_xor<2>(zs);
    if (r == 0) nw_z[wv][h] = zs;  // read in the merge, after its barrier
  }
  // The new position's score for head h (log2 units).
  auto z_new = [&](int h) {
    float z = 0.0f;
#pragma unroll
    for (int k = 0; k < NW; ++k) z += nw_z[k][h];
    return z * a.c2;
  };

  WaveAcc<S> acc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int n = 0; n < S::VB; ++n) acc[rb].o[n] = (f32x4){0.f, 0.f, 0.f, 0.f};
    acc[rb].l = (f32x4){0.f, 0.f, 0.f, 0.f};
    acc[rb].m_ref = -INFINITY;
  }

  // Chunk: keys [rlo, rhi) of the lane's query row c16 of block rb (none for
  // rows past nh).
  int rlo[RB], rhi[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    rlo[rb] = 0;
    rhi[rb] = 0;
    if constexpr (CHUNK) {
      const int r = 16 * rb + c16;
      const int P = s0 + (fr0 + r) / a.G;
      rhi[rb] = (r < nh && P < a.max_ctx) ? P + 1 : 0;
      rlo[rb] = a.window > 0 ? max(0, P + 1 - a.window) : 0;
    }
  }

  if constexpr (kStaged) {
    // Pipeline over this wavefront's tiles p0, p0 + STEP, ... For tile t:
    //   S^T from the K operands already in registers;
    //   V half of t landed -> V operands to registers; softmax;
    //   the V half starts loading tile t+1; first half of P.V;
    //   K half of t+1 landed -> K operands to registers; second half of P.V;
    //   the K half starts loading tile t+2.
    // Every half is in flight for about one tile of compute, and the LDS reads
    // of each half overlap the arithmetic that precedes their use.
    constexpr int NH = kHalfLoads<S>;
    uint8_t* const st = lds_st + wv * STAGE_BYTES;
    if (p0 < end) {
      wait_vm<NH>();  // K half of the first tile landed (its V half may still be loading)
      stage_read_k<S>(tk, st, c16, q4);
      if (p0 + STEP < end) stage_issue<S, 0>(st, krw, ksrw, p0 + STEP, end - p0 - STEP, krow, srow, lane);
    }
    for (; p0 < end; p0 += STEP) {
      const int pn = p0 + STEP;
      const bool more = pn < end;
      const bool more2 = pn + STEP < end;
      // (the blocks written out, not as a loop: a one-trip unrolled loop
      // around the scores changed the register allocation of the decode
      // instances, 248 -> 292 registers at head_dim 256)
      float z[RB][2][4];
      auto scores = [&](int rb) {
        if constexpr (CHUNK)
          tile_scores<S>(tk, rlo[rb] - p0, min(rhi[rb], end) - p0, z[rb], qb + rb * QB, corr[rb], a.c2, q4);
        else tile_scores<S>(tk, end - p0, z[rb], qb, corr[rb], a.c2, q4);
      };
      scores(0);
      if constexpr (RB == 2) scores(1);
      if (more) wait_vm<NH>();  // V half of this tile landed; the next K half is in flight
      else wait_vm<0>();
      VRegs<S> tv;
      stage_read_v<S>(tv, st, c16, q4);
      f16x8 pa[RB];
      pa[0] = tile_softmax<S>(z[0], acc[0], q4);
      if constexpr (RB == 2) pa[1] = tile_softmax<S>(z[1], acc[1], q4);
      if (more) stage_issue<S, 1>(st, vrw, vsrw, pn, end - pn, krow, srow, lane);
      tile_pv_rows<S, 1, RB>(tv, pa, acc);
      if (more) {
        wait_vm<NH>();  // K half of the next tile landed; its V half is in flight
        stage_read_k<S>(tk, st, c16, q4);
      }
      tile_pv_rows<S, 2, RB>(tv, pa, acc);
      if (more2) stage_issue<S, 0>(st, krw, ksrw, pn + STEP, end - pn - STEP, krow, srow, lane);
    }
  } else if constexpr (kMix) {
    // Pipeline over this wavefront's tiles: at the start of tile t all of its
    // loads have landed; its fp32 operands are copied from the stage into
    // registers, then tile t + 1's int8 operands (to a second register set)
    // and fp32 tile (to the stage) start loading, in flight while t is
    // computed.
    uint8_t* const st = lds_st + wv * STAGE_BYTES;
    const uint32_t frow = KI8 ? vrow : krow;
    KRegs<S> tkn = {};  // the int8 operands of tile t + 1 (after the last tile: the last ones again)
    VRegs<S> tvn = {};
    for (; p0 < end; p0 += STEP) {
      const int pn = p0 + STEP;
      const bool more = pn < end;
      wait_vm0_visible();
      if constexpr (KI8) f32stage_read_v<S>(tv, st, c16, q4);
      else f32stage_read_k<S>(tk, st, c16, q4);
      if (more) {
        if constexpr (KI8) load_k_global<S>(tkn, krs, ksrs, pn, end, krow, srow, c16, q4);
        else load_v_global<S>(tvn, vrs, vsrs, pn, end, vrow, srow, c16, q4);
        f32stage_issue<S, !KI8>(st, frw, pn, end - pn, frow, lane);
      }
      float z[2][4];
      if constexpr (CHUNK) tile_scores<S>(tk, rlo[0] - p0, min(rhi[0], end) - p0, z, qb, corr[0], a.c2, q4);
      else tile_scores<S>(tk, end - p0, z, qb, corr[0], a.c2, q4);
      const f16x8 pa = tile_softmax<S>(z, acc[0], q4);
      tile_pv<S>(tv, pa, acc[0]);
      if constexpr (KI8) tk = tkn;
      else tv = tvn;
    }
  } else {
    for (; p0 < end; p0 += STEP) {
      load_k_global<S>(tk, krs, ksrs, p0, end, krow, srow, c16, q4);
      load_v_global<S>(tv, vrs, vsrs, p0, end, vrow, srow, c16, q4);
      float z[2][4];
      if constexpr (CHUNK) tile_scores<S>(tk, rlo[0] - p0, min(rhi[0], end) - p0, z, qb, corr[0], a.c2, q4);
      else tile_scores<S>(tk, end - p0, z, qb, corr[0], a.c2, q4);
      const f16x8 pa = tile_softmax<S>(z, acc[0], q4);
      tile_pv<S>(tv, pa, acc[0]);
    }
  }

  // ---- merge the wavefronts of the workgroup -----------------------------------
  // Each wavefront stores its unscaled O rows (in its own stage), its max and
  // its sum; after one barrier every lane combines the wavefronts for one
  // (head, 4 dims) with weights 2^(m_k - M). Row block rb has nr rows.
  auto merge = [&](const int rb, const int nr) {
    if (q4 == 0) sm_m[wv][c16] = acc[rb].m_ref;
    if (c16 == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_l[wv][4 * q4 + i] = acc[rb].l[i];
    }
    {
      float* slot = reinterpret_cast<float*>(lds_st + wv * SLOT_PITCH);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * q4 + i;
        if (h < nr) {
#pragma unroll
          for (int n4 = 0; n4 < S::VB / 4; ++n4) {
            const int f = (S::VB * c16 + 4 * n4) / 4;  // float4 index within the row
            const float4 v = {acc[rb].o[4 * n4 + 0][i], acc[rb].o[4 * n4 + 1][i], acc[rb].o[4 * n4 + 2][i],
                              acc[rb].o[4 * n4 + 3][i]};
            reinterpret_cast<float4*>(slot + h * D)[merge_swz(f)] = v;
          }
        }
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < nr * (D / 4); idx += NW * 64) {
      const int h = idx / (D / 4);
      const int d = 4 * (idx % (D / 4));
      const float zn = own_new ? z_new(h) : -INFINITY;  // the fused new position
      float M = zn;
#pragma unroll
      for (int k = 0; k < NW; ++k) M = fmaxf(M, sm_m[k][h]);
      const int f = merge_swz(d / 4);
      float4 v = {0.f, 0.f, 0.f, 0.f};
      if (own_new) {
        const float wn = __builtin_amdgcn_exp2f(zn - M);
        const float4 u = *reinterpret_cast<const float4*>(&nw_val[1][d]);
        v = make_float4(wn * u.x, wn * u.y, wn * u.z, wn * u.w);
      }
#pragma unroll
      for (int k = 0; k < NW; ++k) {
        const float mk = sm_m[k][h];
        const float wk = mk == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mk - M);
        const float4 u = reinterpret_cast<const float4*>(lds_st + k * SLOT_PITCH)[h * (D / 4) + f];
        v.x = fmaf(wk, u.x, v.x);
        v.y = fmaf(wk, u.y, v.y);
        v.z = fmaf(wk, u.z, v.z);
        v.w = fmaf(wk, u.w, v.w);
      }
      put_o(rowid(16 * rb + h), d, v);
    }
    if (threadIdx.x < nr) {
      const int h = threadIdx.x;
      const float zn = own_new ? z_new(h) : -INFINITY;
      float M = zn;
#pragma unroll
      for (int k = 0; k < NW; ++k) M = fmaxf(M, sm_m[k][h]);
      float l = own_new ? __builtin_amdgcn_exp2f(zn - M) : 0.0f;
#pragma unroll
      for (int k = 0; k < NW; ++k) {
        const float mk = sm_m[k][h];
        if (mk != -INFINITY) l += sm_l[k][h] * __builtin_amdgcn_exp2f(mk - M);
      }
      put_ml(rowid(16 * rb + h), make_float2(M, l));
    }
  };
  if constexpr (RB == 1) {
    merge(0, nh);
    arrive_and_combine();
  } else {
    merge(0, min(16, nh));
    if (nh > 16) {
      __syncthreads();  // the first block's slots and maxima have been read
      merge(1, nh - 16);
    }
  }
}

template <int D, bool KI8, bool VI8, bool G64>
static void launch_partial_t(const PartialArgs& a, dim3 grid, hipStream_t s) {
  // Four wavefronts per workgroup, and several workgroups per compute unit
  // (two at D = 256, three at D = 128): one workgroup's start (query load,
  // first tiles in flight) and end (merge, partial stores) overlap another's
  // streaming, which measured faster than one 8-wavefront workgroup per unit.
  constexpr int NW = kPartialWaves;
  if constexpr (KI8 && VI8) {
    if (a.out) {  // the one-launch step of kv_decode_attn
      hipLaunchKernelGGL((kvq_partial_kernel<D, KI8, VI8, G64, NW, false, 1, true>), grid, dim3(NW * 64), 0, s, a);
      return;
    }
  }
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
                   const uint16_t* k_scales, const uint16_t* v_scales, const uint16_t* k_new,
                   const uint16_t* v_new, const uint16_t* q, int32_t batch, int32_t n_q_heads,
                   const int32_t* d_seq_lens, int32_t window, float sm_scale, const kvq_plan_t& plan,
                   void* ws, void* stream, uint16_t* out, uint32_t* arrive) {
  if ((out != nullptr) != (arrive != nullptr)) return KVQ_ERR_NULL;
  if (out && !one_launch_ok(L, batch, n_q_heads, plan)) return KVQ_ERR_UNSUPPORTED;
  PartialArgs a{};
  a.out = out;
  a.arrive = arrive;
  a.rows_per_block = kHeadsPerBlock;
  // the partial region, when one buffer resource covers it (write-through stores)
  if (workspace_bytes(batch, n_q_heads, plan.n_splits, L.head_dim) <= 0x7fffffff)
    a.ws_bytes = (uint32_t)workspace_bytes(batch, n_q_heads, plan.n_splits, L.head_dim);
  if (out) {
    a.rows_per_block = one_launch_rows(L.head_dim, n_q_heads / L.n_kv_heads);
  }
  a.k_store = k_store;
  a.v_store = v_store;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.k_new = k_new;
  a.v_new = v_new;
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
  a.head_blocks = (a.G + a.rows_per_block - 1) / a.rows_per_block;
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

template <int D, bool KI8, bool VI8, bool G64, int RB>
static void launch_rows_t(const PartialArgs& a, dim3 grid, hipStream_t s) {
  constexpr int NW = kPartialWaves;
  hipLaunchKernelGGL((kvq_partial_kernel<D, KI8, VI8, G64, NW, true, RB>), grid, dim3(NW * 64), 0, s, a);
}

template <int D>
static void dispatch_rows(const kvq_layout& L, const PartialArgs& a, dim3 grid, hipStream_t s, int rb) {
  const bool ki8 = L.k_dtype == KVQ_STORE_INT8, vi8 = L.v_dtype == KVQ_STORE_INT8;
  const bool g64 = L.scale_group == 64 && L.head_dim != 64;  // at D = 64 both granularities coincide
  if (ki8 && vi8) {
    if (rb == 2) g64 ? launch_rows_t<D, true, true, true, 2>(a, grid, s) : launch_rows_t<D, true, true, false, 2>(a, grid, s);
    else g64 ? launch_rows_t<D, true, true, true, 1>(a, grid, s) : launch_rows_t<D, true, true, false, 1>(a, grid, s);
  } else if (ki8) {
    g64 ? launch_rows_t<D, true, false, true, 1>(a, grid, s) : launch_rows_t<D, true, false, false, 1>(a, grid, s);
  } else if (vi8) {
    g64 ? launch_rows_t<D, false, true, true, 1>(a, grid, s) : launch_rows_t<D, false, true, false, 1>(a, grid, s);
  } else {
    launch_rows_t<D, false, false, false, 1>(a, grid, s);
  }
}

int launch_chunk_rows(const kvq_layout& L, const void* k_store, const void* v_store, const uint16_t* k_scales,
                      const uint16_t* v_scales, const uint16_t* q, int32_t batch, int32_t n_tok, int32_t n_q_heads,
                      const int32_t* d_start_pos, int32_t window, float sm_scale, const kvq_plan_t& plan, void* ws,
                      void* stream) {
  if (has_q4(L)) return KVQ_ERR_UNSUPPORTED;
  PartialArgs a{};
  a.k_store = k_store;
  a.v_store = v_store;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.q = q;
  a.start_pos = d_start_pos;
  a.T = n_tok;
  const int64_t ws_rows = (int64_t)batch * n_tok * n_q_heads * plan.n_splits;
  a.ws_o = static_cast<float*>(ws);
  a.ws_ml = static_cast<float*>(ws) + ws_rows * L.head_dim;
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
  // One or two row blocks of 16 per workgroup (all rows sharing every key and
  // value operand).
  const int per_wg = chunk_rows_per_block(L, n_tok, a.G);
  const int rb = per_wg / kHeadsPerBlock;
  a.head_blocks = (int32_t)(((int64_t)n_tok * a.G + per_wg - 1) / per_wg);
  a.n_splits = plan.n_splits;
  a.chunk = plan.chunk;
  a.window = window;
  a.c2 = sm_scale * kLog2e;
  dim3 grid(plan.n_splits, L.n_kv_heads * a.head_blocks, batch);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (L.head_dim) {
    case 64: dispatch_rows<64>(L, a, grid, s, rb); break;
    case 128: dispatch_rows<128>(L, a, grid, s, rb); break;
    case 256: dispatch_rows<256>(L, a, grid, s, rb); break;
    default: return KVQ_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace kvq
