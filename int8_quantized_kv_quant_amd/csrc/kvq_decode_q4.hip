// kv_decode_attn_splitk for the 4-bit layouts: q4 K and V (q4_0) and int8 K with
// q4 V (k8v4), head_dim 256, on the gfx950 matrix cores.
//
// Strata PR 2698, "Not in this PR": the 4-bit stores hold Q4_0 blocks of rows
// rotated by the 256-point Hadamard transform; K is rotated together with the
// queries and V's output is rotated back. genie-ai-runtime v1.3.0 "split-K
// decode attention": per-split online-softmax partials, combined by the reduce.
//
// Mapping as in the int8 kernel (kvq_decode.hip): a workgroup of four
// wavefronts = (sequence, kv head, up to 16 query heads, split); wavefronts take
// 32-position tiles round-robin, each staging its tiles' K and V halves in LDS
// with direct-to-LDS loads, one half refilling while the other is computed.
//
// Query. A q4 K store holds rotated keys, so the query rows are rotated the
// same way in LDS (fwht256 in fp32, lane exchanges in registers) before any
// score; with H / 16 orthonormal, q_rot . k_rot = q . k. The rotated rows are
// kept as hi + lo fp16 terms (22 significant bits), with their fp32 sums per
// Q4_0 block; each lane holds its operands of them in registers for the whole
// split.
// Keys (q4), exact scores. One pair of MFMAs v_mfma_f32_16x16x32_f16 contracts
// one Q4_0 block (32 dims) of 16 positions with the hi and the lo query terms;
// the codes enter as the fp16 subnormals code * 2^-24 (a byte permute, no
// arithmetic), so every product is exact. Each block's fp32 result, less 8
// times the query's block sum, is scaled by the position's fp16 block scale in
// fp32: the key (code - 8) * d is never rounded. (Rounding the rotated query
// and fp16((code - 8) * d) instead measured up to 2.0e-3 on short, peaked
// contexts with 16 query heads per kv head.)
// Keys (int8, k8v4): the int8 kernel's operands and scores, unrotated.
// Values (q4). Lane (column c16) holds dims 16 c16 .. +15, i.e. the low
// (c16 even) or high (c16 odd) nibbles of 16 bytes of block c16 / 2, masked in
// place (bytes q or 16 q), transposed per position pair by byte permutes into
// the fp16 operand (code - 8) * d_b, one rounding, exactly as the int8 kernel
// builds code * scale: 1024 + byte (exact) minus 1032 or 1152 gives q - 8 or
// 16 (q - 8), and the high lanes multiply by d_b / 16 (exact).
// Output. O of each split stays in the rotated basis through the softmax; the
// merged partial rows are rotated back (fwht256, fp32) before they are
// written, so the reduce (linear in O) combines unrotated rows.
// Chunk rows (the CHUNK instances; Strata PR 2698 "What it does": verify
// windows read the same cache as decode). The 16 rows of a workgroup are
// (token, head) pairs t * G + h of a chunk of T tokens at positions start + t,
// each rotated like a decode query and masking keys outside its own causal
// (and window) range; the partials go to rows (b, t, hq) for the same reduce.
#include <math.h>

#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_q4.h"
#include "kvq_q4_tile.h"
#include "kvq_tile.h"

namespace kvq {

struct Q4Args {
  const void* k_store;
  const void* v_store;
  const uint16_t* k_scales;
  const uint16_t* v_scales;
  // Fused append: the new token's K and V rows, fp16 [B][n_kv][D] (null: none);
  // row L - 1 of the stores and scales is then written through the pointers
  // above (the fused entry point receives them writable).
  const uint16_t* k_new;
  const uint16_t* v_new;
  const uint16_t* q;
  const int32_t* seq_lens;
  float* ws_o;   // [B][Hq][n_splits][D]
  float* ws_ml;  // [B][Hq][n_splits][2]
  int64_t s_seq, s_pos, s_head;     // element strides (a q4 element is half a byte)
  int64_t ss_seq, ss_pos, ss_head;  // fp16 scale strides
  int32_t max_ctx;
  int32_t n_kv, G, n_q, head_blocks;
  int32_t n_splits, chunk, window;
  float c2;  // sm_scale * log2(e)
  // Chunk attention through this kernel (the CHUNK instances): T tokens per
  // sequence at positions start_pos[b] + t; the query rows of a kv head are
  // its (token, head) pairs t * G + h in blocks of 16 (head_blocks of them), q
  // is fp16 [B][T][n_q][D], and the partial rows are (b, t, hq).
  const int32_t* start_pos;
  int32_t T;
};

// ---- values ---------------------------------------------------------------------------
// v[e][w]: bytes holding the codes of dims 16 c16 + 4 w .. +3 at position
// kpos(e, q4) (q for even c16, 16 q for odd c16); vs[e]: that position's scale
// of block c16 / 2.
struct VQ4Regs {
  uint32_t v[8][4];
  uint32_t vs[8];
};

template <bool KQ4, bool KG64>
__device__ __forceinline__ void read_v_q4(VQ4Regs& t, const uint8_t* __restrict__ st, int c16, int q4) {
  using T = Q4Stage<KQ4, KG64>;
  const uint32_t mask = (c16 & 1) ? 0xF0F0F0F0u : 0x0F0F0F0Fu;
  const int blk = c16 >> 1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int r = kpos(e, q4);
    const u32x4 raw = *reinterpret_cast<const u32x4*>(st + T::V_OFF + r * T::VRB + 16 * (blk ^ swz<8>(r)));
#pragma unroll
    for (int w = 0; w < 4; ++w) t.v[e][w] = raw[w] & mask;
    t.vs[e] = *reinterpret_cast<const uint16_t*>(st + T::VS_OFF + r * 16 + 2 * blk);
  }
}

// O += P . V_hat with V_hat = fp16((code - 8) * d) and l += P . 1; PART 1 and 2
// split the output columns in halves (l with PART 2) so that a wait can sit
// between them.
// vbias: fp16 pair (-1032, -1032) for even c16 lanes, (-1152, -1152) for odd
// ones; vsc: (1, 1) or (1/16, 1/16).
template <int PART>
__device__ __forceinline__ void pv_q4(const VQ4Regs& t, f16x8 pa, WaveAcc<Shape<256, true, true, true>>& acc,
                                      uint32_t vbias, f16x2 vsc) {
  constexpr int W0 = PART == 2 ? 2 : 0, W1 = PART == 1 ? 2 : 4;
  f16x2 sv[4];
#pragma unroll
  for (int pi = 0; pi < 4; ++pi)
    sv[pi] = as_h2(__builtin_amdgcn_perm(t.vs[2 * pi + 1], t.vs[2 * pi], 0x05040100u)) * vsc;
#pragma unroll
  for (int w = W0; w < W1; ++w) {
    uint32_t z01[4], z23[4];
#pragma unroll
    for (int pi = 0; pi < 4; ++pi) {
      z01[pi] = zip_lo(t.v[2 * pi + 1][w], t.v[2 * pi][w]);
      z23[pi] = zip_hi(t.v[2 * pi + 1][w], t.v[2 * pi][w]);
    }
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      u32x4 r;
#pragma unroll
      for (int pi = 0; pi < 4; ++pi) {
        const uint32_t src = bb < 2 ? z01[pi] : z23[pi];
        const uint32_t biased = (bb & 1) ? biased_h2_hi(src) : biased_h2_lo(src);  // 1024 + byte
        const f16x2 c = as_h2(biased) + as_h2(vbias);                              // q - 8 or 16 (q - 8), exact
        r[pi] = as_u32(c * sv[pi]);                                                 // fp16((code - 8) * d)
      }
      acc.o[4 * w + bb] = mfma16(pa, __builtin_bit_cast(f16x8, r), acc.o[4 * w + bb]);
    }
  }
  if constexpr (PART != 1) {
    const f16x8 ones = {(f16)1, (f16)1, (f16)1, (f16)1, (f16)1, (f16)1, (f16)1, (f16)1};
    acc.l = mfma16(pa, ones, acc.l);
  }
}

// Float4 position of float4 f of a merge-slot row: the 16 lanes that write one
// row at a time hold f = 4c + n for c = 0..15; XOR-ing bits 0-1 with bits 4-5
// spreads them over the 16 distinct 16-byte bank groups.
__device__ __forceinline__ int slot_swz(int f) { return f ^ ((f >> 4) & 3); }

// ---- kernel ------------------------------------------------------------------------
template <bool KQ4, bool KG64, bool CHUNK = false>
__global__ __launch_bounds__(256) void kvq_partial_q4_kernel(Q4Args a) {
  constexpr int D = 256, NW = 4;
  using T = Q4Stage<KQ4, KG64>;
  using SA = Shape<256, true, true, true>;  // accumulators (16 heads x 256 dims per wavefront)
  using SK = Shape<256, true, true, KG64>;  // int8 keys (k8v4)
  constexpr int kQGL = KG64 ? 16 : D / 4;   // lanes of one int8 key scale group in the fused quantizer
  static_assert(D % (32 * NW) == 0, "the new position's score: 8-dim steps per lane");
  constexpr int SLOT_BYTES = 16 * D * 4;    // merge slot: 16 head rows of D floats
  constexpr int PITCH = T::BYTES > SLOT_BYTES ? T::BYTES : SLOT_BYTES;
  constexpr int QROW = QOperand<SA>::ROW;
  __shared__ __attribute__((aligned(16))) uint8_t lds_st[NW * PITCH];
  __shared__ __attribute__((aligned(16))) uint8_t lds_q[16 * QROW];
  // q4 keys: the lo fp16 terms of the rotated query rows (lds_q holds the hi
  // terms) and each row's fp32 sums over the 8 Q4_0 blocks.
  __shared__ __attribute__((aligned(16))) uint8_t lds_ql[KQ4 ? 16 * QROW : 16];
  __shared__ __attribute__((aligned(16))) uint16_t lds_qsh[16][8];  // block sums, hi fp16 terms
  __shared__ __attribute__((aligned(16))) uint16_t lds_qsl[16][8];  // and lo terms
  __shared__ float sm_m[NW][16];
  __shared__ float sm_l[NW][16];
  // The new token's rows when the append is fused ([0] = K, [1] = V): the fp16
  // input (landing place of its direct-to-LDS load), the dequantized values (in
  // the stored, rotated basis for a q4 store), the bytes and scales for the
  // cache, and the new position's scores.
  __shared__ __attribute__((aligned(16))) uint16_t nw_in[2][D];
  __shared__ __attribute__((aligned(16))) float nw_val[2][D];
  __shared__ __attribute__((aligned(16))) uint32_t nw_code[2][D / 4];
  __shared__ uint16_t nw_scale[2][D / kQ4Block];
  __shared__ float nw_z[NW][16];

  const int split = blockIdx.x;
  const int hk = blockIdx.y / a.head_blocks;
  const int hblk = blockIdx.y % a.head_blocks;
  const int b = blockIdx.z;
  // Query rows of the workgroup (up to 16) and the keys [lo, L) they attend.
  // Decode: heads hblk * 16 .. of kv head hk at context seq_lens[b]. Chunk:
  // flat rows fr0 + r = t * G + h of kv head hk; token t sits at s0 + t and
  // attends [max(0, s0 + t + 1 - window) (window > 0), s0 + t + 1).
  const int fr0 = hblk * 16;
  const int nh = CHUNK ? min(16, a.T * a.G - fr0) : min(16, a.G - fr0);
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
  // Split s takes the blocks s, s + S, ... of BLK positions of [lo, L),
  // S = min(n_splits, ceil((L - lo) / chunk)) (block-cyclic, as in the int8
  // kernel).
  constexpr int BLK = NW * kTile;
  const int n_used = (int)min((int64_t)a.n_splits, ((int64_t)L - lo + a.chunk - 1) / a.chunk);
  const int64_t start64 = (int64_t)lo + (int64_t)split * BLK;
  if (split >= n_used || start64 >= L) {  // empty split: (m, l) = (-inf, 0), O not written
    if (threadIdx.x < nh) ml[rowid(threadIdx.x)] = make_float2(-INFINITY, 0.0f);
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

  // ---- buffer resources of this (sequence, kv head) slice: each ends at the
  // last row of the context.
  const int64_t st_off = (int64_t)b * a.s_seq + (int64_t)hk * a.s_head;  // elements
  const int64_t sc_off = (int64_t)b * a.ss_seq + (int64_t)hk * a.ss_head;
  const int64_t last = (int64_t)(L - 1) * a.s_pos + D;
  const uint32_t krow = (uint32_t)(KQ4 ? a.s_pos / 2 : a.s_pos);
  const uint32_t vrow = (uint32_t)(a.s_pos / 2);
  const uint32_t srow = (uint32_t)(a.ss_pos * 2);
  const u32x4 krw = rsrc_words(static_cast<const char*>(a.k_store) + (KQ4 ? st_off / 2 : st_off),
                               (uint32_t)(KQ4 ? last / 2 : last));
  const u32x4 vrw = rsrc_words(static_cast<const char*>(a.v_store) + st_off / 2, (uint32_t)(last / 2));
  const u32x4 ksrw = rsrc_words(a.k_scales + sc_off, (uint32_t)(((int64_t)(L - 1) * a.ss_pos + T::KNG) * 2));
  const u32x4 vsrw = rsrc_words(a.v_scales + sc_off, (uint32_t)(((int64_t)(L - 1) * a.ss_pos + D / kQ4Block) * 2));

  const int STEP = BLK * n_used;  // from a tile to the same tile of the split's next block
  int p0 = start + wv * kTile;
  // The new K (wavefront 0) or V (wavefront 1) row when the append is fused,
  // the query rows (4 per wavefront; rows past nh read as zeros), then this
  // wavefront's first tile, all as counted direct-to-LDS loads.
  if (own_new && wv < 2) {
    const uint16_t* src = (wv == 0 ? a.k_new : a.v_new) + ((int64_t)b * a.n_kv + hk) * D;
    if (lane < D / 8) dma<16>(rsrc_words(src, 2 * D), lds_addr_of(reinterpret_cast<const uint8_t*>(nw_in[wv])),
                              16u * lane, 0u);
  }
  if constexpr (CHUNK) {  // the rows of this block: q [b][t][hk * G + h]
    const u32x4 qrs = rsrc_words(a.q + (int64_t)b * a.T * a.n_q * D, (uint32_t)((int64_t)a.T * a.n_q * D * 2));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wv * 4 + i;
      const int fr = fr0 + r;
      const uint32_t off = (uint32_t)((((int64_t)(fr / a.G) * a.n_q + hk * a.G + fr % a.G) * D) * 2);
      if (lane < D / 8) dma<16>(qrs, lds_addr_of(lds_q + r * QROW), r < nh ? off + 16 * lane : kOOB, 0u);
    }
  } else {
    const u32x4 qrs = rsrc_words(a.q + ((int64_t)b * a.n_q + hq0) * D, (uint32_t)(nh * D * 2));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wv * 4 + i;
      if (lane < D / 8) dma<16>(qrs, lds_addr_of(lds_q + r * QROW), r < nh ? (uint32_t)(r * 2 * D + 16 * lane) : kOOB, 0u);
    }
  }
  uint8_t* const st = lds_st + wv * PITCH;
  if (p0 < end) {
    issue_half<KQ4, KG64, 0>(st, krw, ksrw, p0, end - p0, krow, srow, lane);
    issue_half<KQ4, KG64, 1>(st, vrw, vsrw, p0, end - p0, vrow, srow, lane);
    wait_vm<T::NK + T::NV>();  // the query rows landed
  } else {
    wait_vm<0>();
  }
  if (own_new && wv < 2) {
    // The new row through the store's quantizer (as kv_quant_append): codes and
    // scales for the cache, dequantized values for this workgroup's attention.
    const uint32_t raw0 = reinterpret_cast<const uint32_t*>(nw_in[wv])[2 * lane];
    const uint32_t raw1 = reinterpret_cast<const uint32_t*>(nw_in[wv])[2 * lane + 1];
    const uint32_t hb[4] = {raw0 & 0xffffu, raw0 >> 16, raw1 & 0xffffu, raw1 >> 16};
    float4 val;
    if (wv == 1 || KQ4) {  // a q4 store: rotate, Q4_0
      float y[4] = {h_bits_to_f32(hb[0]), h_bits_to_f32(hb[1]), h_bits_to_f32(hb[2]), h_bits_to_f32(hb[3])};
      fwht256(y, lane);
      uint16_t sb;
      uint32_t own;
      const uint32_t packed = q4_quantize(y, lane, &sb, &own);
      const float d = h_bits_to_f32(sb);
      val = make_float4((float)((int)(own & 0xff) - 8) * d, (float)((int)((own >> 8) & 0xff) - 8) * d,
                        (float)((int)((own >> 16) & 0xff) - 8) * d, (float)((int)(own >> 24) - 8) * d);
      if ((lane & 7) < 4) nw_code[wv][4 * (lane >> 3) + (lane & 7)] = packed;  // byte 16 (lane >> 3) + 4 (lane & 7)
      if ((lane & 7) == 0) nw_scale[wv][lane >> 3] = sb;
    } else {  // int8 keys (k8v4)
      uint16_t sb;
      const uint32_t code = quantize4<kQGL>(hb, &sb);
      const float sc = h_bits_to_f32(sb);
      val = make_float4((float)(int8_t)(code & 0xff) * sc, (float)(int8_t)((code >> 8) & 0xff) * sc,
                        (float)(int8_t)((code >> 16) & 0xff) * sc, (float)(int8_t)(code >> 24) * sc);
      nw_code[wv][lane] = code;
      if (lane % kQGL == 0) nw_scale[wv][lane / kQGL] = sb;
    }
    *reinterpret_cast<float4*>(&nw_val[wv][4 * lane]) = val;
  }
  if constexpr (KQ4) {
    // Rotate this wavefront's 4 query rows: lane l holds dims 4l .. 4l+3. The
    // hi terms replace the row in lds_q, the lo terms go to lds_ql, dims 16..31
    // of each block (lanes with l & 7 >= 4) divided by 16 (exact; see
    // scores_q4), and lanes 8j hold the sum over block j (dims 32j .. 32j+31,
    // lanes 8j .. 8j+7), split hi + lo into lds_qsh / lds_qsl.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wv * 4 + i;
      uint8_t* qr = lds_q + r * QROW + 8 * lane;
      const u32x2 raw = *reinterpret_cast<const u32x2*>(qr);
      float v[4] = {h_bits_to_f32(raw.x & 0xffffu), h_bits_to_f32(raw.x >> 16), h_bits_to_f32(raw.y & 0xffffu),
                    h_bits_to_f32(raw.y >> 16)};
      fwht256(v, lane);
      f16 hi[4], lo[4];
      const float f = (lane & 7) >= 4 ? 0.0625f : 1.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hi[e] = (f16)(v[e] * f);
        lo[e] = (f16)(v[e] * f - (float)hi[e]);
      }
      const f16x2 h01 = {hi[0], hi[1]}, h23 = {hi[2], hi[3]}, l01 = {lo[0], lo[1]}, l23 = {lo[2], lo[3]};
      *reinterpret_cast<u32x2*>(qr) = (u32x2){as_u32(h01), as_u32(h23)};
      *reinterpret_cast<u32x2*>(lds_ql + r * QROW + 8 * lane) = (u32x2){as_u32(l01), as_u32(l23)};
      float bs = (v[0] + v[1]) + (v[2] + v[3]);
      bs += lane_xor<1>(bs);
      bs += lane_xor<2>(bs);
      bs += lane_xor<4>(bs);
      if ((lane & 7) == 0) {
        const f16 bh = (f16)bs;
        lds_qsh[r][lane >> 3] = __builtin_bit_cast(uint16_t, bh);
        lds_qsl[r][lane >> 3] = __builtin_bit_cast(uint16_t, (f16)(bs - (float)bh));
      }
    }
  }
  __syncthreads();  // every query row in LDS (rotated for a q4 K store), the new rows quantized
  // ---- fused append: the new row into the cache (one head block writes it),
  // issued right after the quantization so that its store latency overlaps
  // the tiles (no workgroup of this launch reads position L - 1 from the
  // cache; the explicit load counts below then over-count by these stores at
  // most, which only makes a wait stricter)
  if (own_new && hblk == 0 && wv < 2) {
    const int64_t r = (int64_t)b * a.s_seq + (int64_t)(L - 1) * a.s_pos + (int64_t)hk * a.s_head;  // elements
    const int64_t sr = (int64_t)b * a.ss_seq + (int64_t)(L - 1) * a.ss_pos + (int64_t)hk * a.ss_head;
    uint16_t* sc = const_cast<uint16_t*>(wv == 0 ? a.k_scales : a.v_scales);
    if (wv == 1 || KQ4) {  // 128 bytes and 8 scales
      uint8_t* store = static_cast<uint8_t*>(const_cast<void*>(wv == 0 ? a.k_store : a.v_store));
      if (lane < D / 8) reinterpret_cast<uint32_t*>(store + r / 2)[lane] = nw_code[wv][lane];
      if (lane < D / kQ4Block) sc[sr + lane] = nw_scale[wv][lane];
    } else {
      int8_t* store = static_cast<int8_t*>(const_cast<void*>(a.k_store));
      reinterpret_cast<uint32_t*>(store + r)[lane] = nw_code[0][lane];
      if (lane % kQGL == 0) sc[sr + lane / kQGL] = nw_scale[0][lane / kQGL];
    }
  }
  const uint8_t* const qrow = lds_q + c16 * QROW;
  if (own_new) {
    // Partial scores of the new position for the 16 heads (rows beyond nh are
    // zero), a quarter of the dims per wavefront: lane 4h + r sums dims
    // 64 wv + 16 r .. + 16 of head h. For q4 keys the query is the rotated row,
    // hi + lo (dims 16..31 of each block stored divided by 16). The merge adds
    // the wavefronts' sums.
    const int h = lane >> 2, r = lane & 3;
    const int d0 = wv * (D / NW) + r * (D / (4 * NW));
    const uint16_t* qr = reinterpret_cast<const uint16_t*>(lds_q + h * QROW);
    const uint16_t* qrl = reinterpret_cast<const uint16_t*>(lds_ql + (KQ4 ? h * QROW : 0));
    const float f = (KQ4 && (d0 & 31) >= 16) ? 16.0f : 1.0f;  // the lane's 16 dims share a half block
    float zs = 0.0f;
#pragma unroll
    for (int d = d0; d < d0 + D / (4 * NW); d += 8) {
      const f16x8 qv = *reinterpret_cast<const f16x8*>(qr + d);
      f16x8 ql = {};
      if constexpr (KQ4) ql = *reinterpret_cast<const f16x8*>(qrl + d);
      const float4 k0 = *reinterpret_cast<const float4*>(&nw_val[0][d]);
      const float4 k1 = *reinterpret_cast<const float4*>(&nw_val[0][d + 4]);
      const float kk[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) zs = fmaf(((float)qv[e] + (float)ql[e]) * f, kk[e], zs);
    }
    zs += lane_xor<1>(zs);
    zs += lane_xor<2>(zs);
    if (r == 0) nw_z[wv][h] = zs;  // read in the merge, after its barrier
  }

  const float c2s = a.c2 * 16777216.0f;
  // q4 values: the bias and scale factor of the lane's nibbles (see pv_q4)
  const uint32_t vbias = (c16 & 1) ? 0xE480E480u : kQ4NegBias;
  const f16x2 vsc = (c16 & 1) ? (f16x2){(f16)0.0625f, (f16)0.0625f} : (f16x2){(f16)1.0f, (f16)1.0f};
  // ---- int8 keys: accumulator start values -1152 * (group sum of q) that
  // cancel the code bias.
  constexpr int NC = KQ4 ? 1 : SK::NG;
  float corr[NC];
  if constexpr (!KQ4) {
    const uint8_t* qb = qrow + 32 * q4;
    float qsum[SK::NJ];
#pragma unroll
    for (int j = 0; j < SK::NJ; ++j) {
      const f16x8 h0 = q_get(qb, j, 0), h1 = q_get(qb, j, 1);
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += (float)h0[e] + (float)h1[e];
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      qsum[j] = s;
    }
#pragma unroll
    for (int g = 0; g < NC; ++g) {
      float t = 0.0f;
      if (KG64) {
        t = qsum[g];
      } else {
#pragma unroll
        for (int j = 0; j < SK::NJ; ++j) t += qsum[j];
      }
      corr[g] = -kCodeBias * t;
    }
  }

  WaveAcc<SA> acc;
#pragma unroll
  for (int n = 0; n < SA::VB; ++n) acc.o[n] = (f32x4){0.f, 0.f, 0.f, 0.f};
  acc.l = (f32x4){0.f, 0.f, 0.f, 0.f};
  acc.m_ref = -INFINITY;

  // ---- pipeline over this wavefront's tiles (as in the int8 kernel): for tile
  // t, scores from the K operands in registers; V half of t landed -> V
  // operands; softmax; V half starts loading t+1; first half of P.V; K half of
  // t+1 landed -> K operands; second half of P.V; K half starts loading t+2.
  using KR = typename std::conditional<KQ4, KQ4Regs, KRegs<SK>>::type;
  KR tk;
  auto read_k = [&](KR& t) {
    if constexpr (KQ4) read_k_q4<KG64>(t, st, c16, q4);
    else read_k_i8<KG64>(t, st, c16, q4);
  };
  // Tile n of this wavefront keeps its q4 K scale rows in half n & 1 of the K
  // scale region until its scores are taken (the K half of tile n + 2 is
  // issued after them).
  Q4Query qy;  // the rotated query's operands, in registers for the whole split
  if constexpr (KQ4)
    load_q4_query(qy, qrow + 16 * q4, lds_ql + c16 * QROW + 16 * q4, reinterpret_cast<const uint8_t*>(lds_qsh[c16]),
                  reinterpret_cast<const uint8_t*>(lds_qsl[c16]), q4);
  int kpar = 0;
  // Chunk: keys [rlo, rhi) of the lane's query row c16 (none for rows past nh).
  int rlo = 0, rhi = 0;
  if constexpr (CHUNK) {
    const int P = s0 + (fr0 + c16) / a.G;
    rhi = (c16 < nh && P < a.max_ctx) ? P + 1 : 0;
    rlo = a.window > 0 ? max(0, P + 1 - a.window) : 0;
  }
  if (p0 < end) {
    wait_vm<T::NV>();  // K half of the first tile landed (its V half may still be loading)
    read_k(tk);
    if (p0 + STEP < end) issue_half<KQ4, KG64, 0>(st, krw, ksrw, p0 + STEP, end - p0 - STEP, krow, srow, lane, 1);
  }
  for (; p0 < end; p0 += STEP, kpar ^= 1) {
    const int pn = p0 + STEP;
    const bool more = pn < end;
    const bool more2 = pn + STEP < end;
    float z[2][4];
    const int vlo = CHUNK ? rlo - p0 : 0, vhi = CHUNK ? min(rhi, end) - p0 : end - p0;
    // decode, int8 keys: only the context's last tile needs the mask (the same
    // skip measured slower with the q4 keys and in the int8 kernel)
    const bool masked = CHUNK || KQ4 || end - p0 < kTile;
    if constexpr (KQ4) {
      scores_q4(tk, vlo, vhi, z, st + T::KS_OFF + 512 * kpar, qy, c2s, c16, q4);
    } else {
      const uint8_t* qb = qrow + 32 * q4;
      f16x8 qv[4][2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qv[j][0] = q_get(qb, j, 0);
        qv[j][1] = q_get(qb, j, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      scores_i8<KG64>(tk, vlo, vhi, z, qv, corr, a.c2, q4, masked);
    }
    if (more) wait_vm<T::NK>();  // V half of this tile landed; the next K half is in flight
    else wait_vm<0>();
    VQ4Regs tv;
    read_v_q4<KQ4, KG64>(tv, st, c16, q4);
    const f16x8 pa = tile_softmax<SA>(z, acc, q4);
    if (more) issue_half<KQ4, KG64, 1>(st, vrw, vsrw, pn, end - pn, vrow, srow, lane);
    pv_q4<1>(tv, pa, acc, vbias, vsc);
    if (more) {
      wait_vm<T::NV>();  // K half of the next tile landed; its V half is in flight
      read_k(tk);
    }
    pv_q4<2>(tv, pa, acc, vbias, vsc);
    if (more2) issue_half<KQ4, KG64, 0>(st, krw, ksrw, pn + STEP, end - pn - STEP, krow, srow, lane, kpar);
  }

  // ---- merge the wavefronts: slots, one barrier, then wavefront w combines head
  // rows w, w + 4, ... (lane l: dims 4l .. 4l+3), rotates each back and stores it.
  if (q4 == 0) sm_m[wv][c16] = acc.m_ref;
  if (c16 == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sm_l[wv][4 * q4 + i] = acc.l[i];
  }
  {
    float* slot = reinterpret_cast<float*>(lds_st + wv * PITCH);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * q4 + i;
      if (h < nh) {
#pragma unroll
        for (int n4 = 0; n4 < SA::VB / 4; ++n4) {
          const int f = (SA::VB * c16 + 4 * n4) / 4;
          const float4 v = {acc.o[4 * n4 + 0][i], acc.o[4 * n4 + 1][i], acc.o[4 * n4 + 2][i], acc.o[4 * n4 + 3][i]};
          reinterpret_cast<float4*>(slot + h * D)[slot_swz(f)] = v;
        }
      }
    }
  }
  __syncthreads();
  for (int h = wv; h < nh; h += NW) {  // uniform per wavefront: the rotation's shuffles see every lane
    const int f = slot_swz(lane);
    const float zn = own_new ? (nw_z[0][h] + nw_z[1][h] + nw_z[2][h] + nw_z[3][h]) * a.c2 : -INFINITY;  // the fused new position
    float M = zn;
#pragma unroll
    for (int k = 0; k < NW; ++k) M = fmaxf(M, sm_m[k][h]);
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    float l = 0.0f;
    if (own_new) {
      const float wn = __builtin_amdgcn_exp2f(zn - M);
      const float4 u = *reinterpret_cast<const float4*>(&nw_val[1][4 * lane]);
      v[0] = wn * u.x;
      v[1] = wn * u.y;
      v[2] = wn * u.z;
      v[3] = wn * u.w;
      l = wn;
    }
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const float mk = sm_m[k][h];
      const float wk = mk == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mk - M);
      const float4 u = reinterpret_cast<const float4*>(lds_st + k * PITCH)[h * (D / 4) + f];
      v[0] = fmaf(wk, u.x, v[0]);
      v[1] = fmaf(wk, u.y, v[1]);
      v[2] = fmaf(wk, u.z, v[2]);
      v[3] = fmaf(wk, u.w, v[3]);
      l = fmaf(wk, sm_l[k][h], l);
    }
    fwht256(v, lane);  // back to the original basis (H / 16 is its own inverse)
    reinterpret_cast<float4*>(a.ws_o + rowid(h) * D)[lane] = make_float4(v[0], v[1], v[2], v[3]);
    if (lane == 0) ml[rowid(h)] = make_float2(M, l);
  }
}

int launch_partial_q4(const kvq_layout& L, const void* k_store, const void* v_store, const uint16_t* k_scales,
                      const uint16_t* v_scales, const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q,
                      int32_t batch, int32_t n_q_heads, const int32_t* d_seq_lens, int32_t window, float sm_scale,
                      const kvq_plan_t& plan, void* ws, void* stream) {
  if (L.head_dim != 256 || !q4_decode_supported(L)) return KVQ_ERR_UNSUPPORTED;
  Q4Args a{};
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
  a.head_blocks = (a.G + kHeadsPerBlock - 1) / kHeadsPerBlock;
  a.n_splits = plan.n_splits;
  a.chunk = plan.chunk;
  a.window = window;
  a.c2 = sm_scale * kLog2e;
  const dim3 grid(plan.n_splits, L.n_kv_heads * a.head_blocks, batch);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (L.k_dtype == KVQ_STORE_Q4)
    hipLaunchKernelGGL((kvq_partial_q4_kernel<true, false>), grid, dim3(256), 0, s, a);
  else if (L.scale_group == 64)
    hipLaunchKernelGGL((kvq_partial_q4_kernel<false, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((kvq_partial_q4_kernel<false, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

int launch_chunk_rows_q4(const kvq_layout& L, const void* k_store, const void* v_store, const uint16_t* k_scales,
                         const uint16_t* v_scales, const uint16_t* q, int32_t batch, int32_t n_tok, int32_t n_q_heads,
                         const int32_t* d_start_pos, int32_t window, float sm_scale, const kvq_plan_t& plan, void* ws,
                         void* stream) {
  if (L.head_dim != 256 || !q4_decode_supported(L)) return KVQ_ERR_UNSUPPORTED;
  Q4Args a{};
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
  a.head_blocks = (int32_t)(((int64_t)n_tok * a.G + kHeadsPerBlock - 1) / kHeadsPerBlock);
  a.n_splits = plan.n_splits;
  a.chunk = plan.chunk;
  a.window = window;
  a.c2 = sm_scale * kLog2e;
  const dim3 grid(plan.n_splits, L.n_kv_heads * a.head_blocks, batch);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (L.k_dtype == KVQ_STORE_Q4)
    hipLaunchKernelGGL((kvq_partial_q4_kernel<true, false, true>), grid, dim3(256), 0, s, a);
  else if (L.scale_group == 64)
    hipLaunchKernelGGL((kvq_partial_q4_kernel<false, true, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((kvq_partial_q4_kernel<false, false, true>), grid, dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace kvq
