// kv_cache_pack / kv_cache_unpack: a contiguous blob of one sequence's cache
// positions -- codes (or fp32 values, or Q4_0 bytes) with the fp16 scales of
// every int8 or q4 store -- and its placement back into a cache of the same
// store types, scale group, head count and head_dim (any strides).
//
// genie-ai-runtime release v0.1.0-alpha.11, "--int8-kv triage": saving a cache
// means saving its scale region as well; release v0.1.0-alpha.12, "Path F (#45)
// interop guard": int8 bytes saved without their per-head scales read back as
// garbage. The payload therefore always carries the scales next to the codes,
// and the host refuses to place a blob whose layout facts differ.
//
// Payload: K values, V values, then K scales and V scales (stores with scales),
// each region positions-major ([position][kv head][...]) and padded to 16
// bytes. One kernel copies either way: rows of the cache (strided, in a slot)
// to or from the packed regions, 16 bytes per lane for values and one fp16
// scale per lane for scales (a bandwidth-bound gather/scatter); pack writes the
// regions' padding as zeros.
#include <algorithm>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

struct BlobArgs {
  char* store[2];          // K, V store of the sequence (bytes)
  uint16_t* scales[2];     // their fp16 scale arrays at the sequence (null: fp32 store)
  char* blob;              // payload
  int64_t s_pos_b[2], s_head_b[2];  // byte strides of the stores
  int64_t ss_pos, ss_head;          // element strides of the scale arrays
  int64_t code_off[2], scale_off[2];  // region offsets in the payload (bytes)
  int32_t row_bytes[2], ng[2];
  int32_t n_rows, n_kv, pos0, unpack;
};

__global__ __launch_bounds__(256) void kvq_blob_kernel(BlobArgs a) {
  const int part = blockIdx.y;  // 0: K values, 1: V values, 2: K scales, 3: V scales
  const int s = part & 1;
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * 256;
  if (part < 2) {
    const int cpr = a.row_bytes[s] / 16;  // 16-byte chunks per row
    const int64_t total = (int64_t)a.n_rows * cpr;
    for (int64_t i = tid; i < total; i += stride) {
      const int64_t r = i / cpr;
      const int c = (int)(i % cpr);
      const int64_t p = r / a.n_kv, h = r % a.n_kv;
      char* cache = a.store[s] + (a.pos0 + p) * a.s_pos_b[s] + h * a.s_head_b[s] + 16 * c;
      char* blob = a.blob + a.code_off[s] + r * a.row_bytes[s] + 16 * c;
      if (a.unpack) *reinterpret_cast<u32x4*>(cache) = *reinterpret_cast<const u32x4*>(blob);
      else *reinterpret_cast<u32x4*>(blob) = *reinterpret_cast<const u32x4*>(cache);
    }
  } else {
    if (!a.scales[s]) return;
    const int ng = a.ng[s];
    const int64_t total = (int64_t)a.n_rows * ng;
    // The region's padding to 16 bytes is written as zeros (a deterministic payload).
    const int64_t pad = (2 * total + 15) / 16 * 16 - 2 * total;
    if (!a.unpack && tid < pad) a.blob[a.scale_off[s] + 2 * total + tid] = 0;
    for (int64_t i = tid; i < total; i += stride) {
      const int64_t r = i / ng;
      const int j = (int)(i % ng);
      const int64_t p = r / a.n_kv, h = r % a.n_kv;
      uint16_t* cache = a.scales[s] + (a.pos0 + p) * a.ss_pos + h * a.ss_head + j;
      uint16_t* blob = reinterpret_cast<uint16_t*>(a.blob + a.scale_off[s]) + i;
      if (a.unpack) *cache = *blob;
      else *blob = *cache;
    }
  }
}

int launch_blob(const kvq_layout& L, void* k_store, void* v_store, uint16_t* k_scales, uint16_t* v_scales,
                int32_t seq, int32_t pos0, int32_t n_pos, void* blob, bool unpack, void* stream) {
  BlobArgs a{};
  const int dts[2] = {L.k_dtype, L.v_dtype};
  void* stores[2] = {k_store, v_store};
  uint16_t* scs[2] = {k_scales, v_scales};
  const int64_t rows = (int64_t)n_pos * L.n_kv_heads;
  int64_t off = 0;
  for (int s = 0; s < 2; ++s) {
    a.store[s] = static_cast<char*>(stores[s]) + store_bytes((int64_t)seq * L.s_seq, dts[s]);
    a.s_pos_b[s] = store_bytes(L.s_pos, dts[s]);
    a.s_head_b[s] = store_bytes(L.s_head, dts[s]);
    a.row_bytes[s] = (int32_t)store_bytes(L.head_dim, dts[s]);
    a.code_off[s] = off;
    off += blob_region_bytes(store_bytes(rows * L.head_dim, dts[s]));
  }
  for (int s = 0; s < 2; ++s) {
    a.ng[s] = scales_per_row(L, dts[s]);
    a.scales[s] = a.ng[s] ? scs[s] + (int64_t)seq * L.ss_seq : nullptr;
    a.scale_off[s] = off;
    if (a.ng[s]) off += blob_region_bytes(rows * a.ng[s] * 2);
  }
  a.ss_pos = L.ss_pos;
  a.ss_head = L.ss_head;
  a.blob = static_cast<char*>(blob);
  a.n_rows = (int32_t)rows;
  a.n_kv = L.n_kv_heads;
  a.pos0 = pos0;
  a.unpack = unpack ? 1 : 0;
  const int64_t chunks = rows * (L.head_dim * 4 / 16);
  const unsigned gx = (unsigned)std::max<int64_t>(1, std::min<int64_t>((chunks + 255) / 256, 8192));
  hipLaunchKernelGGL(kvq_blob_kernel, dim3(gx, 4), dim3(256), 0, static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace kvq
