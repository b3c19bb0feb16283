// KV-cache layout conversion: token-major pages <-> the blocked layout the attention kernels read.
//
// Paged caches are commonly kept token-major: each (page, KV head) block holds page_size rows of
// head_dim elements.  The attention kernels of this library read the blocked layout instead (K as
// [head_dim / w][page][w] and V as [page / w][head_dim][w], w = 64 bytes of elements), in which
// every matrix-core operand load covers whole 128-byte lines.  This kernel converts a cache between
// the two, one 64-token slice of one (page, KV head) block per workgroup: K moves as 16-byte pieces
// (a permutation of its 64-byte dim tiles), V is transposed through LDS.

#include "common.h"
#include "lbsa.h"

namespace lbsa {

constexpr int kSlice = 64;   // tokens per workgroup (a page is a multiple of 64 tokens)

struct LayoutParams {
  const uint8_t* src_k;
  const uint8_t* src_v;
  uint8_t* dst_k;
  uint8_t* dst_v;
  int32_t Hkv, page, D;
};

// ELEM: element bytes (2 bf16, 1 E4M3).  TO_BLOCKED: token-major -> blocked, else the reverse.
template <int ELEM, bool TO_BLOCKED>
__global__ __launch_bounds__(256) void kv_layout_kernel(LayoutParams p) {
  constexpr int W = 64 / ELEM;                // elements per 64-byte row
  __shared__ __attribute__((aligned(16))) uint8_t sv[kSlice * 128 * ELEM + 16 * kSlice];   // V slice, padded rows
  const int tid = threadIdx.x;
  const int slices = p.page / kSlice;
  const int64_t blk_id = blockIdx.x / slices;           // (page, KV head) block
  const int sb = blockIdx.x - (int)(blk_id * slices);   // 64-token slice of the block
  const int row_bytes = p.D * ELEM;                     // one token-major row
  const int srow = row_bytes + 16;                      // staged V row (padded)
  const size_t blk = (size_t)blk_id * p.page * row_bytes;   // bytes of one block in either layout
  const int gpr = row_bytes / 16;                       // 16-byte granules per token row
  const int tok0 = sb * kSlice;

  // K: granule j of token t's row <-> piece (dim tile j / 4, token t), granule j % 4 of the blocked row
  for (int i = tid; i < kSlice * gpr; i += 256) {
    const int t = i / gpr, j = i - t * gpr;
    const size_t tm = blk + (size_t)(tok0 + t) * row_bytes + 16 * j;
    const size_t bl = blk + ((size_t)(j >> 2) * p.page + tok0 + t) * 64 + 16 * (j & 3);
    if (TO_BLOCKED)
      *reinterpret_cast<u32x4*>(p.dst_k + bl) = *reinterpret_cast<const u32x4*>(p.src_k + tm);
    else
      *reinterpret_cast<u32x4*>(p.dst_k + tm) = *reinterpret_cast<const u32x4*>(p.src_k + bl);
  }

  // V: the slice's kSlice / W token tiles; blocked row (tile, dim d) = W consecutive tokens of dim d
  const int vrows = (kSlice / W) * p.D;   // 64-byte rows of the slice in the blocked layout
  if (TO_BLOCKED) {
    for (int i = tid; i < kSlice * gpr; i += 256) {
      const int t = i / gpr, j = i - t * gpr;
      *reinterpret_cast<u32x4*>(sv + t * srow + 16 * j) =
          *reinterpret_cast<const u32x4*>(p.src_v + blk + (size_t)(tok0 + t) * row_bytes + 16 * j);
    }
    __syncthreads();
    for (int i = tid; i < vrows * 4; i += 256) {   // one 16-byte quarter of a blocked row per step
      const int r = i >> 2, q = i & 3;
      const int tt = r / p.D, d = r - tt * p.D;
      const int t_first = tt * W + q * (16 / ELEM);
      uint8_t out[16];
#pragma unroll
      for (int e = 0; e < 16 / ELEM; ++e)
#pragma unroll
        for (int c = 0; c < ELEM; ++c) out[e * ELEM + c] = sv[(t_first + e) * srow + d * ELEM + c];
      const size_t bl = blk + ((size_t)(tok0 / W + tt) * p.D + d) * 64 + 16 * q;
      *reinterpret_cast<u32x4*>(p.dst_v + bl) = *reinterpret_cast<const u32x4*>(out);
    }
  } else {
    for (int i = tid; i < vrows * 4; i += 256) {
      const int r = i >> 2, q = i & 3;
      const int tt = r / p.D, d = r - tt * p.D;
      const int t_first = tt * W + q * (16 / ELEM);
      const size_t bl = blk + ((size_t)(tok0 / W + tt) * p.D + d) * 64 + 16 * q;
      const u32x4 x = *reinterpret_cast<const u32x4*>(p.src_v + bl);
      const uint8_t* in = reinterpret_cast<const uint8_t*>(&x);
#pragma unroll
      for (int e = 0; e < 16 / ELEM; ++e)
#pragma unroll
        for (int c = 0; c < ELEM; ++c) sv[(t_first + e) * srow + d * ELEM + c] = in[e * ELEM + c];
    }
    __syncthreads();
    for (int i = tid; i < kSlice * gpr; i += 256) {
      const int t = i / gpr, j = i - t * gpr;
      *reinterpret_cast<u32x4*>(p.dst_v + blk + (size_t)(tok0 + t) * row_bytes + 16 * j) =
          *reinterpret_cast<const u32x4*>(sv + t * srow + 16 * j);
    }
  }
}

}  // namespace lbsa

extern "C" int attn_kv_layout(const void* src_k, const void* src_v, void* dst_k, void* dst_v, int32_t num_pages,
                              int32_t num_kv_heads, int32_t page_size, int32_t head_dim, int32_t kv_dtype,
                              int32_t direction, void* stream) {
  if (num_pages < 0 || num_kv_heads < 1 || page_size < 1 || head_dim < 1) return LBSA_ERR_INVALID;
  if (!src_k || !src_v || !dst_k || !dst_v) return LBSA_ERR_INVALID;
  if (kv_dtype != LBSA_KV_BF16 && kv_dtype != LBSA_KV_FP8_E4M3) return LBSA_ERR_INVALID;
  if (direction != 0 && direction != 1) return LBSA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(src_k) | reinterpret_cast<uintptr_t>(src_v) | reinterpret_cast<uintptr_t>(dst_k) |
       reinterpret_cast<uintptr_t>(dst_v)) & 15)
    return LBSA_ERR_INVALID;
  if (head_dim != 128 || page_size % lbsa::kSlice != 0) return LBSA_ERR_UNSUPPORTED;
  const int elem = kv_dtype == LBSA_KV_BF16 ? 2 : 1;
  // the caches must not overlap (the conversion is out of place)
  const uint64_t bytes = (uint64_t)num_pages * num_kv_heads * page_size * head_dim * elem;
  auto overlap = [bytes](const void* a, const void* b) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + bytes && y < x + bytes;
  };
  if (overlap(src_k, dst_k) || overlap(src_k, dst_v) || overlap(src_v, dst_k) || overlap(src_v, dst_v))
    return LBSA_ERR_INVALID;
  const int64_t grid = (int64_t)num_pages * num_kv_heads * (page_size / lbsa::kSlice);
  if (grid > INT32_MAX) return LBSA_ERR_INVALID;
  if (grid == 0) return LBSA_OK;
  lbsa::LayoutParams p{static_cast<const uint8_t*>(src_k), static_cast<const uint8_t*>(src_v),
                       static_cast<uint8_t*>(dst_k), static_cast<uint8_t*>(dst_v), num_kv_heads, page_size, head_dim};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 g((unsigned)grid), b(256);
  if (elem == 2) {
    if (direction == 0) hipLaunchKernelGGL((lbsa::kv_layout_kernel<2, true>), g, b, 0, st, p);
    else hipLaunchKernelGGL((lbsa::kv_layout_kernel<2, false>), g, b, 0, st, p);
  } else {
    if (direction == 0) hipLaunchKernelGGL((lbsa::kv_layout_kernel<1, true>), g, b, 0, st, p);
    else hipLaunchKernelGGL((lbsa::kv_layout_kernel<1, false>), g, b, 0, st, p);
  }
  return hipGetLastError() == hipSuccess ? LBSA_OK : LBSA_ERR_HIP;
}
