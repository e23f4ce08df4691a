// Slot-scatter KV append (pkv_write) and copy-on-write block copy
// (pkv_copy_blocks) for gfx950.
//
// Both are pure data movement on the pool layout
// [num_blocks][block_size][num_kv_heads][head_dim] ([KVM §19.2.3]).  One
// token's K (or V) row is num_kv_heads * head_dim contiguous elements, and one
// whole block is block_size such rows, also contiguous; both kernels therefore
// move contiguous 16-byte chunks with coalesced loads and stores.  Page keys
// are listed in include/pkv.h.
#include <hip/hip_runtime.h>

#include "geom.h"
#include "pkv_device.h"

namespace {

constexpr int kCopyThreads = 256;

// One workgroup per token: threads stride over the 16-byte chunks of the K row
// and then of the V row.  The slot is uniform per workgroup (scalar load).
__global__ void __launch_bounds__(kCopyThreads)
write_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v,
             const int32_t* __restrict__ slot_mapping, uint4* __restrict__ k_cache,
             uint4* __restrict__ v_cache, int32_t row_chunks, int64_t num_slots) {
  const int64_t tok = blockIdx.x;
  const int32_t slot = slot_mapping[tok];
  if (slot < 0 || slot >= num_slots) return;  // skip (negative) / out of pool
  const int64_t src = tok * row_chunks;
  const int64_t dst = int64_t(slot) * row_chunks;
  for (int32_t i = threadIdx.x; i < 2 * row_chunks; i += kCopyThreads) {
    if (i < row_chunks) {
      k_cache[dst + i] = k[src + i];
    } else {
      v_cache[dst + i - row_chunks] = v[src + i - row_chunks];
    }
  }
}

// grid = (chunk groups, pairs, 2 = K|V); each thread copies one 16-byte chunk
// of one block.
__global__ void __launch_bounds__(kCopyThreads)
copy_blocks_kernel(const int32_t* __restrict__ pairs, uint4* __restrict__ k_cache,
                   uint4* __restrict__ v_cache, int32_t block_chunks, int32_t num_blocks) {
  const int32_t src = pairs[2 * blockIdx.y];
  const int32_t dst = pairs[2 * blockIdx.y + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
  uint4* pool = blockIdx.z == 0 ? k_cache : v_cache;
  const int32_t i = blockIdx.x * kCopyThreads + threadIdx.x;
  if (i >= block_chunks) return;
  pool[int64_t(dst) * block_chunks + i] = pool[int64_t(src) * block_chunks + i];
}

}  // namespace

extern "C" {

pkv_status pkv_write(const void* k, const void* v, const int32_t* slot_mapping,
                     int32_t num_tokens, void* k_cache, void* v_cache, const pkv_geom* geom,
                     void* stream) {
  if (pkv_status st = pkv::check_geom(geom, "pkv_write")) return st;
  if (num_tokens < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "pkv_write: num_tokens < 0");
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache)
    return pkv::fail(PKV_ERR_INVALID_ARG, "pkv_write: null pointer");
  if (!pkv::aligned16(k) || !pkv::aligned16(v) || !pkv::aligned16(k_cache) ||
      !pkv::aligned16(v_cache) || (reinterpret_cast<uintptr_t>(slot_mapping) & 3u))
    return pkv::fail(PKV_ERR_INVALID_ARG, "pkv_write: misaligned pointer");
  const int32_t row_chunks =
      geom->num_kv_heads * geom->head_dim * pkv::elem_size(geom->dtype) / 16;
  const int64_t num_slots = int64_t(geom->num_blocks) * geom->block_size;
  hipLaunchKernelGGL(write_kernel, dim3(num_tokens), dim3(kCopyThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(k),
                     static_cast<const uint4*>(v), slot_mapping, static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), row_chunks, num_slots);
  if (hipError_t e = hipGetLastError())
    return pkv::fail(PKV_ERR_HIP, "pkv_write: launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

pkv_status pkv_copy_blocks(const int32_t* src_dst_pairs, int32_t num_pairs, void* k_cache,
                           void* v_cache, const pkv_geom* geom, void* stream) {
  if (pkv_status st = pkv::check_geom(geom, "pkv_copy_blocks")) return st;
  if (num_pairs < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "pkv_copy_blocks: num_pairs < 0");
  if (num_pairs == 0) return PKV_OK;
  if (num_pairs > 65535)
    return pkv::fail(PKV_ERR_INVALID_ARG, "pkv_copy_blocks: more than 65535 pairs per call");
  if (!src_dst_pairs || !k_cache || !v_cache)
    return pkv::fail(PKV_ERR_INVALID_ARG, "pkv_copy_blocks: null pointer");
  if (!pkv::aligned16(k_cache) || !pkv::aligned16(v_cache) ||
      (reinterpret_cast<uintptr_t>(src_dst_pairs) & 3u))
    return pkv::fail(PKV_ERR_INVALID_ARG, "pkv_copy_blocks: misaligned pointer");
  const int64_t block_bytes = int64_t(geom->block_size) * geom->num_kv_heads * geom->head_dim *
                              pkv::elem_size(geom->dtype);
  if (block_bytes / 16 >= (int64_t(1) << 31))
    return pkv::fail(PKV_ERR_INVALID_ARG, "pkv_copy_blocks: block too large");
  const int32_t block_chunks = static_cast<int32_t>(block_bytes / 16);
  dim3 grid((block_chunks + kCopyThreads - 1) / kCopyThreads, num_pairs, 2);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kCopyThreads), 0,
                     static_cast<hipStream_t>(stream), src_dst_pairs,
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), block_chunks,
                     geom->num_blocks);
  if (hipError_t e = hipGetLastError())
    return pkv::fail(PKV_ERR_HIP, "pkv_copy_blocks: launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

}  // extern "C"
