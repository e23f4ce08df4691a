// Slot-scatter KV append (pkv_write, pkv_write_quant) and copy-on-write block
// copy (pkv_copy_blocks, pkv_copy_blocks_quant) for gfx950.
//
// Both are pure data movement on the pool layout
// [num_blocks][block_size][num_kv_heads][head_dim] ([KVM §19.2.3]).  One
// token's K (or V) row is num_kv_heads * head_dim contiguous elements, and one
// whole block is block_size such rows, also contiguous; both kernels therefore
// move contiguous 16-byte chunks with coalesced loads and stores.  Page keys
// are listed in include/pkv.h.
#include <hip/hip_runtime.h>

#include <cmath>

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

// bf16 -> OCP e4m3 code: |x| saturated to 448, rounded to the nearest code,
// ties to the even code; the sign bit is kept (a negative value that rounds to
// zero gives 0x80); NaN -> 0x7F.  Normal results keep 3 of the 23 fp32
// mantissa bits (round half to even on the 20 dropped); below 2^-6 the code is
// the subnormal step count round(|x| * 2^9) (0..8; 8 is the smallest normal).
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  if (x != x) return 0x7Fu;
  const float a = fminf(fabsf(x), 448.0f);
  const uint32_t u = __float_as_uint(a);
  const int e = static_cast<int>(u >> 23) - 127;
  if (e >= -6) {
    uint32_t keep = (u >> 20) & 7u;
    const uint32_t rest = u & 0xFFFFFu;
    if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
    uint32_t be = static_cast<uint32_t>(e + 7);
    if (keep == 8u) {
      keep = 0;
      ++be;
    }
    return sign | (be << 3) | keep;
  }
  return sign | static_cast<uint32_t>(rintf(a * 512.0f));
}

// Per-vector INT8 code of x with scale s > 0: round half to even, clamp +-127.
__device__ __forceinline__ uint32_t int8_encode(float x, float s) {
  const float q = fminf(fmaxf(rintf(x / s), -127.0f), 127.0f);
  return static_cast<uint32_t>(static_cast<int32_t>(q)) & 0xFFu;
}

// One wave per (token, KV head) (grid x = tokens, y = heads): lane i quantizes elements 2i, 2i+1 of the
// head_dim = 128 row (one bf16 pair in, one pair of codes out), first K then
// V.  INT8 scales: max |x| over the row (whole-wave reduction) / 127, written
// by lane 0 at [slot][head].
template <bool kInt8>
__global__ void __launch_bounds__(64)
write_quant_kernel(const uint32_t* __restrict__ k, const uint32_t* __restrict__ v,
                   const int32_t* __restrict__ slot_mapping, uint16_t* __restrict__ k_cache,
                   uint16_t* __restrict__ v_cache, float* __restrict__ k_scales,
                   float* __restrict__ v_scales, float k_scale, float v_scale, int32_t num_heads,
                   int64_t num_slots) {
  const int64_t tok = blockIdx.x;
  const int h = blockIdx.y;
  const int32_t slot = slot_mapping[tok];
  if (slot < 0 || slot >= num_slots) return;  // skip (negative) / out of pool
  const int lane = threadIdx.x;
  const int64_t row = tok * num_heads + h, drow = int64_t(slot) * num_heads + h;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t x = (w == 0 ? k : v)[row * 64 + lane];
    const float a = pkv::bf16lo(x), b = pkv::bf16hi(x);
    uint32_t ca, cb;
    if constexpr (kInt8) {
      const float amax = pkv::wave_max(fmaxf(fabsf(a), fabsf(b)));
      const float s = amax / 127.0f;
      ca = s > 0.0f ? int8_encode(a, s) : 0u;
      cb = s > 0.0f ? int8_encode(b, s) : 0u;
      if (lane == 0) (w == 0 ? k_scales : v_scales)[drow] = s;
    } else {
      const float sc = w == 0 ? k_scale : v_scale;
      ca = e4m3_encode(a / sc);
      cb = e4m3_encode(b / sc);
    }
    (w == 0 ? k_cache : v_cache)[drow * 64 + lane] = static_cast<uint16_t>(ca | (cb << 8));
  }
}

pkv_status launch_copy(const char* who, const int32_t* pairs, int32_t num_pairs, void* k_pool,
                       void* v_pool, int64_t block_bytes, int32_t num_blocks, void* stream) {
  if (block_bytes / 16 >= (int64_t(1) << 31))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: block too large", who);
  const int32_t block_chunks = static_cast<int32_t>(block_bytes / 16);
  dim3 grid((block_chunks + kCopyThreads - 1) / kCopyThreads, num_pairs, 2);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kCopyThreads), 0,
                     static_cast<hipStream_t>(stream), pairs, static_cast<uint4*>(k_pool),
                     static_cast<uint4*>(v_pool), block_chunks, num_blocks);
  if (hipError_t e = hipGetLastError())
    return pkv::fail(PKV_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return PKV_OK;
}

// Checks shared by the two copy entry points.
pkv_status check_copy(const char* who, const int32_t* pairs, int32_t num_pairs, void* k_cache,
                      void* v_cache, const pkv_geom* geom) {
  if (pkv_status st = pkv::check_geom(geom, who)) return st;
  if (num_pairs < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: num_pairs < 0", who);
  if (num_pairs > 65535)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: more than 65535 pairs per call", who);
  if (num_pairs > 0 && (!pairs || !k_cache || !v_cache))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: null pointer", who);
  if (num_pairs > 0 && (!pkv::aligned16(k_cache) || !pkv::aligned16(v_cache) ||
                        (reinterpret_cast<uintptr_t>(pairs) & 3u)))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: misaligned pointer", who);
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_write(const void* k, const void* v, const int32_t* slot_mapping,
                     int32_t num_tokens, void* k_cache, void* v_cache, const pkv_geom* geom,
                     void* stream) {
  if (pkv_status st = pkv::check_geom(geom, "pkv_write")) return st;
  if (geom->dtype == PKV_INT8)
    return pkv::fail(PKV_ERR_INVALID_ARG, "pkv_write: INT8 pools need scales (pkv_write_quant)");
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
  const char* who = "pkv_copy_blocks";
  if (pkv_status st = check_copy(who, src_dst_pairs, num_pairs, k_cache, v_cache, geom)) return st;
  if (geom->dtype == PKV_INT8)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: INT8 pools need scales (pkv_copy_blocks_quant)",
                     who);
  if (num_pairs == 0) return PKV_OK;
  const int64_t block_bytes = int64_t(geom->block_size) * geom->num_kv_heads * geom->head_dim *
                              pkv::elem_size(geom->dtype);
  return launch_copy(who, src_dst_pairs, num_pairs, k_cache, v_cache, block_bytes,
                     geom->num_blocks, stream);
}

pkv_status pkv_write_quant(const void* k, const void* v, const int32_t* slot_mapping,
                           int32_t num_tokens, void* k_cache, void* v_cache,
                           const pkv_kv_scales* scales, const pkv_geom* geom, void* stream) {
  const char* who = "pkv_write_quant";
  if (pkv_status st = pkv::check_geom(geom, who)) return st;
  if (!pkv::is_quant(geom->dtype))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: dtype %d is not a quantized cache type", who,
                     geom->dtype);
  if (geom->head_dim != 128)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "%s: head_dim %d (quantized caches: 128)", who,
                     geom->head_dim);
  if (!scales) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: null scales", who);
  const bool i8 = geom->dtype == PKV_INT8;
  if (!i8 && !(std::isfinite(scales->k_scale) && scales->k_scale > 0.0f &&
               std::isfinite(scales->v_scale) && scales->v_scale > 0.0f))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: FP8 scales must be finite and > 0", who);
  if (num_tokens < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: num_tokens < 0", who);
  if (num_tokens == 0) return PKV_OK;
  if (geom->num_kv_heads > 65535)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: more than 65535 KV heads", who);
  if (!k || !v || !slot_mapping || !k_cache || !v_cache || (i8 && (!scales->k_scales || !scales->v_scales)))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!pkv::aligned16(k) || !pkv::aligned16(v) || !pkv::aligned16(k_cache) ||
      !pkv::aligned16(v_cache) || (reinterpret_cast<uintptr_t>(slot_mapping) & 3u) ||
      (i8 && ((reinterpret_cast<uintptr_t>(scales->k_scales) & 3u) ||
              (reinterpret_cast<uintptr_t>(scales->v_scales) & 3u))))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: misaligned pointer", who);
  const int64_t num_slots = int64_t(geom->num_blocks) * geom->block_size;
  const dim3 grid(num_tokens, geom->num_kv_heads);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  auto kk = static_cast<const uint32_t*>(k);
  auto vv = static_cast<const uint32_t*>(v);
  auto kc = static_cast<uint16_t*>(k_cache);
  auto vc = static_cast<uint16_t*>(v_cache);
  if (i8)
    hipLaunchKernelGGL(write_quant_kernel<true>, grid, dim3(64), 0, st, kk, vv, slot_mapping, kc,
                       vc, scales->k_scales, scales->v_scales, 1.0f, 1.0f, geom->num_kv_heads,
                       num_slots);
  else
    hipLaunchKernelGGL(write_quant_kernel<false>, grid, dim3(64), 0, st, kk, vv, slot_mapping, kc,
                       vc, nullptr, nullptr, scales->k_scale, scales->v_scale,
                       geom->num_kv_heads, num_slots);
  if (hipError_t e = hipGetLastError())
    return pkv::fail(PKV_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return PKV_OK;
}

pkv_status pkv_copy_blocks_quant(const int32_t* src_dst_pairs, int32_t num_pairs, void* k_cache,
                                 void* v_cache, const pkv_kv_scales* scales,
                                 const pkv_geom* geom, void* stream) {
  const char* who = "pkv_copy_blocks_quant";
  if (pkv_status st = check_copy(who, src_dst_pairs, num_pairs, k_cache, v_cache, geom)) return st;
  if (!pkv::is_quant(geom->dtype))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: dtype %d is not a quantized cache type", who,
                     geom->dtype);
  const bool i8 = geom->dtype == PKV_INT8;
  const int64_t scale_block_bytes = int64_t(geom->block_size) * geom->num_kv_heads * 4;
  if (i8) {
    if (!scales || !scales->k_scales || !scales->v_scales)
      return pkv::fail(PKV_ERR_INVALID_ARG, "%s: null scales", who);
    if (!pkv::aligned16(scales->k_scales) || !pkv::aligned16(scales->v_scales))
      return pkv::fail(PKV_ERR_INVALID_ARG, "%s: misaligned scale pools", who);
    if (scale_block_bytes % 16 != 0)
      return pkv::fail(PKV_ERR_UNSUPPORTED,
                       "%s: block_size * num_kv_heads must be a multiple of 4", who);
  }
  if (num_pairs == 0) return PKV_OK;
  const int64_t block_bytes = int64_t(geom->block_size) * geom->num_kv_heads * geom->head_dim;
  if (pkv_status st = launch_copy(who, src_dst_pairs, num_pairs, k_cache, v_cache, block_bytes,
                                  geom->num_blocks, stream))
    return st;
  if (i8)
    return launch_copy(who, src_dst_pairs, num_pairs, scales->k_scales, scales->v_scales,
                       scale_block_bytes, geom->num_blocks, stream);
  return PKV_OK;
}

}  // extern "C"
