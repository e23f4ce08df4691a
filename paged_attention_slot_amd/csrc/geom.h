// Host-side argument checks shared by the device entry points.
#pragma once

#include <cstdint>

#include "pkv_internal.h"

namespace pkv {

inline int elem_size(int32_t dtype) {
  switch (dtype) {
    case PKV_F32: return 4;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3:
    case PKV_INT8: return 1;
    default: return 0;
  }
}

// One-byte code pools that need scales and bf16 tokens.
inline bool is_quant(int32_t dtype) { return dtype == PKV_FP8_E4M3 || dtype == PKV_INT8; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int log2_exact(int32_t v) {
  int s = 0;
  while ((int64_t(1) << s) < v) ++s;
  return (int64_t(1) << s) == v ? s : -1;
}

// Common geometry validation: dtype known, block size a power of two, sizes
// positive, pool index space below 2^31 slots, token row a multiple of 16 B,
// one block under 2 GiB (kernels take byte offsets inside a block in 32 bits).
inline pkv_status check_geom(const pkv_geom* g, const char* who) {
  if (!g) return fail(PKV_ERR_INVALID_ARG, "%s: null geometry", who);
  if (elem_size(g->dtype) == 0) return fail(PKV_ERR_INVALID_ARG, "%s: unknown dtype %d", who, g->dtype);
  if (g->num_blocks <= 0 || g->block_size <= 0 || g->num_kv_heads <= 0 || g->head_dim <= 0)
    return fail(PKV_ERR_INVALID_ARG, "%s: non-positive geometry", who);
  if (log2_exact(g->block_size) < 0)
    return fail(PKV_ERR_INVALID_ARG, "%s: block_size %d is not a power of two", who, g->block_size);
  if (int64_t(g->num_blocks) * g->block_size >= (int64_t(1) << 31))
    return fail(PKV_ERR_INVALID_ARG, "%s: num_blocks * block_size must be < 2^31", who);
  const int64_t row = int64_t(g->num_kv_heads) * g->head_dim * elem_size(g->dtype);
  if (row % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG, "%s: token row of %lld bytes is not a multiple of 16", who,
                (long long)row);
  if (row * g->block_size >= (int64_t(1) << 31))
    return fail(PKV_ERR_INVALID_ARG, "%s: one block of %lld bytes must be under 2 GiB", who,
                (long long)(row * g->block_size));
  return PKV_OK;
}

}  // namespace pkv
