// Decode attention on the matrix cores: the route pkv_attention_decode takes
// for groups of 8 or more query heads per KV head, where the vector kernels
// are bound by instruction issue (shared by attn_decode.hip and
// attn_multi.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv.h"

namespace pkv {

// One query row per sequence (row s of q and out, [num_seqs][num_q_heads][D]
// bf16) against its history through the block tables, with the matrix-core
// pass of pkv_attention_multi.  num_parts == 1: out is written; otherwise each
// partition's (reference, sum, weighted sum) goes to ws_ml / ws_acc at row
// (s * num_q_heads + h) * num_parts + part (the layout of the decode kernels'
// fixed partitions), for the caller's merge.  part_tokens is a multiple of
// 32.  Scales: kind 0 bf16, 1 FP8 (k_scale, v_scale), 2 INT8 (k_scales,
// v_scales).  stream_kv: non-temporal K/V loads (off when sequences share
// blocks).  Host checks are the caller's; this only enqueues.
pkv_status mfma_decode(const void* q, const void* k_cache, const void* v_cache, int kind,
                       float k_scale, float v_scale, const float* k_scales,
                       const float* v_scales, const int32_t* block_tables, int32_t max_blocks,
                       const int32_t* seq_lens, float scale, void* out, int32_t num_seqs,
                       int32_t num_q_heads, int32_t len_cap, int32_t part_tokens,
                       int32_t num_parts, float* ws_acc, float2* ws_ml, bool stream_kv,
                       const pkv_geom* g, hipStream_t st);

}  // namespace pkv
