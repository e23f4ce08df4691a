// Decode attention on the matrix cores: the route pkv_attention_decode takes
// for groups of 8 or more query heads per KV head, where the vector kernels
// are bound by instruction issue (shared by attn_decode.hip and
// attn_multi.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv.h"

namespace pkv {

// How the matrix-core decode cuts each (sequence, KV head) history among
// workgroups: run r covers positions [r * run_tokens, (r + 1) * run_tokens)
// (run_tokens a multiple of 32) and leaves one piece, the online-softmax
// state of its positions, at piece index r.  Runs are single partitions when
// those alone fill the GPU; with more partitions than that (or whole runs of
// PKV_ATTN_PARTS_PER_WG partitions) a run folds consecutive whole partitions
// into one piece, which is what a merge of their partition pieces would
// give, up to fp32 rounding order: on the decode route about 2048 runs per
// batch, as many single-wave workgroups as are resident at once on 256 CUs
// (8 per CU: their LDS tiles), so every resident slot walks about as many
// positions in one round and no piece is stored mid-stream (a store in
// flight makes the next tile's wait wait for it as well).
struct DecodeRuns {
  int32_t run_tokens, runs;
};

// fill: the number of workgroups past which partitions are folded into runs,
// and about the number of runs then.
DecodeRuns decode_runs(int32_t num_seqs, int32_t num_kv_heads, int32_t len_cap,
                       int32_t part_tokens, int32_t num_parts, int64_t fill);

// One query row per sequence (row s of q and out, [num_seqs][num_q_heads][D]
// bf16) against its history through the block tables, with the matrix-core
// pass of pkv_attention_multi.  num_parts == 1: out is written; otherwise each
// run's (reference, sum, weighted sum) goes to ws_ml / ws_acc at row
// (s * num_q_heads + h) * runs.runs + run, for the caller's merge over the
// ceil(L_s / runs.run_tokens) runs holding positions.  part_tokens is a
// multiple of 32; runs from decode_runs() with the same sizes.  Scales: kind 0 bf16, 1 FP8 (k_scale, v_scale), 2 INT8
// (k_scales, v_scales).  stream_kv: non-temporal K/V loads (off when sequences
// share blocks).  Host checks are the caller's; this only enqueues.
pkv_status mfma_decode(const void* q, const void* k_cache, const void* v_cache, int kind,
                       float k_scale, float v_scale, const float* k_scales,
                       const float* v_scales, const int32_t* block_tables, int32_t max_blocks,
                       const int32_t* seq_lens, float scale, void* out, int32_t num_seqs,
                       int32_t num_q_heads, int32_t len_cap, int32_t part_tokens,
                       int32_t num_parts, const DecodeRuns& runs, float* ws_acc,
                       float2* ws_ml, bool stream_kv, const pkv_geom* g, hipStream_t st);

}  // namespace pkv
