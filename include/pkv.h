/*
 * pkv.h -- C ABI of libpkv: the data-parallel hot path of PagedAttention on
 * AMD Instinct MI355X (gfx950), plus the host block manager that produces its
 * block tables and slot lists.
 *
 * Pages cited (titles as they appear on each page):
 *   [KVM]  "19.2 KV Cache 系统化管理" -- book chapter, sections 19.2.1-19.2.6,
 *          figures 19-5..19-8; section 19.2.3 holds a simplified implementation
 *          (block pool, block table, block-wise online-softmax attention).
 *   [KVX]  "KV Cache：长上下文为什么吃显存，PagedAttention 怎么救" -- explainer,
 *          numbered sections 00-07 (01: new-token attention equation;
 *          02: memory formula, GQA ratio; 03: MHA/MQA/GQA table).
 *   [SLOT] "推理与 KV Cache 02:分页、共享与回收如何协作" -- blog post; sections
 *          "从一个位置找到缓存块" (locate), "按整块分配,会多占多少空间"
 *          (whole-block), "请求结束后,缓存会立刻消失吗" (release).
 *   [PFX]  "学习大模型推理的显存优化：PagedAttention 与前缀缓存" -- blog post;
 *          sections "PagedAttention 原理" (principle), "前缀缓存" (prefix).
 *   [ENG]  the PagedAttention engineering article served under the page title
 *          "企业官网建设流程全解析"; numbered sections 1.1-8.3.
 *
 * Conventions shared by every device entry point
 * ----------------------------------------------
 *  - Cache pools: ``k_cache`` and ``v_cache`` are device buffers laid out as
 *    [num_blocks][block_size][num_kv_heads][head_dim] (row-major), the pool
 *    shape of [KVM §19.2.3].  Token slot ``s`` is row ``s`` of the pool viewed
 *    as [num_blocks * block_size][num_kv_heads][head_dim]: slot = physical
 *    block id * block_size + offset in block ([SLOT §locate], token-slot
 *    equation).
 *  - Element type: ``pkv_geom.dtype`` for the pools.  With fp32 or bf16 pools
 *    every K/V/Q/output buffer has the pool's type and no conversion is made;
 *    with the one-byte code types (FP8 e4m3, INT8) tokens, queries and
 *    outputs are bf16 and the *_quant entry points quantize and dequantize.
 *  - Ownership: the caller allocates and owns every buffer (pools, tokens,
 *    index arrays, query, output, workspace).  The library keeps no pointer
 *    after a call returns and allocates no device memory on these paths.
 *  - Streams: ``stream`` is a ``hipStream_t`` passed as ``void*`` (NULL = the
 *    null stream).  Calls only enqueue work; they never synchronise.  A device
 *    fault surfaces at the caller's next synchronisation.
 *  - Errors: every entry point returns a ``pkv_status``; on any non-OK status
 *    nothing was enqueued and ``pkv_last_error()`` (per host thread) says why.
 *    Argument checks are made on the host from sizes and pointers only; no
 *    device data is read on the host.
 *  - Index safety: kernels skip (do not dereference) slots, block ids and pairs
 *    outside the pool, so bad indices never touch memory outside the pools;
 *    the *values* produced for such entries are unspecified.
 *  - Alignment: every device pointer must be 16-byte aligned and one token row
 *    (num_kv_heads * head_dim * element size) a multiple of 16 bytes.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pkv_status;
#define PKV_OK 0
#define PKV_ERR_INVALID_ARG 1    /* bad shape, pointer, alignment or size     */
#define PKV_ERR_UNSUPPORTED 2    /* valid but not built (e.g. head_dim 96)    */
#define PKV_ERR_NO_FREE_BLOCKS 3 /* block manager: pool exhausted             */
#define PKV_ERR_HIP 4            /* the HIP runtime refused a launch          */

/* Element types.  PKV_F32 and PKV_BF16 pools hold values of the model dtype.
 * PKV_FP8_E4M3 and PKV_INT8 pools hold one-byte codes ([KVM §19.2.4] precision
 * table; [PFX] section "KV Cache 量化"): their tokens, queries and outputs are
 * bf16, and the *_quant entry points below convert. */
typedef enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2, PKV_INT8 = 3 } pkv_dtype;

/* Geometry of one cache pool pair.  block_size must be a power of two;
 * num_blocks * block_size < 2^31, and one block of a pool
 * (block_size * num_kv_heads * head_dim * element size) under 2 GiB. */
typedef struct pkv_geom {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype; /* pkv_dtype */
} pkv_geom;

/* Library version (major * 10000 + minor * 100 + patch). */
int32_t pkv_version(void);

/* Message of the last non-OK status returned on this host thread ("" if none). */
const char* pkv_last_error(void);

/* ------------------------------------------------------------------------- */
/* Device entry points                                                        */
/* ------------------------------------------------------------------------- */

/* pkv_write -- slot-scatter KV append ([KVM §19.2.3] writing one token's K and
 * V into its block slot; [KVX §01] the new token's K/V are appended to the
 * layer cache before its query reads the history).
 *   k, v          device [num_tokens][num_kv_heads][head_dim], pool dtype.
 *   slot_mapping  device int32 [num_tokens]; token i goes to slot
 *                 slot_mapping[i]; a negative slot means "skip this token".
 *   k_cache/v_cache  the pools (modified in place).
 * Bit copy: the stored bits equal the input bits.  Slots must be distinct
 * (repeated slots race: which token wins is unspecified).  num_tokens == 0 is a
 * no-op.  Errors: INVALID_ARG (null/misaligned pointer, bad geometry,
 * num_tokens < 0), HIP. */
pkv_status pkv_write(const void* k, const void* v, const int32_t* slot_mapping,
                     int32_t num_tokens, void* k_cache, void* v_cache,
                     const pkv_geom* geom, void* stream);

/* pkv_copy_blocks -- copy-on-write block copy ([KVM §19.2.2], Fig. 19-8: when a
 * block with reference count > 1 is written, a new block receives a copy of the
 * original contents; [ENG §4.2]).
 *   src_dst_pairs device int32 [num_pairs][2]; for each pair the whole dst block
 *                 (all block_size slots, K and V, stale slots included) becomes
 *                 a bit copy of the src block.
 * A dst must not repeat nor be any pair's src (those races are unspecified).
 * num_pairs == 0 is a no-op.  Errors: INVALID_ARG, HIP. */
pkv_status pkv_copy_blocks(const int32_t* src_dst_pairs, int32_t num_pairs,
                           void* k_cache, void* v_cache, const pkv_geom* geom,
                           void* stream);

/* ---- Quantized caches ([KVM §19.2.4]; [PFX] "KV Cache 量化"; [ENG §7.5]) ----
 *
 * PKV_FP8_E4M3: codes are OCP e4m3 (1 sign, 4 exponent bits with bias 7, 3
 *   mantissa bits; largest magnitude 448; S.1111.111 is NaN).  One scale per
 *   tensor: value = e4m3(code) * k_scale (or v_scale); the engine default the
 *   pages give is 1.0.  Writing encodes x / scale, computed in fp32, saturated
 *   to +-448 and rounded to the nearest code (ties to the even code).
 * PKV_INT8: per-token codes: every (token, KV head) vector of head_dim values
 *   has its own scale = max|x| / 127 and code = round(x / scale) (fp32, round
 *   half to even, clamped to +-127; an all-zero vector gets scale 0 and codes
 *   0); value = code * scale.  The scales live in fp32 pools laid out like the
 *   slots, [num_blocks * block_size][num_kv_heads].
 * Quantized pools need head_dim 128. */
typedef struct pkv_kv_scales {
  float k_scale;        /* PKV_FP8_E4M3: per-tensor scales (finite, > 0)       */
  float v_scale;
  float* k_scales;      /* PKV_INT8: device fp32 [num_blocks*block_size][H_kv] */
  float* v_scales;      /*   (ignored, may be NULL, for PKV_FP8_E4M3)          */
} pkv_kv_scales;

/* pkv_write_quant -- quantizing slot write: bf16 token rows k, v (device
 * [num_tokens][num_kv_heads][head_dim]) are encoded as above and scattered to
 * slot_mapping[i] as pkv_write does (negative slot = skip; slots must be
 * distinct); INT8 also stores each (token, head) scale at [slot][head] of the
 * scale pools.  Errors: INVALID_ARG (including a non-quantized dtype),
 * UNSUPPORTED (head_dim other than 128), HIP. */
pkv_status pkv_write_quant(const void* k, const void* v, const int32_t* slot_mapping,
                           int32_t num_tokens, void* k_cache, void* v_cache,
                           const pkv_kv_scales* scales, const pkv_geom* geom, void* stream);

/* pkv_copy_blocks_quant -- pkv_copy_blocks for quantized pools: the codes of
 * each dst block become a bit copy of the src block's, and for PKV_INT8 so do
 * the scale rows of the block (with per-token scales the copy stays a plain
 * bit copy, [ENG §7.5]).  Same pair rules and errors as pkv_copy_blocks. */
pkv_status pkv_copy_blocks_quant(const int32_t* src_dst_pairs, int32_t num_pairs,
                                 void* k_cache, void* v_cache, const pkv_kv_scales* scales,
                                 const pkv_geom* geom, void* stream);

/* ---- Shared-prefix decode attention ([KVM §19.2.5]: requests that reuse a
 * prefix point their tables at the same physical blocks; [KVX §04], [KVX §05]:
 * paging dedupes the storage, whether the reads are shared depends on the
 * kernel) --------------------------------------------------------------------
 *
 * pkv_attention_decode_shared computes exactly what pkv_attention_decode
 * computes (bf16 pools) but reads each group's shared prefix once per block of
 * 32 (member, query head) rows instead of once per sequence.  With a suffix
 * hint of at most 1024 positions one launch does the step: each block's
 * workgroup walks its members' own positions and the prefix on the matrix
 * cores and combines the states in LDS by log-sum-exp, and further workgroups
 * attend the sequences that share nothing.  Otherwise every sequence's own
 * positions go first (fp32 partial states in the workspace), then the prefix
 * positions of all members, each block's result combined with its members'
 * partial states.
 *   group_starts  device int32 [num_groups + 1]: group g is sequences
 *                 group_starts[g] .. group_starts[g+1]-1 (non-decreasing,
 *                 from 0 to num_seqs);
 *   prefix_lens   device int32 [num_groups]: tokens of the shared prefix
 *                 (rounded down to whole blocks; a group of one shares
 *                 nothing); the members' tables must hold the same blocks for
 *                 those tokens -- pkv_prefix_groups produces such groups.  A
 *                 member shorter than the prefix attends only its own tokens.
 *   max_group_size, max_prefix_len  host bounds that size the grid (a group
 *                 larger than max_group_size shares nothing).
 *   max_suffix_len  host hint: the longest run of positions after a
 *                 sequence's shared prefix (pkv_prefix_groups reports it);
 *                 it chooses the form above and sizes the suffix partitions
 *                 (0 = max_seq_len; a longer suffix is still attended in
 *                 full).
 * Other arguments as pkv_attention_decode (q, out [num_seqs][H_q][D] bf16).
 * The workspace is required (pkv_attention_shared_workspace_bytes).  Groups
 * that break the contract give unspecified values, never out-of-pool reads.
 * Errors: INVALID_ARG, UNSUPPORTED (not bf16; head_dim other than 64/128;
 * block_size < 8; more than 64 query heads per KV head), HIP. */
size_t pkv_attention_shared_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                            int32_t num_groups, int32_t max_group_size,
                                            int32_t max_prefix_len, int32_t max_suffix_len,
                                            int32_t max_seq_len, const pkv_geom* geom);
pkv_status pkv_attention_decode_shared(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* seq_lens, const int32_t* group_starts,
                                       const int32_t* prefix_lens, int32_t num_groups,
                                       int32_t max_group_size, int32_t max_prefix_len,
                                       int32_t max_suffix_len, float scale, void* out,
                                       int32_t num_seqs, int32_t num_q_heads, int32_t max_seq_len,
                                       void* workspace, size_t workspace_bytes,
                                       const pkv_geom* geom, void* stream);

/* pkv_attention_decode_shared_quant -- the same over an FP8 e4m3 or INT8 cache
 * (scales as pkv_kv_scales; head_dim 128); codes decoded exactly, scales
 * applied to scores and weights.  Workspace as for the bf16 call. */
pkv_status pkv_attention_decode_shared_quant(
    const void* q, const void* k_cache, const void* v_cache, const pkv_kv_scales* scales,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
    const int32_t* group_starts, const int32_t* prefix_lens, int32_t num_groups,
    int32_t max_group_size, int32_t max_prefix_len, int32_t max_suffix_len, float scale,
    void* out, int32_t num_seqs, int32_t num_q_heads, int32_t max_seq_len, void* workspace,
    size_t workspace_bytes, const pkv_geom* geom, void* stream);

/* pkv_prefix_groups -- groups of a batch, from its host block tables [num_seqs]
 * [max_blocks] and lengths: maximal runs of consecutive sequences whose first
 * valid entry is the same block; a group's prefix is the longest run of leading
 * entries that every member holds as valid entries (entry i valid when i <
 * ceil(L / block_size)) and that agree, in tokens; a group of one shares
 * nothing.  Outputs (host): group_starts_out [num_seqs + 1], prefix_lens_out
 * [num_seqs] (the first *num_groups_out entries are used), the largest group
 * and prefix, and the most positions any sequence has after its group's
 * prefix.  Errors: INVALID_ARG. */
pkv_status pkv_prefix_groups(const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks,
                             const int32_t* seq_lens, int32_t block_size,
                             int32_t* group_starts_out, int32_t* prefix_lens_out,
                             int32_t* num_groups_out, int32_t* max_group_size_out,
                             int32_t* max_prefix_len_out, int32_t* max_suffix_len_out);

/* ---- Block swap to host memory ([KVM §19.2.6]: a paused request's KV cache
 * moves to CPU memory and comes back when device memory frees; [KVM §19.2.2]
 * concept table, swap in/out; [ENG §8.2]: CPU memory as a second-level block
 * pool that attention never sees, because only block tables change) ----------
 *
 * The host pool mirrors the device pools' layout with its own block count:
 * K and V [num_blocks][block_size][num_kv_heads][head_dim] of the cache dtype
 * and, for PKV_INT8 caches, fp32 scale pools [num_blocks*block_size][H_kv].
 * It must be pinned host memory allocated through the HIP runtime
 * (hipHostMalloc, or a framework's pinned allocator built on it): the kernel
 * reads and writes it directly over the host link.  Pageable memory is
 * refused (INVALID_ARG).  The caller owns it. */
typedef struct pkv_host_pool {
  int32_t num_blocks;   /* host blocks (> 0; num_blocks * block_size < 2^31) */
  void* k;              /* pinned host pools, 16-byte aligned                */
  void* v;
  float* k_scales;      /* PKV_INT8 only (ignored, may be NULL, otherwise)   */
  float* v_scales;
} pkv_host_pool;

/* pkv_swap_out -- copy whole device blocks into host blocks.
 *   pairs  int32 [num_pairs][2] = (device block, host block), device memory
 *          or pinned host memory; pkv_bm_swap_out returns them.  For each
 *          pair the host block (every slot, stale ones included) becomes a
 *          bit copy of the device block: K, V and, for PKV_INT8, both scale
 *          blocks.
 *   scales device scale pools (PKV_INT8; may be NULL for other dtypes).
 * Host destinations must not repeat (a repeated destination races).  Pairs
 * with an id outside either pool are skipped.  num_pairs == 0 is a no-op.
 * The host copy is complete, for the host and for later device work, once
 * the stream has reached this point (e.g. after hipStreamSynchronize).
 * Errors: INVALID_ARG (bad pointer, memory kind, alignment or size), UNSUPPORTED
 * (PKV_INT8 with block_size * num_kv_heads not a multiple of 4), HIP. */
pkv_status pkv_swap_out(const int32_t* pairs, int32_t num_pairs, const void* k_cache,
                        const void* v_cache, const pkv_kv_scales* scales,
                        const pkv_host_pool* host, const pkv_geom* geom, void* stream);

/* pkv_swap_in -- the reverse: pairs = (host block, device block), as
 * pkv_bm_swap_in returns them; each device block becomes a bit copy of the
 * host block.  Device destinations must not repeat.  Same errors. */
pkv_status pkv_swap_in(const int32_t* pairs, int32_t num_pairs, const pkv_host_pool* host,
                       void* k_cache, void* v_cache, const pkv_kv_scales* scales,
                       const pkv_geom* geom, void* stream);

/* Split-KV partition length (tokens) that pkv_attention_decode uses when its
 * partition_tokens argument is 0 and it splits by fixed partitions: max_seq_len
 * rounded up to a whole tile (no split) when one partition per sequence is
 * enough, else a multiple of both block_size and 16 (of 32 on the matrix-core
 * route).  Returns 0 when the automatic plan is the balanced split (shares of
 * equal work per wave group, see pkv_attention_decode) or on invalid
 * arguments. */
int32_t pkv_attention_partition_tokens(int32_t num_seqs, int32_t num_q_heads,
                                       int32_t max_seq_len, const pkv_geom* geom);

/* Positions one split-KV piece of pkv_attention_decode covers for these
 * arguments (partition_tokens as passed to it, 0 = automatic): what a given
 * partition length binds on each route.  On the vector kernels with fixed
 * partitions a piece is exactly one partition (the result is the log-sum-exp
 * merge of the partitions' states).  On the matrix-core route the partition
 * length is the finest split asked for: when there are more (sequence, KV
 * head, partition) items than the GPU holds at once, one workgroup walks a
 * run of consecutive whole partitions (about 2048 runs in all) and folds it
 * into one piece (the merge of its partitions' states up to fp32 rounding
 * order), so a piece can span several partitions: for 4 histories of
 * 131,072 positions, 8 KV heads and 512-token partitions, 64 pieces of 2,048
 * positions each.  Returns the history length rounded up to a whole tile
 * when nothing is split, 0 on the balanced splits (their pieces are
 * intervals of the batch's global tile order, not of one history) or on
 * invalid arguments. */
int32_t pkv_attention_piece_tokens(int32_t num_seqs, int32_t num_q_heads, int32_t max_seq_len,
                                   int32_t partition_tokens, const pkv_geom* geom);

/* Which kernels pkv_attention_decode (and its _phase, _append and _quant
 * forms) runs for these sizes: PKV_ROUTE_PARTITIONS (vector kernels, fixed
 * partitions), PKV_ROUTE_BALANCED (vector kernels, the balanced split) or
 * PKV_ROUTE_MATRIX (head_dim 128, bf16 or one-byte pools: more than 16
 * query heads per KV head with partition_tokens 0 or a multiple of 32, or 8
 * to 16 with a given multiple of 32: the matrix-core pass of
 * pkv_attention_multi with one query per sequence, fixed partitions merged by
 * log-sum-exp) or PKV_ROUTE_MATRIX_BALANCED (2 to 16 query heads per KV head
 * at head_dim 128, bf16 or one-byte pools, partition_tokens 0: the balanced
 * split's intervals walked by one-wave workgroups on the matrix cores, the
 * group's heads as the rows of the products).  PKV_ATTN_MODE overrides.  -1
 * on invalid arguments. */
enum { PKV_ROUTE_PARTITIONS = 0, PKV_ROUTE_BALANCED = 1, PKV_ROUTE_MATRIX = 2,
       PKV_ROUTE_MATRIX_BALANCED = 3 };
int32_t pkv_attention_decode_route(int32_t num_seqs, int32_t num_q_heads, int32_t max_seq_len,
                                   int32_t partition_tokens, const pkv_geom* geom);

/* Whether pkv_attention_decode_append stores the new K/V rows from inside
 * the attention kernel (1) or launches a row-copy kernel before it (0) for
 * these sizes: the results are the same either way; this reports which
 * kernels run, for profiling.  kv_shared: nonzero when the call carries
 * PKV_KV_SHARED.  bf16 and f32 pools only; -1 on invalid arguments or a
 * one-byte pool dtype. */
int32_t pkv_attention_decode_append_folded(int32_t num_seqs, int32_t num_q_heads,
                                           int32_t max_seq_len, int32_t partition_tokens,
                                           int32_t kv_shared, const pkv_geom* geom);

/* Workspace bytes pkv_attention_decode needs for these sizes (0 when no split
 * happens).  partition_tokens as for pkv_attention_decode (0 = automatic).
 * Returns (size_t)-1 on invalid arguments. */
size_t pkv_attention_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                     int32_t max_seq_len, int32_t partition_tokens,
                                     const pkv_geom* geom);

/* pkv_attention_decode -- block-table-driven decode attention with grouped
 * query heads ([KVM §19.2.3] paged attention with block-wise online softmax,
 * Fig. 19-5; [KVX §01] new-token attention equation; [KVX §02]/[KVX §03] GQA).
 * For every sequence s and query head h (group g = h / (num_q_heads /
 * num_kv_heads)):
 *     out[s][h] = sum_{t < L_s} softmax_t(scale * q[s][h] . K_s[t]) * V_s[t]
 * with K_s[t]/V_s[t] at block block_tables[s][t / block_size], offset
 * t % block_size ([SLOT §locate]) and L_s = seq_lens[s]; L_s == 0 gives zeros.
 *   q, out        device [num_seqs][num_q_heads][head_dim], pool dtype; out is
 *                 rounded to nearest-even from fp32 for bf16.
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]; entries past
 *                 ceil(L_s / block_size) are never read.
 *   seq_lens      device int32 [num_seqs].
 *   max_seq_len   host-side upper bound of seq_lens; tokens beyond
 *                 min(max_seq_len, max_blocks_per_seq * block_size) are ignored.
 *   partition_tokens  0 = automatic, else the split-KV partition length (a
 *                 multiple of block_size and of 16).  With fixed partitions,
 *                 each partition's (max, sum, weighted sum) goes to the
 *                 workspace and a log-sum-exp merge kernel produces out.  The
 *                 automatic plan (up to 4096 sequences) is the balanced split:
 *                 a persistent grid in which every wave group takes an equal
 *                 share of 85 % of all K/V tiles of the batch, and further
 *                 workgroups, dispatched as those retire, take small chunks of
 *                 the rest; a sequence's history that spans several of these
 *                 intervals is merged the same way.  With 2 to 16 query
 *                 heads per KV head at head_dim 128 (bf16 or one-byte pools)
 *                 the intervals (of 32-position tiles) are walked on the
 *                 matrix cores, the group's heads as the rows of the
 *                 products; with one head per group, head_dim 64 or fp32
 *                 pools, on the vector units.  Groups of more than 16 query
 *                 heads per KV head, and groups of 8 to 16 with a given
 *                 partition length (a multiple of 32), run on the matrix
 *                 cores with fixed partitions (automatic: about 3072
 *                 (sequence, KV head, partition) items of at least 256
 *                 positions); see pkv_attention_decode_route.  There a
 *                 workgroup folds the positions it walks into one piece:
 *                 single partitions when they alone fill the GPU, else runs
 *                 of consecutive whole partitions (about 2048 workgroups in
 *                 all), which equals the merge of the partition pieces up to
 *                 fp32 rounding order.  So on that route partition_tokens is
 *                 the finest split asked for, not the split that runs:
 *                 pkv_attention_piece_tokens says what one piece covers.
 *   workspace     device buffer of at least pkv_attention_workspace_bytes(...)
 *                 bytes (may be NULL when that is 0); contents on entry are
 *                 ignored.  Calls that may run at the same time need
 *                 workspaces of their own.
 * Supported: head_dim 64 or 128; block_size a power of two >= 8;
 * num_q_heads a multiple of num_kv_heads with at most 64 heads per group.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP. */
pkv_status pkv_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* seq_lens, float scale, void* out,
                                int32_t num_seqs, int32_t num_q_heads, int32_t max_seq_len,
                                int32_t partition_tokens, void* workspace,
                                size_t workspace_bytes, const pkv_geom* geom, void* stream);

/* pkv_attention_decode_noalloc -- pkv_attention_decode (both phases) for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The workspace is a
 * device array inside the library of 64 MiB (PKV_NOALLOC_SCRATCH_BYTES), one
 * per GPU, held from the library's load to the end of the process; its device
 * address is looked up on the first call on each device (with that device
 * current).  The call allocates nothing (no hipMalloc, no allocating library
 * routine).  Arguments as for pkv_attention_decode without workspace and
 * workspace_bytes; bf16 and f32 pools.  Sizes whose workspace
 * (pkv_attention_workspace_bytes) exceeds the scratch are rejected with
 * PKV_ERR_INVALID_ARG before anything is enqueued.  Every call on one GPU
 * shares that GPU's scratch, which keeps the last call's contents (nothing in
 * it has to start at zero): calls that may overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP. */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
pkv_status pkv_attention_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* seq_lens, float scale, void* out,
                                        int32_t num_seqs, int32_t num_q_heads,
                                        int32_t max_seq_len, int32_t partition_tokens,
                                        const pkv_geom* geom, void* stream);

/* pkv_attention_decode_phase -- the same computation in two enqueued phases,
 * for callers that time, overlap or order them separately.  phases: 1 = the
 * per-partition kernel only (writes out directly when one partition covers
 * every sequence, else the workspace), 2 = the log-sum-exp merge only (reads
 * the workspace a previous phase-1 call with identical arguments filled;
 * nothing is enqueued when there is a single partition), 3 = both, which is
 * exactly pkv_attention_decode.  Either may be or-ed with PKV_KV_SHARED: the
 * batch's sequences share blocks (prefix sharing, forks), so the kernels read
 * K/V with cacheable loads and a block read by many sequences is served from
 * the caches; without it every K/V byte is assumed to be read once per call
 * and is streamed with non-temporal loads (faster by 8-9 % on unshared
 * batches, up to 40 % slower on shared ones) where one wave carries a KV
 * head's whole query group (groups split over several waves re-read each
 * tile and keep cacheable loads).  Same results either way.
 * Arguments and errors as for pkv_attention_decode; INVALID_ARG for any
 * other phases value. */
#define PKV_KV_SHARED 4
pkv_status pkv_attention_decode_phase(int32_t phases, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                      float scale, void* out, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t max_seq_len,
                                      int32_t partition_tokens, void* workspace,
                                      size_t workspace_bytes, const pkv_geom* geom,
                                      void* stream);

/* pkv_attention_decode_append -- the KV append and the decode attention of one
 * step ([KVX §01]: the new token's K/V join the cache before its query reads
 * the history; [KVM §19.2.3] slot write and paged attention).  The new token
 * of sequence s is its position L_s - 1 (L_s = seq_lens[s]); its K/V rows are
 * stored (bit copy) to slot slot_mapping[s] when that slot is in the pool and
 * 1 <= L_s <= min(max_seq_len, max_blocks_per_seq * block_size); otherwise
 * nothing is written for s.  With slot_mapping[s] the slot of position L_s - 1
 * (its table entry for block (L_s - 1) / block_size at offset
 * (L_s - 1) % block_size, as the block manager hands it out) the result is
 * exactly pkv_write(k_new, v_new, slot_mapping, num_seqs, ...) followed by
 * pkv_attention_decode_phase(phases, ...).  On the balanced split on the
 * matrix cores, and on the vector kernels for waves of up to two query heads,
 * the attention kernel does the append itself: the wave that attends position
 * L_s - 1 takes its K/V from the new-token rows and stores them to the slot;
 * elsewhere a copy kernel runs first.
 *   k_new, v_new  device [num_seqs][num_kv_heads][head_dim], pool dtype.
 *   slot_mapping  device int32 [num_seqs].
 *   k_cache, v_cache  modified in place at those slots only.
 * The slot's block must not be read by another sequence of the same call
 * (copy-on-write makes the block a sequence appends to its own).  phases as
 * for pkv_attention_decode_phase (the append happens in phase 1).  Pools of
 * dtype bf16 or f32; UNSUPPORTED for one-byte codes.  Other arguments and
 * errors as for pkv_attention_decode. */
pkv_status pkv_attention_decode_append(int32_t phases, const void* q, const void* k_new,
                                       const void* v_new, const int32_t* slot_mapping,
                                       void* k_cache, void* v_cache, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                       float scale, void* out, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t max_seq_len,
                                       int32_t partition_tokens, void* workspace,
                                       size_t workspace_bytes, const pkv_geom* geom,
                                       void* stream);

/* pkv_attention_decode_quant -- pkv_attention_decode_phase over a quantized
 * cache (PKV_FP8_E4M3 or PKV_INT8 pools, scales as described with
 * pkv_kv_scales): the same attention of bf16 queries over the dequantized K/V
 * values, written as bf16.  phases, workspace, partition_tokens and errors as
 * for pkv_attention_decode_phase; pkv_attention_workspace_bytes and
 * pkv_attention_partition_tokens take the quantized geometry as well. */
pkv_status pkv_attention_decode_quant(int32_t phases, const void* q, const void* k_cache,
                                      const void* v_cache, const pkv_kv_scales* scales,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* seq_lens, float scale, void* out,
                                      int32_t num_seqs, int32_t num_q_heads, int32_t max_seq_len,
                                      int32_t partition_tokens, void* workspace,
                                      size_t workspace_bytes, const pkv_geom* geom,
                                      void* stream);

/* pkv_attention_multi -- paged attention for several new query tokens per
 * sequence: a prefill chunk, or draft tokens to verify ([KVX §01] new-token
 * attention applied to each new token; [KVM §19.2.3] paged attention; GQA as
 * for pkv_attention_decode).  Sequence s owns query rows q_offsets[s] ..
 * q_offsets[s+1]-1 (n_s rows): its newest tokens, whose K/V are already in
 * the cache, so seq_lens[s] counts them.  Query j of s is at position
 * P = seq_lens[s] - n_s + j and attends positions 0..P (P < 0: zeros).
 *   q, out        device bf16 [total_q][num_q_heads][head_dim].
 *   q_offsets     device int32 [num_seqs + 1], non-decreasing, q_offsets[0] = 0
 *                 and q_offsets[num_seqs] = total_q; max_q_per_seq bounds every
 *                 n_s (rows beyond it are not computed).
 *   block_tables, seq_lens, max_seq_len, max_blocks_per_seq as for decode.
 *   partition_tokens  0 = automatic, else a multiple of 32: histories are cut
 *                 into partitions merged by log-sum-exp.
 *   workspace     pkv_attention_multi_workspace_bytes(...) bytes (NULL if 0).
 * Runs on the matrix cores (bf16 operands, fp32 accumulation; the softmax
 * weights enter the P.V product as a sum of two bf16 terms).  Supported: bf16 pools,
 * head_dim 64 or 128, at most 64 query heads per KV head.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP. */
size_t pkv_attention_multi_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                           int32_t total_q, int32_t max_q_per_seq,
                                           int32_t max_seq_len, int32_t partition_tokens,
                                           const pkv_geom* geom);
pkv_status pkv_attention_multi(const void* q, const int32_t* q_offsets, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* seq_lens, float scale,
                               void* out, int32_t num_seqs, int32_t num_q_heads, int32_t total_q,
                               int32_t max_q_per_seq, int32_t max_seq_len,
                               int32_t partition_tokens, void* workspace,
                               size_t workspace_bytes, const pkv_geom* geom, void* stream);

/* pkv_attention_multi_quant -- pkv_attention_multi over an FP8 e4m3 or INT8
 * cache (scales as described with pkv_kv_scales; head_dim 128): the codes are
 * decoded exactly when tiles are staged and the scales applied to the scores
 * (K) and weights (V), so the result is the attention over the dequantized
 * values; q and out stay bf16.  Workspace: pkv_attention_multi_workspace_bytes
 * with the quantized geometry.  Errors as pkv_attention_multi, INVALID_ARG
 * for a non-quantized dtype or missing scales. */
pkv_status pkv_attention_multi_quant(const void* q, const int32_t* q_offsets, const void* k_cache,
                                     const void* v_cache, const pkv_kv_scales* scales,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* seq_lens, float scale, void* out,
                                     int32_t num_seqs, int32_t num_q_heads, int32_t total_q,
                                     int32_t max_q_per_seq, int32_t max_seq_len,
                                     int32_t partition_tokens, void* workspace,
                                     size_t workspace_bytes, const pkv_geom* geom, void* stream);

/* Tuning knobs of the attention entry points.  Each starts from the
 * environment variable of its name, read once per process at the first use
 * of any knob (unset or out of range = 0, the library's heuristic); later
 * changes to the environment have no effect.  pkv_set_tuning sets a knob
 * (0 = back to the heuristic; INVALID_ARG for an unknown name or a value out
 * of range); pkv_get_tuning returns its current value, -1 for an unknown
 * name.  Knobs are process-wide: a change applies to calls enqueued after it.
 * Names and ranges:
 *   PKV_ATTN_HEADS_PER_WAVE  1..4  upper bound on query heads one wave carries
 *   PKV_ATTN_PREFETCH        2..4  K/V tiles of 16 positions in flight per wave
 *                                  (bf16: at most 4 / 3 / 2 for 1 / 2 / 3-4
 *                                  heads per wave; one-byte codes: up to 4;
 *                                  fp32 always uses 2)
 *   PKV_ATTN_WAVES_PER_BLOCK 1,2,4,8  fixed partitions: waves per workgroup
 *                                  (the waves of one (sequence, partition)
 *                                  are packed together)
 *   PKV_ATTN_MODE            1 = fixed partitions, 2 = balanced split,
 *                                  3 = the matrix-core route where it applies,
 *                                  4 = the balanced split on the matrix cores
 *                                  where it applies (head_dim 128, bf16 or
 *                                  one-byte pools, up to 16 heads per group)
 *   PKV_ATTN_PARTS_PER_WG    1..65535  matrix-core passes: consecutive
 *                                  partitions one workgroup walks (the decode
 *                                  route folds them into one piece, instead
 *                                  of its automatic runs)
 *   PKV_ATTN_APPEND          pkv_attention_decode_append: 1 = copy kernel
 *                                  first, 2 = folded into the attention kernel
 *                                  (vector routes with non-temporal loads only)
 * They change speed and register use, never results beyond fp32 rounding
 * order across query-head groupings (each head's arithmetic is unchanged). */
pkv_status pkv_set_tuning(const char* name, int32_t value);
int32_t pkv_get_tuning(const char* name);

/* pkv_stream_read -- calibration, not part of the method: reads ``bytes``
 * (a multiple of 16) from device buffer ``src`` with a coalesced
 * 16-byte-per-lane stream of non-temporal loads (as the attention kernels
 * read K/V) by ``num_workgroups`` x 256 threads, the practical read-bandwidth
 * ceiling that the attention kernel is compared with.  ``sink``
 * is a device buffer of num_workgroups uint32 that is only written if the data
 * hashes to one specific value.  Errors: INVALID_ARG, HIP. */
pkv_status pkv_stream_read(const void* src, size_t bytes, void* sink, int32_t num_workgroups,
                           void* stream);

/* ------------------------------------------------------------------------- */
/* Host block manager (host memory only; one handle must not be used from two */
/* threads at once).                                                          */
/* ------------------------------------------------------------------------- */

/* Pool of num_blocks blocks of block_size slots ([KVM §19.2.2], [KVM §19.2.3]).
 * free_order (host int32 [num_blocks], a permutation of 0..num_blocks-1, or
 * NULL for 0..num_blocks-1) is the initial free list; blocks are taken from its
 * end and returned to its end (most recently freed first, [ENG §3.2]).
 * Returns NULL on invalid arguments. */
typedef struct pkv_bm pkv_bm;
pkv_bm* pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order);
void pkv_bm_destroy(pkv_bm* bm);

/* New empty sequence: an empty block table of its own ([KVM §19.2.2] block
 * partitioning: every request has an independent block table; [ENG §5.1]
 * one table row per sequence, grown as the sequence grows).  INVALID_ARG if
 * the id exists. */
pkv_status pkv_bm_add_seq(pkv_bm* bm, int64_t seq);

/* Empty sequence dst takes src's first num_tokens tokens by reference: the
 * blocks holding them get one more reference each ([KVM §19.2.5], [PFX
 * §prefix]).  INVALID_ARG if dst is not empty or src is shorter. */
pkv_status pkv_bm_share_prefix(pkv_bm* bm, int64_t dst, int64_t src, int32_t num_tokens);

/* New sequence child as a copy of parent: same table and length, one more
 * reference on every block ([ENG §5.1], [KVM §19.2.2] parallel sampling). */
pkv_status pkv_bm_fork(pkv_bm* bm, int64_t parent, int64_t child);

/* Append tokens_each tokens to each of the n sequences seqs[0..n) in order
 * (sequence-major).  For each token: logical block = filled / block_size,
 * offset = filled % block_size ([SLOT §locate]); a new block is allocated when
 * the logical block does not exist yet ([KVM §19.2.2] step 2); if it exists but
 * is shared (reference count > 1) it is replaced by a fresh block and the pair
 * (old, new) is emitted for pkv_copy_blocks while the old block loses one
 * reference ([KVM §19.2.2], Fig. 19-8).  slots_out (host int32
 * [n * tokens_each]) receives slot = block * block_size + offset.
 * cow_pairs_out (host int32 [n][2], at most one pair per sequence per call) and
 * *num_cow_out receive the copy pairs in order; cow_pairs_out may be NULL only
 * if no copy is needed.  All-or-nothing: on NO_FREE_BLOCKS (or any error) the
 * manager is left exactly as before ([KVM §19.2.6]; [ENG §3.2]). */
pkv_status pkv_bm_append_slots(pkv_bm* bm, const int64_t* seqs, int32_t n,
                               int32_t tokens_each, int32_t* slots_out,
                               int32_t* cow_pairs_out, int32_t* num_cow_out);

/* Release every block of the sequence, the partly filled last one included
 * ([KVM §19.2.3]; [ENG §7.1]); blocks reaching zero references go back to the
 * free list, their data untouched ([ENG §3.2]). */
pkv_status pkv_bm_free_seq(pkv_bm* bm, int64_t seq);

/* Block tables of seqs[0..n) as host int32 [n][max_blocks] padded with -1, and
 * their token counts (host int32 [n]): the batched form the kernel takes
 * ([ENG §5.1] a two-dimensional array, sequence by logical block, one int
 * block id per entry ([ENG §2.1]); [ENG §5.2] the kernel receives the table
 * pointer).  INVALID_ARG if a table is longer than max_blocks or a sequence is
 * unknown. */
pkv_status pkv_bm_export(const pkv_bm* bm, const int64_t* seqs, int32_t n, int32_t max_blocks,
                         int32_t* block_tables_out, int32_t* seq_lens_out);

/* Blocks on the free list ([ENG §3.2]: every physical block is either named
 * by a logical block or on the free list). */
int32_t pkv_bm_num_free(const pkv_bm* bm);
/* Reference count of a block: the number of table entries naming it ([KVM
 * §19.2.2] copy-on-write: a shared block keeps a reference count; [ENG §4.2]);
 * -1 if out of range. */
int32_t pkv_bm_refcount(const pkv_bm* bm, int32_t block);
/* Tokens in a sequence: its write position ([ENG §2.1] the per-sequence
 * offset kept apart from the table); -1 if unknown. */
int32_t pkv_bm_num_tokens(const pkv_bm* bm, int64_t seq);
/* Copy the free list (bottom to top; blocks are taken from and returned to
 * the top, [KVM §19.2.3]) into out[0..cap); *n_out = its length. */
pkv_status pkv_bm_free_list(const pkv_bm* bm, int32_t* out, int32_t cap, int32_t* n_out);
/* ---- Preemption by swap ([KVM §19.2.6]; [ENG §8.2]) --------------------------
 * A manager may hold a second pool of host blocks with its own free list
 * (taken from and returned to its end) and reference counts.  Preempting a
 * sequence by recomputation is pkv_bm_free_seq; preempting it by swap is
 * pkv_bm_swap_out followed by pkv_swap_out on the returned pairs, and resuming
 * it is pkv_bm_swap_in followed by pkv_swap_in.  A swapped-out sequence's
 * table names host blocks; append, fork, share_prefix (either side) and
 * export refuse it (INVALID_ARG) until it is swapped back in; free_seq
 * releases its host blocks. */

/* Give the manager its host pool of num_host_blocks blocks (once per manager).
 * free_order: host int32 permutation of 0..num_host_blocks-1, or NULL. */
pkv_status pkv_bm_add_host_pool(pkv_bm* bm, int32_t num_host_blocks, const int32_t* free_order);

/* Pause the n distinct resident sequences seqs[0..n) together.  Every distinct
 * device block their tables name gets one host block (a block shared between
 * them moves once and stays shared); table entries are remapped, table by
 * table in order, and each releases its device reference, so blocks no longer
 * referenced return to the device free list ([KVM §19.2.6]: all of the
 * request's blocks at once).  pairs_out (host int32 [cap][2]) receives the
 * (device block, host block) pairs in order of first appearance and
 * *num_pairs_out their count; pkv_bm_distinct_blocks gives the capacity
 * needed.  All-or-nothing: NO_FREE_BLOCKS if the host pool has too few free
 * blocks, INVALID_ARG (unknown, repeated or already swapped sequence, small
 * capacity); the manager is unchanged on any error. */
pkv_status pkv_bm_swap_out(pkv_bm* bm, const int64_t* seqs, int32_t n, int32_t* pairs_out,
                           int32_t cap, int32_t* num_pairs_out);

/* Resume swapped-out sequences: the reverse, with fresh device blocks from the
 * device free list and (host block, device block) pairs.  NO_FREE_BLOCKS if
 * the device pool has too few free blocks; all-or-nothing as above. */
pkv_status pkv_bm_swap_in(pkv_bm* bm, const int64_t* seqs, int32_t n, int32_t* pairs_out,
                          int32_t cap, int32_t* num_pairs_out);

/* Number of distinct blocks the sequences' tables name (each on its own tier):
 * the pair count a swap of exactly these sequences produces, and the free
 * blocks it needs.  -1 on an unknown sequence or bad argument. */
int32_t pkv_bm_distinct_blocks(const pkv_bm* bm, const int64_t* seqs, int32_t n);
/* 1 if swapped out, 0 if resident, -1 if unknown. */
int32_t pkv_bm_is_swapped(const pkv_bm* bm, int64_t seq);
int32_t pkv_bm_num_free_host(const pkv_bm* bm);
/* Reference count of a host block (-1 if out of range). */
int32_t pkv_bm_host_refcount(const pkv_bm* bm, int32_t block);
/* Copy the host free list (bottom to top) into out[0..cap); *n_out = its length. */
pkv_status pkv_bm_host_free_list(const pkv_bm* bm, int32_t* out, int32_t cap, int32_t* n_out);

/* Invariants ([ENG §7.1], [ENG §7.2]), for the device pool and the host pool
 * alike: free list without duplicates; free and referenced blocks partition
 * the pool; every reference count equals the number of table entries naming
 * that block (resident tables for the device pool, swapped-out tables for the
 * host pool); every table holds ceil(tokens / block_size) blocks.  INVALID_ARG (with a message) on violation. */
pkv_status pkv_bm_check(const pkv_bm* bm);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
