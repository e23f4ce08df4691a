// Paged attention for several new query tokens per sequence (a prefill chunk,
// or draft tokens to verify) on the gfx950 matrix cores: pkv_attention_multi.
//
// What is computed ([KVX §01] new-token attention, applied to each new token;
// [KVM §19.2.3] paged attention; [KVX §02]/[KVX §03] grouped-query heads; page
// keys in include/pkv.h): sequence s owns query rows q_offsets[s] ..
// q_offsets[s+1]-1, its n_s newest tokens, already written to the cache, so
// L_s counts them.  Query j sits at position P = L_s - n_s + j and attends
// positions 0..P:
//     out[row][h] = sum_{t <= P} softmax_t(scale * q[row][h] . K_s[t]) V_s[t].
//
// How (MI355X design): one workgroup per (block of query tokens, partition
// of positions, KV head, sequence).  Its rows are (query token, query head of
// the group) pairs, 16 per wave, so each K/V byte read serves every head of
// the group and every query token of the block; the pass itself (LDS-staged
// tiles, scores and P V on the matrix cores, online softmax) is
// pkv::mfma::attend.  Positions past a row's own (the causal rule) are
// masked.  Long histories with few query blocks are split into partitions
// merged by log-sum-exp (attn_multi_merge_kernel).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>

#include "geom.h"
#include "lse_merge.h"
#include "mfma_attend.h"
#include "mfma_route.h"
#include "pkv_device.h"

namespace {

using pkv::mfma::kKT;

struct MultiArgs {
  const uint16_t* q;
  const int32_t* q_offsets;  // null: one query per sequence, row s (decode)
  const void* k_cache;      // bf16 bits or one-byte codes
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  uint16_t* out;
  float* ws_acc;    // [row * H_q + h][part][D]
  float2* ws_ml;    // [row * H_q + h][part] (reference, sum)
  int32_t* ws_np;   // [row * H_q + h]: partitions holding positions <= P (or null)
  int64_t block_elems;
  int32_t row_elems;
  int32_t max_blocks;
  int32_t num_q_heads;
  int32_t total_q;
  int32_t group;
  int32_t num_blocks;
  int32_t block_shift;
  int32_t len_cap;
  int32_t q_per_block;
  int32_t num_qblocks;
  int32_t num_kv_heads;
  int32_t num_sg;           // (sequence, KV head) pairs (set at launch)
  int32_t num_parts;
  int32_t part_tokens;
  int32_t run_tokens;       // positions one workgroup walks (a multiple of 32)
  int32_t piece_tokens;     // a piece ends at each multiple of this (and at t_hi)
  int32_t piece_stride;     // workspace rows per (row, head)
  float scale_log2;         // FP8: the K tensor scale folded in
  float v_scale;            // FP8
  const float* k_scales;    // INT8
  const float* v_scales;
};

// RG row groups of 16 per wave (16 NW RG rows per workgroup).  Register
// budgets that keep workgroups resident: eight-wave ones two per CU (<= 128
// registers a lane), four-wave ones three, or two with two row groups a wave
// (the 128-row instance).
template <int D, int NW, int Q, bool kStream, int RG = 1>
__global__ void __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(NW == 8 ? 4 : (NW == 4 ? (RG == 2 ? 2 : 3) : 1))))
attn_multi_kernel(MultiArgs a) {
  __shared__ __align__(16) uint16_t k_lds[pkv::mfma::k_lds_elems<D, NW, Q, RG>()];
  __shared__ __align__(16) uint16_t v_lds[pkv::mfma::v_lds_elems<D, NW, Q, RG>()];
  __shared__ float s_lds[pkv::mfma::s_lds_elems<Q, NW>()];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(tid >> 6));
  // grid = (query blocks * (sequence, KV head) pairs, runs of run_tokens
  // positions).  Workgroups go to the XCDs round robin in launch order.
  // One query block per pair (decode): rotating the item by the run (item =
  // x + run) spreads both every run over all XCDs and the runs of one item
  // (one long history) over different XCDs; run-fastest order put all of
  // run p on one XCD whenever the run count divides 8.  Several query blocks
  // (prefill chunks) all read their pair's history: they go to one XCD, in
  // consecutive dispatch slots there, so that XCD's L2 fetches the history
  // once for all of them (x = 8 k + c: XCD c, slot k; gridDim.x is a
  // multiple of 8, padded with idle workgroups).
  const int qbs = a.num_qblocks;
  const int run = blockIdx.y;
  int item;
  if (qbs == 1) {
    item = static_cast<int>((blockIdx.x + uint32_t(run)) % uint32_t(a.num_sg));
  } else {
    const int c = static_cast<int>(blockIdx.x & 7u), k = static_cast<int>(blockIdx.x >> 3);
    const int sg = 8 * (k / qbs) + c;
    if (sg >= a.num_sg) return;  // padding
    item = sg * qbs + k % qbs;
  }
  const int qb = item % qbs;
  const int g = (item / qbs) % a.num_kv_heads;
  const int s = item / (qbs * a.num_kv_heads);
  const int q0 = a.q_offsets ? a.q_offsets[s] : s;
  const int n = a.q_offsets ? a.q_offsets[s + 1] - q0 : 1;
  const int j0 = qb * a.q_per_block;
  if (q0 < 0 || j0 >= n) return;  // uniform over the workgroup
  const int jn = min(a.q_per_block, n - j0);
  const int Lraw = a.seq_lens[s];
  const int L = Lraw < 0 ? 0 : (Lraw > a.len_cap ? a.len_cap : Lraw);
  const int p_first = L - n + j0;          // position of the block's first query
  const int p_last = p_first + jn - 1;
  const int t_lo = run * a.run_tokens;
  const int t_hi = min(min(t_lo + a.run_tokens, a.num_parts * a.part_tokens), p_last + 1);
  if (run > 0 && t_lo >= t_hi) return;     // no row of this block reaches these parts

  // This lane's rows, one per row group: (query token jl of the block, head
  // hh of the group).
  const int G = a.group;
  bool row_ok[RG];
  int p_row[RG];
  int64_t qh[RG];  // (row, head) index
  const uint16_t* qrow[RG];
#pragma unroll
  for (int gi = 0; gi < RG; ++gi) {
    const int row = 16 * (RG * w + gi) + (lane & 15);
    const int jl = row / G, hh = row - jl * G;
    row_ok[gi] = jl < jn && q0 + j0 + jl < a.total_q;  // rows outside q: never touched
    p_row[gi] = p_first + jl;
    qh[gi] = int64_t(q0 + j0 + jl) * a.num_q_heads + g * G + hh;
    qrow[gi] = a.q + qh[gi] * D;
  }

  const pkv::mfma::History hist{a.k_cache,    a.v_cache,      a.block_tables + int64_t(s) * a.max_blocks,
                                L,            g,              a.block_elems,
                                a.row_elems,  a.num_blocks,   a.block_shift,
                                a.num_kv_heads, a.v_scale,    a.k_scales,
                                a.v_scales};
  pkv::mfma::RowAcc<D> r[RG];
#pragma unroll
  for (int gi = 0; gi < RG; ++gi) pkv::mfma::start(r[gi]);
  constexpr int kPD = NW >= 2 ? 2 : 1;
  if (a.piece_stride == 1) {
    // one run covers the history: every row of the block sees the positions
    // up to its first query's
    pkv::mfma::attend_rows<D, NW, kPD, Q, kStream, pkv::mfma::NoEmit, false, false, RG>(
        hist, t_lo, t_hi, qrow, row_ok, p_row, p_first, a.scale_log2, k_lds, v_lds, r, s_lds);
#pragma unroll
    for (int gi = 0; gi < RG; ++gi)
      if (row_ok[gi]) pkv::mfma::store_row_bf16<D>(r[gi], a.out + qh[gi] * D);
    return;
  }
  // one piece per piece_tokens positions (a partition, or the whole run on
  // the decode route), at [row, head][piece]; t_lo is a multiple of
  // piece_tokens
  const auto emit = [&](int t, pkv::mfma::RowAcc<D>& rr, int gi) {
    if (!row_ok[gi]) return;
    const int64_t prow = qh[gi] * a.piece_stride + t / a.piece_tokens;
    pkv::mfma::store_piece<D>(rr, a.ws_acc + prow * D, a.ws_ml + prow);
  };
  pkv::mfma::attend_rows<D, NW, kPD, Q, kStream, decltype(emit), false, false, RG>(
      hist, t_lo, t_hi, qrow, row_ok, p_row, p_first, a.scale_log2, k_lds, v_lds, r, s_lds,
      a.piece_tokens, emit);
#pragma unroll
  for (int gi = 0; gi < RG; ++gi)
    if (row_ok[gi] && a.ws_np && (lane >> 4) == 0 && run == 0) {
      const int np = p_row[gi] < 0 ? 0 : min(a.piece_stride, p_row[gi] / a.piece_tokens + 1);
      a.ws_np[qh[gi]] = np;
    }
}

// Log-sum-exp merge of the partitions of one (query row, head): one wave,
// each lane owns D/64 output elements.
template <int D>
__global__ void __launch_bounds__(64)
attn_multi_merge_kernel(MultiArgs a) {
  constexpr int kE = D / 64;
  const int64_t qh = int64_t(blockIdx.y) * a.num_q_heads + blockIdx.x;
  const int lane = threadIdx.x;
  const int np_raw = a.ws_np[qh];
  const int np = np_raw < 0 ? 0 : (np_raw > a.piece_stride ? a.piece_stride : np_raw);
  const int64_t base = qh * a.piece_stride;
  float M = -INFINITY;
  for (int p = lane; p < np; p += 64) M = fmaxf(M, a.ws_ml[base + p].x);
  M = pkv::wave_max(M);
  float lsum = 0.f, acc[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) acc[e] = 0.f;
  for (int p = 0; p < np; ++p) {
    const float2 ml = a.ws_ml[base + p];
    const float wgt = pkv::fast_exp2(ml.x - M);
    lsum = fmaf(wgt, ml.y, lsum);
    const float* src = a.ws_acc + (base + p) * D;
#pragma unroll
    for (int e = 0; e < kE; ++e) acc[e] = fmaf(wgt, src[lane * kE + e], acc[e]);
  }
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  uint16_t* dst = a.out + qh * D + lane * kE;
#pragma unroll
  for (int e = 0; e < kE; ++e) dst[e] = static_cast<uint16_t>(pkv::f32_to_bf16_bits(acc[e] * inv));
}

// The same merge for many partitions: one 256-thread workgroup per (query
// row, head), 64 pieces per memory round trip (pkv::merge_rows).
template <int D>
__global__ void __launch_bounds__(pkv::kMergeThreads)
attn_multi_merge_wide_kernel(MultiArgs a) {
  const int64_t qh = int64_t(blockIdx.y) * a.num_q_heads + blockIdx.x;
  const int np_raw = a.ws_np[qh];
  const int np = np_raw < 0 ? 0 : (np_raw > a.piece_stride ? a.piece_stride : np_raw);
  pkv::merge_rows<uint16_t, D>(a.ws_acc, a.ws_ml, np, qh * a.piece_stride, 1,
                               reinterpret_cast<char*>(a.out + qh * D));
}

struct MultiPlan {
  int nw, q_per_block, qblocks, part_tokens, num_parts, run_tokens, runs;
  size_t ws_bytes, ws_ml_off, ws_np_off;
};

int64_t round_up_to(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// PKV_ATTN_PARTS_PER_WG (pkv_set_tuning in include/pkv.h): partitions one
// matrix-core workgroup walks; 0 = the heuristic.
int knob_parts_per_wg() { return pkv::tuning(pkv::kKnobPartsPerWg); }

// Which cache types a caller accepts: 0 = bf16 only, 1 = one-byte codes only,
// 2 = any of them (workspace sizing).
pkv_status multi_plan(int32_t num_seqs, int32_t num_q_heads, int32_t total_q,
                      int32_t max_q_per_seq, int32_t max_seq_len, int32_t partition_tokens,
                      const pkv_geom* g, const char* who, MultiPlan* pl, int types = 0) {
  if (pkv_status st = pkv::check_geom(g, who)) return st;
  const bool quant = pkv::is_quant(g->dtype);
  if ((types == 0 && g->dtype != PKV_BF16) || (types == 1 && !quant) ||
      (types == 2 && g->dtype != PKV_BF16 && !quant))
    return pkv::fail(types == 1 ? PKV_ERR_INVALID_ARG : PKV_ERR_UNSUPPORTED,
                     "%s: dtype %d is not %s", who, g->dtype,
                     types == 1 ? "a quantized cache type" : "bf16 or a quantized cache type");
  if (g->head_dim != 64 && g->head_dim != 128)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "%s: head_dim %d (built: 64, 128)", who, g->head_dim);
  if (quant && g->head_dim != 128)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "%s: quantized pools need head_dim 128", who);
  if (g->block_size < 8)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "%s: block_size %d < 8", who, g->block_size);
  if (num_seqs < 0 || num_q_heads <= 0 || total_q < 0 || max_q_per_seq < 0 || max_seq_len < 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: negative size", who);
  if (num_q_heads % g->num_kv_heads != 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: num_q_heads %d is not a multiple of num_kv_heads %d",
                     who, num_q_heads, g->num_kv_heads);
  const int G = num_q_heads / g->num_kv_heads;
  if (G > 64) return pkv::fail(PKV_ERR_UNSUPPORTED, "%s: more than 64 query heads per group", who);
  if (num_seqs > 65535 || g->num_kv_heads > 65535)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: more than 65535 sequences or KV heads", who);
  if (partition_tokens < 0 || partition_tokens % kKT != 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: partition_tokens %d must be a multiple of %d",
                     who, partition_tokens, kKT);
  const int mq = max_q_per_seq > 0 ? max_q_per_seq : 1;
  // 16 rows per wave, up to 4 waves; 128 rows (nw = 8 here: four waves of
  // two 16-row groups, launched as such) for longer chunks of bf16 rows of
  // 128, whose K/V tiles then serve twice the rows per staging (one-byte and
  // 64-wide tiles keep 64 rows)
  const bool wide = g->head_dim == 128 && !quant;
  const int cap = (wide ? 128 : 64) / G;
  const int rows = (mq < cap ? mq : cap) * G;
  pl->nw = rows <= 16 ? 1 : (rows <= 32 ? 2 : (rows <= 64 ? 4 : 8));
  pl->q_per_block = 16 * pl->nw / G;
  pl->qblocks = (mq + pl->q_per_block - 1) / pl->q_per_block;
  const int len = max_seq_len > 0 ? max_seq_len : 1;
  if (partition_tokens > 0) {
    pl->part_tokens = partition_tokens;
  } else {
    // Enough workgroups to fill the GPU: split long histories into about
    // 3072 workgroups when the (block, head, sequence) items alone are fewer
    // than 2048; partitions stay >= 256.
    const int64_t items = int64_t(num_seqs) * g->num_kv_heads * pl->qblocks;
    int64_t parts = items >= 2048 ? 1 : (3072 + items - 1) / (items > 0 ? items : 1);
    int64_t pt = round_up_to((len + parts - 1) / parts, kKT);
    if (pt < 256) pt = 256;
    pl->part_tokens = static_cast<int>(pt < round_up_to(len, kKT) ? pt : round_up_to(len, kKT));
  }
  const int64_t np = (int64_t(len) + pl->part_tokens - 1) / pl->part_tokens;
  if (np > 65535 ||
      int64_t(pl->qblocks) * ((int64_t(g->num_kv_heads) * num_seqs + 7) / 8 * 8) > 2147483647LL)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: too many partitions or query blocks", who);
  pl->num_parts = static_cast<int>(np);
  // Runs of positions per workgroup, each folded into one piece (as on the
  // decode route): single partitions up to 4096 workgroups, else runs of
  // whole partitions, about 4096 of them.
  const pkv::DecodeRuns dr =
      pkv::decode_runs(static_cast<int32_t>(int64_t(num_seqs) * pl->qblocks), g->num_kv_heads,
                       len, pl->part_tokens, pl->num_parts, 4096);
  pl->run_tokens = dr.run_tokens;
  pl->runs = dr.runs;
  if (pl->runs > 1) {
    const size_t rowsq = size_t(total_q) * num_q_heads;
    pl->ws_ml_off = rowsq * pl->runs * g->head_dim * sizeof(float);
    pl->ws_np_off = pl->ws_ml_off + rowsq * pl->runs * sizeof(float2);
    pl->ws_bytes = pl->ws_np_off + rowsq * sizeof(int32_t);
  } else {
    pl->ws_bytes = pl->ws_ml_off = pl->ws_np_off = 0;
  }
  return PKV_OK;
}

template <int D, int Q, bool kStream>
void launch_multi_variant(const MultiPlan& pl, const MultiArgs& a, int num_seqs,
                          int num_kv_heads, hipStream_t st);

// The main kernel only (no merge).  K/V are streamed with non-temporal loads
// when each (sequence, KV head) history is read by one query block and the
// caller does not report shared blocks; with several query blocks (prefill
// chunks) every block re-reads the history, which then stays cacheable.
template <int D, int Q>
void launch_multi_main(const MultiPlan& pl, const MultiArgs& a, int num_seqs, int num_kv_heads,
                       hipStream_t st, bool shared_blocks = false) {
  if (pl.qblocks == 1 && !shared_blocks)
    launch_multi_variant<D, Q, true>(pl, a, num_seqs, num_kv_heads, st);
  else
    launch_multi_variant<D, Q, false>(pl, a, num_seqs, num_kv_heads, st);
}

template <int D, int Q, bool kStream>
void launch_multi_variant(const MultiPlan& pl, const MultiArgs& args, int num_seqs,
                          int num_kv_heads, hipStream_t st) {
  MultiArgs a = args;
  a.num_sg = num_kv_heads * num_seqs;
  const int sgs = pl.qblocks == 1 ? a.num_sg : (a.num_sg + 7) / 8 * 8;  // see the kernel
  const dim3 grid(pl.qblocks * sgs, pl.runs);
  switch (pl.nw) {
    case 1: hipLaunchKernelGGL((attn_multi_kernel<D, 1, Q, kStream>), grid, dim3(64), 0, st, a); break;
    case 2: hipLaunchKernelGGL((attn_multi_kernel<D, 2, Q, kStream>), grid, dim3(128), 0, st, a); break;
    case 4: hipLaunchKernelGGL((attn_multi_kernel<D, 4, Q, kStream>), grid, dim3(256), 0, st, a); break;
    default:
      if constexpr (D == 128 && Q == pkv::mfma::kBf16)  // the plan's condition for 128 rows
        hipLaunchKernelGGL((attn_multi_kernel<D, 4, Q, kStream, 2>), grid, dim3(256), 0, st, a);
      break;
  }
}

template <int D, int Q>
void launch_multi(const MultiPlan& pl, const MultiArgs& a, int num_seqs, int num_kv_heads,
                  int total_q, hipStream_t st) {
  launch_multi_main<D, Q>(pl, a, num_seqs, num_kv_heads, st);
  if (pl.runs > 16 && total_q > 0)
    hipLaunchKernelGGL((attn_multi_merge_wide_kernel<D>), dim3(a.num_q_heads, total_q),
                       dim3(pkv::kMergeThreads), 0, st, a);
  else if (pl.runs > 1 && total_q > 0)
    hipLaunchKernelGGL((attn_multi_merge_kernel<D>), dim3(a.num_q_heads, total_q), dim3(64), 0,
                       st, a);
}

pkv_status multi_impl(const char* who, int types, const void* q, const int32_t* q_offsets,
                      const void* k_cache, const void* v_cache, const pkv_kv_scales* scales,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* seq_lens, float scale, void* out, int32_t num_seqs,
                      int32_t num_q_heads, int32_t total_q, int32_t max_q_per_seq,
                      int32_t max_seq_len, int32_t partition_tokens, void* workspace,
                      size_t workspace_bytes, const pkv_geom* geom, void* stream) {
  MultiPlan pl;
  if (pkv_status st = multi_plan(num_seqs, num_q_heads, total_q, max_q_per_seq, max_seq_len,
                                 partition_tokens, geom, who, &pl, types))
    return st;
  const int kind = geom->dtype == PKV_FP8_E4M3 ? pkv::mfma::kFp8
                 : geom->dtype == PKV_INT8 ? pkv::mfma::kInt8 : pkv::mfma::kBf16;
  if (kind != pkv::mfma::kBf16) {
    if (!scales) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: null scales", who);
    if (kind == pkv::mfma::kFp8 &&
        !(std::isfinite(scales->k_scale) && scales->k_scale > 0.f &&
          std::isfinite(scales->v_scale) && scales->v_scale > 0.f))
      return pkv::fail(PKV_ERR_INVALID_ARG, "%s: FP8 scales must be finite and > 0", who);
    if (kind == pkv::mfma::kInt8 &&
        (!scales->k_scales || !scales->v_scales ||
         (reinterpret_cast<uintptr_t>(scales->k_scales) & 3u) ||
         (reinterpret_cast<uintptr_t>(scales->v_scales) & 3u)))
      return pkv::fail(PKV_ERR_INVALID_ARG, "%s: INT8 scale pools missing or misaligned", who);
  }
  if (!std::isfinite(scale)) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: scale is not finite", who);
  if (max_blocks_per_seq < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: negative size", who);
  if (num_seqs == 0 || total_q == 0 || max_q_per_seq == 0) return PKV_OK;
  if (!q || !q_offsets || !k_cache || !v_cache || !block_tables || !seq_lens || !out)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!pkv::aligned16(q) || !pkv::aligned16(out) || !pkv::aligned16(k_cache) ||
      !pkv::aligned16(v_cache) || (reinterpret_cast<uintptr_t>(block_tables) & 3u) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u) || (reinterpret_cast<uintptr_t>(q_offsets) & 3u))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: misaligned pointer", who);
  if (pl.ws_bytes > 0) {
    if (!workspace || workspace_bytes < pl.ws_bytes)
      return pkv::fail(PKV_ERR_INVALID_ARG, "%s: workspace of %zu bytes needed, %zu given", who,
                       pl.ws_bytes, workspace ? workspace_bytes : size_t(0));
    if (!pkv::aligned16(workspace))
      return pkv::fail(PKV_ERR_INVALID_ARG, "%s: misaligned workspace", who);
  }
  MultiArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.q_offsets = q_offsets;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.out = static_cast<uint16_t*>(out);
  char* ws = static_cast<char*>(workspace);
  a.ws_acc = pl.ws_bytes ? reinterpret_cast<float*>(ws) : nullptr;
  a.ws_ml = pl.ws_bytes ? reinterpret_cast<float2*>(ws + pl.ws_ml_off) : nullptr;
  a.ws_np = pl.ws_bytes ? reinterpret_cast<int32_t*>(ws + pl.ws_np_off) : nullptr;
  a.row_elems = geom->num_kv_heads * geom->head_dim;
  a.block_elems = int64_t(geom->block_size) * a.row_elems;
  a.max_blocks = max_blocks_per_seq;
  a.num_q_heads = num_q_heads;
  a.total_q = total_q;
  a.group = num_q_heads / geom->num_kv_heads;
  a.num_blocks = geom->num_blocks;
  a.block_shift = pkv::log2_exact(geom->block_size);
  const int64_t cap = int64_t(max_blocks_per_seq) * geom->block_size;
  a.len_cap = static_cast<int32_t>(max_seq_len < cap ? max_seq_len : cap);
  a.q_per_block = pl.q_per_block;
  a.num_qblocks = pl.qblocks;
  a.num_kv_heads = geom->num_kv_heads;
  a.num_parts = pl.num_parts;
  a.part_tokens = pl.part_tokens;
  a.run_tokens = pl.run_tokens;
  a.piece_tokens = pl.run_tokens;
  a.piece_stride = pl.runs;
  a.scale_log2 = static_cast<float>(double(scale) * 1.4426950408889634 *
                                    (kind == pkv::mfma::kFp8 ? double(scales->k_scale) : 1.0));
  a.v_scale = kind == pkv::mfma::kFp8 ? scales->v_scale : 1.f;
  a.k_scales = kind == pkv::mfma::kInt8 ? scales->k_scales : nullptr;
  a.v_scales = kind == pkv::mfma::kInt8 ? scales->v_scales : nullptr;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (kind == pkv::mfma::kFp8)
    launch_multi<128, pkv::mfma::kFp8>(pl, a, num_seqs, geom->num_kv_heads, total_q, st);
  else if (kind == pkv::mfma::kInt8)
    launch_multi<128, pkv::mfma::kInt8>(pl, a, num_seqs, geom->num_kv_heads, total_q, st);
  else if (geom->head_dim == 128)
    launch_multi<128, pkv::mfma::kBf16>(pl, a, num_seqs, geom->num_kv_heads, total_q, st);
  else
    launch_multi<64, pkv::mfma::kBf16>(pl, a, num_seqs, geom->num_kv_heads, total_q, st);
  if (hipError_t e = hipGetLastError())
    return pkv::fail(PKV_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return PKV_OK;
}


}  // namespace

namespace pkv {

DecodeRuns decode_runs(int32_t num_seqs, int32_t num_kv_heads, int32_t len_cap,
                       int32_t part_tokens, int32_t num_parts, int64_t fill) {
  DecodeRuns d;
  const int64_t items = int64_t(num_seqs) * num_kv_heads;
  const int64_t wgs = items * num_parts;
  const int knob = knob_parts_per_wg();
  if (knob) {
    const int64_t ppw = knob < num_parts ? knob : num_parts;
    d.run_tokens = static_cast<int32_t>(ppw * part_tokens);
    d.runs = static_cast<int32_t>((num_parts + ppw - 1) / ppw);
  } else if (wgs > fill) {
    // runs of whole partitions, about fill / items per history
    int64_t w = (fill + items - 1) / (items > 0 ? items : 1);
    if (w > num_parts) w = num_parts;
    const int64_t ppw = (num_parts + w - 1) / w;
    d.run_tokens = static_cast<int32_t>(ppw * part_tokens);
    d.runs = static_cast<int32_t>((num_parts + ppw - 1) / ppw);
  } else {
    d.run_tokens = part_tokens;
    d.runs = num_parts;
  }
  return d;
}

pkv_status mfma_decode(const void* q, const void* k_cache, const void* v_cache, int kind,
                       float k_scale, float v_scale, const float* k_scales,
                       const float* v_scales, const int32_t* block_tables, int32_t max_blocks,
                       const int32_t* seq_lens, float scale, void* out, int32_t num_seqs,
                       int32_t num_q_heads, int32_t len_cap, int32_t part_tokens,
                       int32_t num_parts, const DecodeRuns& runs, float* ws_acc,
                       float2* ws_ml, bool stream_kv, const pkv_geom* g, hipStream_t st) {
  const int G = num_q_heads / g->num_kv_heads;
  MultiPlan pl;
  pl.nw = G <= 16 ? 1 : (G <= 32 ? 2 : 4);
  pl.q_per_block = 16 * pl.nw / G;
  if (pl.q_per_block < 1) pl.q_per_block = 1;
  pl.qblocks = 1;
  pl.part_tokens = part_tokens;
  pl.num_parts = num_parts;
  pl.run_tokens = runs.run_tokens;
  pl.runs = runs.runs;
  pl.ws_bytes = pl.ws_ml_off = pl.ws_np_off = 0;
  MultiArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.q_offsets = nullptr;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.out = static_cast<uint16_t*>(out);
  a.ws_acc = ws_acc;
  a.ws_ml = ws_ml;
  a.ws_np = nullptr;
  a.row_elems = g->num_kv_heads * g->head_dim;
  a.block_elems = int64_t(g->block_size) * a.row_elems;
  a.max_blocks = max_blocks;
  a.num_q_heads = num_q_heads;
  a.total_q = num_seqs;
  a.group = G;
  a.num_blocks = g->num_blocks;
  a.block_shift = pkv::log2_exact(g->block_size);
  a.len_cap = len_cap;
  a.q_per_block = pl.q_per_block;
  a.num_qblocks = 1;
  a.num_kv_heads = g->num_kv_heads;
  a.num_parts = num_parts;
  a.part_tokens = part_tokens;
  a.run_tokens = runs.run_tokens;
  a.piece_tokens = runs.run_tokens;
  a.piece_stride = runs.runs;
  a.scale_log2 = static_cast<float>(double(scale) * 1.4426950408889634 *
                                    (kind == pkv::mfma::kFp8 ? double(k_scale) : 1.0));
  a.v_scale = kind == pkv::mfma::kFp8 ? v_scale : 1.f;
  a.k_scales = kind == pkv::mfma::kInt8 ? k_scales : nullptr;
  a.v_scales = kind == pkv::mfma::kInt8 ? v_scales : nullptr;
  if (kind == pkv::mfma::kFp8)
    launch_multi_main<128, pkv::mfma::kFp8>(pl, a, num_seqs, g->num_kv_heads, st, !stream_kv);
  else if (kind == pkv::mfma::kInt8)
    launch_multi_main<128, pkv::mfma::kInt8>(pl, a, num_seqs, g->num_kv_heads, st, !stream_kv);
  else
    launch_multi_main<128, pkv::mfma::kBf16>(pl, a, num_seqs, g->num_kv_heads, st, !stream_kv);
  if (hipError_t e = hipGetLastError())
    return pkv::fail(PKV_ERR_HIP, "pkv_attention_decode: matrix-core launch failed: %s",
                     hipGetErrorString(e));
  return PKV_OK;
}

}  // namespace pkv

extern "C" {

size_t pkv_attention_multi_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                           int32_t total_q, int32_t max_q_per_seq,
                                           int32_t max_seq_len, int32_t partition_tokens,
                                           const pkv_geom* geom) {
  MultiPlan pl;
  if (multi_plan(num_seqs, num_q_heads, total_q, max_q_per_seq, max_seq_len, partition_tokens,
                 geom, "pkv_attention_multi_workspace_bytes", &pl, 2) != PKV_OK)
    return static_cast<size_t>(-1);
  return pl.ws_bytes;
}

pkv_status pkv_attention_multi(const void* q, const int32_t* q_offsets, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* seq_lens, float scale,
                               void* out, int32_t num_seqs, int32_t num_q_heads, int32_t total_q,
                               int32_t max_q_per_seq, int32_t max_seq_len,
                               int32_t partition_tokens, void* workspace,
                               size_t workspace_bytes, const pkv_geom* geom, void* stream) {
  return multi_impl("pkv_attention_multi", 0, q, q_offsets, k_cache, v_cache, nullptr,
                    block_tables, max_blocks_per_seq, seq_lens, scale, out, num_seqs, num_q_heads,
                    total_q, max_q_per_seq, max_seq_len, partition_tokens, workspace,
                    workspace_bytes, geom, stream);
}

pkv_status pkv_attention_multi_quant(const void* q, const int32_t* q_offsets, const void* k_cache,
                                     const void* v_cache, const pkv_kv_scales* scales,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* seq_lens, float scale, void* out,
                                     int32_t num_seqs, int32_t num_q_heads, int32_t total_q,
                                     int32_t max_q_per_seq, int32_t max_seq_len,
                                     int32_t partition_tokens, void* workspace,
                                     size_t workspace_bytes, const pkv_geom* geom, void* stream) {
  return multi_impl("pkv_attention_multi_quant", 1, q, q_offsets, k_cache, v_cache, scales,
                    block_tables, max_blocks_per_seq, seq_lens, scale, out, num_seqs, num_q_heads,
                    total_q, max_q_per_seq, max_seq_len, partition_tokens, workspace,
                    workspace_bytes, geom, stream);
}

}  // extern "C"
