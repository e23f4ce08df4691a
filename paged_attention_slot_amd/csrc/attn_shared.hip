// Decode attention that reads a shared prefix once per group of sequences:
// pkv_attention_decode_shared (the groups come from pkv_prefix_groups, on the
// host, in prefix_groups.cpp).
//
// What is computed is decode attention ([KVM §19.2.3] paged attention; [KVX
// §01] the new token's attention; [KVX §02]/[KVX §03] grouped-query heads;
// page keys in include/pkv.h): out[s][h] = softmax over positions t < L_s of
// scale * q[s][h] . K_s[t], applied to V_s.  Sequences that took a prefix by
// reference hold the same blocks at the start of their tables ([KVM §19.2.5]);
// paging alone does not make a kernel read them once ([KVX §04], [KVX §05]:
// read reuse depends on the kernel).  Here the caller names groups of
// consecutive sequences and the length of the prefix they share, and
//
//  * attn_prefix_kernel reads the prefix of a group once per (block of
//    members, KV head, partition): its rows are (member, query head of the
//    KV head's group) pairs, up to 64 per workgroup, all attending the shared
//    positions (a member shorter than the prefix only its own), on the matrix
//    cores (pkv::mfma::attend);
//  * attn_suffix_kernel reads every sequence's remaining positions, one
//    (sequence, KV head, partition) per workgroup, the G query heads as rows;
//  * attn_shared_merge_kernel combines each (sequence, head)'s pieces by
//    log-sum-exp: the partial states of the online softmax of the positions
//    split between the two ([KVM §19.2.3] block-wise online softmax).
//
// The pieces are fp32 (weighted sum, reference, sum), so only the final
// result is rounded to bf16.
#include <hip/hip_runtime.h>

#include <cmath>

#include "geom.h"
#include "mfma_attend.h"
#include "pkv_device.h"

namespace {

using pkv::mfma::kKT;

struct SharedArgs {
  const uint16_t* q;
  const void* k_cache;           // bf16 bits or one-byte codes
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* group_starts;   // [num_groups + 1]
  const int32_t* prefix_lens;    // [num_groups]
  uint16_t* out;
  float* ws_acc;                 // [(s * H_q + h) * slots + slot][D]
  float2* ws_ml;                 // [(s * H_q + h) * slots + slot]
  int64_t block_elems;
  int32_t row_elems;
  int32_t max_blocks;
  int32_t num_seqs;
  int32_t num_groups;
  int32_t num_q_heads;
  int32_t group;                 // G = H_q / H_kv
  int32_t num_blocks;
  int32_t block_shift;
  int32_t len_cap;
  int32_t max_prefix;            // prefix lengths are clamped to this
  int32_t max_group;             // larger groups share nothing (the grid has no rows for them)
  int32_t members_per_block;     // prefix kernel: members per workgroup
  int32_t pre_parts, pre_tokens; // prefix partitions: count and length
  int32_t suf_parts, suf_tokens; // suffix partitions
  int32_t num_kv_heads;
  float scale_log2;              // FP8: the K tensor scale folded in
  float v_scale;                 // FP8
  const float* k_scales;         // INT8
  const float* v_scales;
};

__device__ __forceinline__ int clamp_len(int v, int cap) { return v < 0 ? 0 : (v > cap ? cap : v); }

// Members [first, first + count) of group gi and the prefix they share: whole
// blocks (a K/V tile then never spans more than 4 blocks), 0 for a group of
// one (nothing to share) or one larger than the grid was sized for.  Indices
// are clamped into the batch.
__device__ __forceinline__ int group_prefix(const SharedArgs& a, int gi, int* first, int* count) {
  int f = a.group_starts[gi], e = a.group_starts[gi + 1];
  f = f < 0 ? 0 : (f > a.num_seqs ? a.num_seqs : f);
  e = e < f ? f : (e > a.num_seqs ? a.num_seqs : e);
  *first = f;
  *count = e - f;
  if (e - f < 2 || e - f > a.max_group) return 0;
  int p = a.prefix_lens[gi];
  p = p < 0 ? 0 : (p > a.max_prefix ? a.max_prefix : p);
  return (p >> a.block_shift) << a.block_shift;
}

// The prefix positions of sequence s (of length L) that the prefix kernel
// serves: its group's prefix, cut at L.  The group is found by binary search
// over group_starts (the last group whose start is <= s).
__device__ __forceinline__ int seq_prefix(const SharedArgs& a, int s, int L) {
  int lo = 0, hi = a.num_groups - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.group_starts[mid] <= s) lo = mid; else hi = mid - 1;
  }
  int first, count;
  const int p = group_prefix(a, lo, &first, &count);
  if (s < first || s >= first + count) return 0;
  return p < L ? p : L;
}

// grid = (row blocks * pre_parts, H_kv, num_groups).
// (four-wave workgroups: a register budget that keeps three resident per CU)
template <int D, int NW, int Q>
__global__ void __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(NW == 4 ? 3 : 1)))
attn_prefix_kernel(SharedArgs a) {
  __shared__ __align__(16) uint16_t k_lds[pkv::mfma::k_lds_elems<D, NW, Q>()];
  __shared__ __align__(16) uint16_t v_lds[pkv::mfma::v_lds_elems<D, NW, Q>()];
  __shared__ float s_lds[pkv::mfma::s_lds_elems<Q, NW>()];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int gi = blockIdx.z, g = blockIdx.y;
  const int rb = blockIdx.x / a.pre_parts, part = blockIdx.x - rb * a.pre_parts;
  int first, count;
  const int P = group_prefix(a, gi, &first, &count);
  const int j0 = rb * a.members_per_block;
  if (P == 0 || j0 >= count) return;  // uniform over the workgroup
  const int jn = min(a.members_per_block, count - j0);
  const int t_lo = part * a.pre_tokens;
  const int t_hi = min(t_lo + a.pre_tokens, P);
  if (t_lo >= t_hi) return;

  const int G = a.group;
  const int row = 16 * w + (lane & 15);
  const int jl = row / G, hh = row - jl * G;
  const bool row_ok = jl < jn;
  const int s = first + j0 + (row_ok ? jl : 0);
  const int L = clamp_len(a.seq_lens[s], a.len_cap);
  const int64_t qh = int64_t(s) * a.num_q_heads + g * G + hh;
  // Positions every member of the block sees: up to the shortest one's last;
  // positions some member sees: up to the longest one's last (members'
  // lengths strided over the lanes, then a wave minimum and maximum).
  int lmin = a.len_cap, lmax = 0;
  for (int m = lane; m < jn; m += 64) {
    const int lm = clamp_len(a.seq_lens[first + j0 + m], a.len_cap);
    lmin = min(lmin, lm);
    lmax = max(lmax, lm);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    lmin = min(lmin, __shfl_xor(lmin, off));
    lmax = max(lmax, __shfl_xor(lmax, off));
  }
  // The prefix is read through the group's first member's table.  A shared
  // last block may be only partly written when no member has appended since
  // the fork: the History stops at the longest member, so slots past it load
  // as zeros instead of whatever bits they hold (a masked score with a NaN or
  // infinite V row would still put 0 * NaN into the products).
  const pkv::mfma::History hist{a.k_cache,      a.v_cache,     a.block_tables + int64_t(first) * a.max_blocks,
                                min(P, lmax),   g,             a.block_elems,
                                a.row_elems,    a.num_blocks,  a.block_shift,
                                a.num_kv_heads, a.v_scale,     a.k_scales,
                                a.v_scales};
  pkv::mfma::RowAcc<D> r;
  pkv::mfma::start(r);
  pkv::mfma::attend<D, NW, (NW >= 2 ? 2 : 1), Q>(hist, t_lo, t_hi, a.q + qh * D, row_ok, L - 1,
                                                lmin - 1, a.scale_log2, k_lds, v_lds, r, s_lds);
  if (!row_ok) return;
  const int64_t slot = qh * (a.pre_parts + a.suf_parts) + part;
  pkv::mfma::store_piece<D>(r, a.ws_acc + slot * D, a.ws_ml + slot);
}

// grid = (suf_parts, H_kv, num_seqs).
template <int D, int NW, int Q>
__global__ void __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(NW == 4 ? 3 : 1)))
attn_suffix_kernel(SharedArgs a) {
  __shared__ __align__(16) uint16_t k_lds[pkv::mfma::k_lds_elems<D, NW, Q>()];
  __shared__ __align__(16) uint16_t v_lds[pkv::mfma::v_lds_elems<D, NW, Q>()];
  __shared__ float s_lds[pkv::mfma::s_lds_elems<Q, NW>()];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int s = blockIdx.z, g = blockIdx.y, part = blockIdx.x;
  const int L = clamp_len(a.seq_lens[s], a.len_cap);
  const int P = seq_prefix(a, s, L);
  if (P + part * a.suf_tokens >= L) return;  // the merge counts only parts holding positions

  const int G = a.group;
  const int hh = 16 * w + (lane & 15);
  const bool row_ok = hh < G;
  const int64_t qh = int64_t(s) * a.num_q_heads + g * G + (row_ok ? hh : 0);
  const pkv::mfma::History hist{a.k_cache,      a.v_cache,     a.block_tables + int64_t(s) * a.max_blocks,
                                L,              g,             a.block_elems,
                                a.row_elems,    a.num_blocks,  a.block_shift,
                                a.num_kv_heads, a.v_scale,     a.k_scales,
                                a.v_scales};
  pkv::mfma::RowAcc<D> r;
  pkv::mfma::start(r);
  // Partitions part, part + suf_parts, ...: a suffix longer than the grid was
  // sized for is folded into the same piece.
  for (int t_lo = P + part * a.suf_tokens; t_lo < L; t_lo += a.suf_parts * a.suf_tokens)
    pkv::mfma::attend<D, NW, (NW >= 2 ? 2 : 1), Q>(hist, t_lo, min(t_lo + a.suf_tokens, L),
                                                  a.q + qh * D, row_ok, L - 1, L - 1,
                                                  a.scale_log2, k_lds, v_lds, r, s_lds);
  if (!row_ok) return;
  const int64_t slot = qh * (a.pre_parts + a.suf_parts) + a.pre_parts + part;
  pkv::mfma::store_piece<D>(r, a.ws_acc + slot * D, a.ws_ml + slot);
}

// One wave per (head, sequence): log-sum-exp over the prefix pieces and the
// suffix pieces that hold positions of this sequence.
template <int D>
__global__ void __launch_bounds__(64)
attn_shared_merge_kernel(SharedArgs a) {
  constexpr int kE = D / 64;
  const int h = blockIdx.x, s = blockIdx.y;
  const int lane = threadIdx.x;
  const int L = clamp_len(a.seq_lens[s], a.len_cap);
  const int P = seq_prefix(a, s, L);
  const int np_pre = (P + a.pre_tokens - 1) / a.pre_tokens;
  const int np_suf = min(a.suf_parts, (L - P + a.suf_tokens - 1) / a.suf_tokens);
  const int64_t qh = int64_t(s) * a.num_q_heads + h;
  const int64_t base = qh * (a.pre_parts + a.suf_parts);
  float M = -INFINITY;
  for (int p = lane; p < np_pre + np_suf; p += 64) {
    const int slot = p < np_pre ? p : a.pre_parts + (p - np_pre);
    M = fmaxf(M, a.ws_ml[base + slot].x);
  }
  M = pkv::wave_max(M);
  float lsum = 0.f, acc[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) acc[e] = 0.f;
  for (int p = 0; p < np_pre + np_suf; ++p) {
    const int slot = p < np_pre ? p : a.pre_parts + (p - np_pre);
    const float2 ml = a.ws_ml[base + slot];
    const float wgt = pkv::fast_exp2(ml.x - M);
    lsum = fmaf(wgt, ml.y, lsum);
    const float* src = a.ws_acc + (base + slot) * D;
#pragma unroll
    for (int e = 0; e < kE; ++e) acc[e] = fmaf(wgt, src[lane * kE + e], acc[e]);
  }
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  uint16_t* dst = a.out + qh * D + lane * kE;
#pragma unroll
  for (int e = 0; e < kE; ++e) dst[e] = static_cast<uint16_t>(pkv::f32_to_bf16_bits(acc[e] * inv));
}

int64_t round_up_to(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Partition length for `items` work items over histories up to `len`: split
// until about 2048 workgroups exist, never below 256 positions.
int part_tokens_for(int64_t items, int len) {
  const int64_t parts = items >= 2048 ? 1 : (2048 + items - 1) / (items > 0 ? items : 1);
  int64_t pt = round_up_to((int64_t(len) + parts - 1) / parts, kKT);
  if (pt < 256) pt = 256;
  const int64_t full = round_up_to(len > 0 ? len : 1, kKT);
  return static_cast<int>(pt < full ? pt : full);
}

struct SharedPlan {
  int nw_pre, nw_suf, members_per_block, row_blocks;
  int pre_parts, pre_tokens, suf_parts, suf_tokens;
  size_t ws_bytes, ws_ml_off;
};

pkv_status shared_plan(int32_t num_seqs, int32_t num_q_heads, int32_t num_groups,
                       int32_t max_group_size, int32_t max_prefix_len, int32_t max_suffix_len,
                       int32_t max_seq_len, const pkv_geom* g, const char* who, SharedPlan* pl,
                       int types = 0) {
  // types: 0 = bf16 only, 1 = one-byte codes only, 2 = any (workspace sizing)
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
  if (num_seqs < 0 || num_q_heads <= 0 || num_groups < 0 || max_group_size < 0 ||
      max_prefix_len < 0 || max_seq_len < 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: negative size", who);
  if (num_seqs > 0 && num_groups < 1)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: the groups must cover the batch", who);
  if (num_q_heads % g->num_kv_heads != 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: num_q_heads %d is not a multiple of num_kv_heads %d",
                     who, num_q_heads, g->num_kv_heads);
  const int G = num_q_heads / g->num_kv_heads;
  if (G > 64) return pkv::fail(PKV_ERR_UNSUPPORTED, "%s: more than 64 query heads per group", who);
  if (num_seqs > 65535 || num_groups > 65535 || g->num_kv_heads > 65535)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: more than 65535 sequences, groups or KV heads", who);
  const int mg = max_group_size > 0 ? max_group_size : 1;
  // 16 (member, head) rows per wave, up to 4 waves (eight measured no faster
  // on the shared-prefix configuration)
  const int per64 = 64 / G;
  const int rows = (mg < per64 ? mg : per64) * G;
  pl->nw_pre = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
  pl->members_per_block = 16 * pl->nw_pre / G;
  pl->row_blocks = (mg + pl->members_per_block - 1) / pl->members_per_block;
  pl->nw_suf = G <= 16 ? 1 : (G <= 32 ? 2 : 4);
  const int pre_len = max_prefix_len > 0 ? max_prefix_len : 1;
  const int seq_len = max_seq_len > 0 ? max_seq_len : 1;
  pl->pre_tokens =
      part_tokens_for(int64_t(num_groups) * g->num_kv_heads * pl->row_blocks, pre_len);
  // Suffix partitions from the longest suffix (a hint: longer suffixes are
  // folded into the grid's pieces): short critical paths, about 4096 items.
  const int suf_len = max_suffix_len > 0 && max_suffix_len < seq_len ? max_suffix_len : seq_len;
  const int64_t suf_items = int64_t(num_seqs) * g->num_kv_heads;
  const int64_t want = suf_items >= 4096 ? 1 : (4096 + suf_items - 1) / (suf_items > 0 ? suf_items : 1);
  int64_t spt = round_up_to((suf_len + want - 1) / want, kKT);
  if (spt < 64) spt = 64;
  pl->suf_tokens = static_cast<int>(spt);
  pl->pre_parts = (pre_len + pl->pre_tokens - 1) / pl->pre_tokens;
  pl->suf_parts = static_cast<int>((suf_len + spt - 1) / spt);
  if (int64_t(pl->row_blocks) * pl->pre_parts > 2147483647LL)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: too many prefix work items", who);
  const size_t slots = size_t(num_seqs) * num_q_heads * (pl->pre_parts + pl->suf_parts);
  pl->ws_ml_off = slots * g->head_dim * sizeof(float);
  pl->ws_bytes = pl->ws_ml_off + slots * sizeof(float2);
  return PKV_OK;
}

template <int D, int Q>
void launch_shared(const SharedPlan& pl, const SharedArgs& a, int num_kv_heads, hipStream_t st) {
  if (a.num_groups > 0 && a.max_prefix > 0) {
    const dim3 grid(pl.row_blocks * pl.pre_parts, num_kv_heads, a.num_groups);
    switch (pl.nw_pre) {
      case 1: hipLaunchKernelGGL((attn_prefix_kernel<D, 1, Q>), grid, dim3(64), 0, st, a); break;
      case 2: hipLaunchKernelGGL((attn_prefix_kernel<D, 2, Q>), grid, dim3(128), 0, st, a); break;
      default: hipLaunchKernelGGL((attn_prefix_kernel<D, 4, Q>), grid, dim3(256), 0, st, a); break;
    }
  }
  const dim3 grid(pl.suf_parts, num_kv_heads, a.num_seqs);
  switch (pl.nw_suf) {
    case 1: hipLaunchKernelGGL((attn_suffix_kernel<D, 1, Q>), grid, dim3(64), 0, st, a); break;
    case 2: hipLaunchKernelGGL((attn_suffix_kernel<D, 2, Q>), grid, dim3(128), 0, st, a); break;
    default: hipLaunchKernelGGL((attn_suffix_kernel<D, 4, Q>), grid, dim3(256), 0, st, a); break;
  }
  hipLaunchKernelGGL((attn_shared_merge_kernel<D>), dim3(a.num_q_heads, a.num_seqs), dim3(64), 0,
                     st, a);
}

pkv_status shared_impl(const char* who, int types, const void* q, const void* k_cache,
                       const void* v_cache, const pkv_kv_scales* scales,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* seq_lens, const int32_t* group_starts,
                       const int32_t* prefix_lens, int32_t num_groups, int32_t max_group_size,
                       int32_t max_prefix_len, int32_t max_suffix_len, float scale, void* out,
                       int32_t num_seqs, int32_t num_q_heads, int32_t max_seq_len,
                       void* workspace, size_t workspace_bytes, const pkv_geom* geom,
                       void* stream) {
  SharedPlan pl;
  if (pkv_status st = shared_plan(num_seqs, num_q_heads, num_groups, max_group_size,
                                  max_prefix_len, max_suffix_len, max_seq_len, geom, who, &pl,
                                  types))
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
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !group_starts || !prefix_lens ||
      !out)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!pkv::aligned16(q) || !pkv::aligned16(out) || !pkv::aligned16(k_cache) ||
      !pkv::aligned16(v_cache) || (reinterpret_cast<uintptr_t>(block_tables) & 3u) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u) ||
      (reinterpret_cast<uintptr_t>(group_starts) & 3u) ||
      (reinterpret_cast<uintptr_t>(prefix_lens) & 3u))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: misaligned pointer", who);
  if (!workspace || workspace_bytes < pl.ws_bytes)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: workspace of %zu bytes needed, %zu given", who,
                     pl.ws_bytes, workspace ? workspace_bytes : size_t(0));
  if (!pkv::aligned16(workspace))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: misaligned workspace", who);
  SharedArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_kv_heads = geom->num_kv_heads;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.group_starts = group_starts;
  a.prefix_lens = prefix_lens;
  a.out = static_cast<uint16_t*>(out);
  char* ws = static_cast<char*>(workspace);
  a.ws_acc = reinterpret_cast<float*>(ws);
  a.ws_ml = reinterpret_cast<float2*>(ws + pl.ws_ml_off);
  a.row_elems = geom->num_kv_heads * geom->head_dim;
  a.block_elems = int64_t(geom->block_size) * a.row_elems;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_groups = num_groups;
  a.num_q_heads = num_q_heads;
  a.group = num_q_heads / geom->num_kv_heads;
  a.num_blocks = geom->num_blocks;
  a.block_shift = pkv::log2_exact(geom->block_size);
  const int64_t cap = int64_t(max_blocks_per_seq) * geom->block_size;
  a.len_cap = static_cast<int32_t>(max_seq_len < cap ? max_seq_len : cap);
  a.max_prefix = max_prefix_len < a.len_cap ? max_prefix_len : a.len_cap;
  a.max_group = max_group_size;
  a.members_per_block = pl.members_per_block;
  a.pre_parts = pl.pre_parts;
  a.pre_tokens = pl.pre_tokens;
  a.suf_parts = pl.suf_parts;
  a.suf_tokens = pl.suf_tokens;
  a.scale_log2 = static_cast<float>(double(scale) * 1.4426950408889634 *
                                    (kind == pkv::mfma::kFp8 ? double(scales->k_scale) : 1.0));
  a.v_scale = kind == pkv::mfma::kFp8 ? scales->v_scale : 1.f;
  a.k_scales = kind == pkv::mfma::kInt8 ? scales->k_scales : nullptr;
  a.v_scales = kind == pkv::mfma::kInt8 ? scales->v_scales : nullptr;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (kind == pkv::mfma::kFp8)
    launch_shared<128, pkv::mfma::kFp8>(pl, a, geom->num_kv_heads, st);
  else if (kind == pkv::mfma::kInt8)
    launch_shared<128, pkv::mfma::kInt8>(pl, a, geom->num_kv_heads, st);
  else if (geom->head_dim == 128)
    launch_shared<128, pkv::mfma::kBf16>(pl, a, geom->num_kv_heads, st);
  else
    launch_shared<64, pkv::mfma::kBf16>(pl, a, geom->num_kv_heads, st);
  if (hipError_t e = hipGetLastError())
    return pkv::fail(PKV_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return PKV_OK;
}


}  // namespace

extern "C" {

size_t pkv_attention_shared_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                            int32_t num_groups, int32_t max_group_size,
                                            int32_t max_prefix_len, int32_t max_suffix_len,
                                            int32_t max_seq_len, const pkv_geom* geom) {
  SharedPlan pl;
  if (shared_plan(num_seqs, num_q_heads, num_groups, max_group_size, max_prefix_len,
                  max_suffix_len, max_seq_len, geom, "pkv_attention_shared_workspace_bytes",
                  &pl, 2) != PKV_OK)
    return static_cast<size_t>(-1);
  return pl.ws_bytes;
}

pkv_status pkv_attention_decode_shared(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* seq_lens, const int32_t* group_starts,
                                       const int32_t* prefix_lens, int32_t num_groups,
                                       int32_t max_group_size, int32_t max_prefix_len,
                                       int32_t max_suffix_len, float scale, void* out,
                                       int32_t num_seqs, int32_t num_q_heads, int32_t max_seq_len,
                                       void* workspace, size_t workspace_bytes,
                                       const pkv_geom* geom, void* stream) {
  return shared_impl("pkv_attention_decode_shared", 0, q, k_cache, v_cache, nullptr, block_tables,
                     max_blocks_per_seq, seq_lens, group_starts, prefix_lens, num_groups,
                     max_group_size, max_prefix_len, max_suffix_len, scale, out, num_seqs,
                     num_q_heads, max_seq_len, workspace, workspace_bytes, geom, stream);
}

pkv_status pkv_attention_decode_shared_quant(
    const void* q, const void* k_cache, const void* v_cache, const pkv_kv_scales* scales,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
    const int32_t* group_starts, const int32_t* prefix_lens, int32_t num_groups,
    int32_t max_group_size, int32_t max_prefix_len, int32_t max_suffix_len, float scale,
    void* out, int32_t num_seqs, int32_t num_q_heads, int32_t max_seq_len, void* workspace,
    size_t workspace_bytes, const pkv_geom* geom, void* stream) {
  return shared_impl("pkv_attention_decode_shared_quant", 1, q, k_cache, v_cache, scales,
                     block_tables, max_blocks_per_seq, seq_lens, group_starts, prefix_lens,
                     num_groups, max_group_size, max_prefix_len, max_suffix_len, scale, out,
                     num_seqs, num_q_heads, max_seq_len, workspace, workspace_bytes, geom,
                     stream);
}

}  // extern "C"
