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
//  * attn_prefix_fused_kernel (suffix hints up to kFusedSuffix positions,
//    one launch): the workgroup of a (KV head, block of 32 (member, query
//    head) rows) first walks its members' own positions after the prefix
//    (items of one member and up to 16 of its rows, its query heads, dealt
//    to the waves in turn), then the prefix, cut among its eight waves so
//    that their walks even out, on the matrix cores (pkv::mfma::attend_rows,
//    two row groups of 16 per wave for the prefix), and combines all the
//    states through LDS by
//    log-sum-exp ([KVM §19.2.3] block-wise online softmax): nothing travels
//    through memory but the result.  The workgroups past the prefix ones
//    attend the sequences that share nothing, whole.
//  * Otherwise, attn_suffix_kernel (first) reads every sequence's positions
//    after its prefix, one (sequence, KV head, partition) per workgroup, and
//    leaves one fp32 piece (weighted sum, reference, sum) per partition (a
//    sequence without a shared prefix is attended whole by its first
//    partition's workgroup, which writes its result); attn_prefix_kernel
//    (second) reads the prefix of a group once per (KV head, block of 32
//    rows), its eight waves an eighth each, and combines their states with
//    the members' suffix pieces.
//
// Only the final result is rounded to bf16.
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
  float* ws_acc;                 // suffix pieces: [(s * H_q + h) * suf_parts + part][D]
  float2* ws_ml;                 // [(s * H_q + h) * suf_parts + part]
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
  int32_t suf_parts, suf_tokens; // suffix partitions
  int32_t row_blocks;            // prefix workgroups per (group, KV head): 32 rows each
  int32_t pre_blocks;            // prefix workgroups in all
  int32_t num_kv_heads;
  int32_t fused;                // the prefix kernel walks its members' suffixes too
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

// attn_suffix_kernel (one wave per workgroup) runs first; attn_prefix_kernel
// (eight waves, each with its own LDS tile area, two row groups of 16 each)
// second, finishing every member's result.
constexpr int kSharedWaves = 8;
constexpr int kPrefixRG = 2;                // row groups of 16 per prefix workgroup
constexpr int kPrefixRows = 16 * kPrefixRG;
constexpr int kFusedSuffix = 1024;         // longest suffix hint the prefix kernel walks itself

template <int D, int Q, int W>
struct SharedLds {
  uint16_t k[W][pkv::mfma::k_lds_elems<D, 1, Q>()];
  uint16_t v[W][pkv::mfma::v_lds_elems<D, 1, Q>()];
  float s[W][pkv::mfma::s_lds_elems<Q, 1>()];
};

// The suffix states of a prefix workgroup's rows when it walks its members'
// suffixes itself: [row][D] weighted sums, then (reference, sum) per row.
template <int D>
struct SuffixStates {
  float acc[32][D];
  float2 ml[32];
};

// One bf16 tile of registers in flight for the single-wave walks, two for
// one-byte codes (as in the single-wave decode walk): with two row groups a
// wave this keeps the prefix walk within 256 registers.
template <int Q> constexpr int shared_pd() { return Q == pkv::mfma::kBf16 ? 1 : 2; }

// Prefix role, workgroup x of pre_blocks = H_kv * row_blocks * num_groups
// (KV head fastest: with 8 KV heads all the row blocks of one head go to one
// XCD, as workgroups are dealt to the XCDs round robin, and share its L2
// copy of that head's prefix).  Rows: 32 (member, query head) pairs of the
// group's members, two row groups of 16 in every wave; the eight waves walk
// an eighth of the prefix each (one workgroup per CU by LDS, 2 waves per
// SIMD: more walks of half the length than four waves of quarters), then
// combine their states through LDS into one piece per row.
//
// kFused: the workgroup also walks its members' own positions after the
// prefix (so the suffix kernel leaves the group's members alone): work items
// (member, up to 16 of its rows in the block) go to the waves round robin,
// each a single-wave walk of that member's suffix with its query heads as
// rows, before the prefix eighths; the states wait in ``suf`` for the
// combine, and no piece travels through memory.
template <int D, int Q, bool kFused>
__device__ void prefix_role(const SharedArgs& a, int x, SharedLds<D, Q, kSharedWaves>& lds,
                            SuffixStates<D>* suf) {
  constexpr int kW = kSharedWaves;
  static_assert(16 * D * 4 + 16 * 8 <= int(sizeof(lds.k[0])) &&
                16 * D * 4 + 16 * 8 <= int(sizeof(lds.v[0])),
                "a row group's state fits a wave's K (group 0) or V (group 1) area");
  static_assert(kPrefixRG == 2, "the states of two row groups per wave");
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int g = x % a.num_kv_heads;
  const int rb = (x / a.num_kv_heads) % a.row_blocks;
  const int gi = x / (a.num_kv_heads * a.row_blocks);
  int first, count;
  const int P = group_prefix(a, gi, &first, &count);
  const int G = a.group;
  const int nrows = count * G;  // (member, query head) rows of the group
  const int r0 = kPrefixRows * rb;
  if (P == 0 || r0 >= nrows) return;  // uniform over the workgroup

  // This lane's rows (lane & 15 of each row group): member j, query head hh
  // of KV head g.
  bool row_ok[kPrefixRG];
  int p_row[kPrefixRG];
  const uint16_t* qrow[kPrefixRG];
#pragma unroll
  for (int rg = 0; rg < kPrefixRG; ++rg) {
    const int rr = r0 + 16 * rg + (lane & 15);
    row_ok[rg] = rr < nrows;
    const int j = row_ok[rg] ? rr / G : 0, hh = row_ok[rg] ? rr - j * G : 0;
    const int s = first + j;
    p_row[rg] = clamp_len(a.seq_lens[s], a.len_cap) - 1;
    qrow[rg] = a.q + (int64_t(s) * a.num_q_heads + g * G + hh) * D;
  }
  // Positions every member of the block sees: up to the shortest one's last;
  // positions some member sees: up to the longest one's last.
  const int j_lo = r0 / G, j_hi = min(count, (r0 + kPrefixRows - 1) / G + 1);
  int lmin = a.len_cap, lmax = 0;
  for (int m = j_lo + lane; m < j_hi; m += 64) {
    const int lm = clamp_len(a.seq_lens[first + m], a.len_cap);
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
  const int len = min(P, lmax);
  const pkv::mfma::History hist{a.k_cache,      a.v_cache,     a.block_tables + int64_t(first) * a.max_blocks,
                                len,            g,             a.block_elems,
                                a.row_elems,    a.num_blocks,  a.block_shift,
                                a.num_kv_heads, a.v_scale,     a.k_scales,
                                a.v_scales};
  if constexpr (kFused) {
    // Suffix items, in member order: member j's rows of the block are
    // [max(j G - r0, 0), min((j + 1) G - r0, 32, nrows - r0)), in chunks of 16.
    int item = 0;
    for (int j = j_lo; j < j_hi; ++j) {
      const int ra = max(j * G - r0, 0);
      const int rb = min(min((j + 1) * G - r0, kPrefixRows), nrows - r0);
      for (int c0 = ra; c0 < rb; c0 += 16, ++item) {
        if (item % kW != w) continue;  // uniform
        const int i = c0 + (lane & 15);  // this lane's row of the block
        const bool ok = i < min(c0 + 16, rb);
        const int sj = first + j;
        const int Lj = clamp_len(a.seq_lens[sj], a.len_cap);
        const int hh = ok ? r0 + i - j * G : 0;
        const uint16_t* const sq[1] = {a.q + (int64_t(sj) * a.num_q_heads + g * G + hh) * D};
        const bool sok[1] = {ok};
        const int sp[1] = {Lj - 1};
        const pkv::mfma::History sh{a.k_cache,      a.v_cache,     a.block_tables + int64_t(sj) * a.max_blocks,
                                    Lj,             g,             a.block_elems,
                                    a.row_elems,    a.num_blocks,  a.block_shift,
                                    a.num_kv_heads, a.v_scale,     a.k_scales,
                                    a.v_scales};
        pkv::mfma::RowAcc<D> rs[1];
        pkv::mfma::start(rs[0]);
        pkv::mfma::attend_rows<D, 1, shared_pd<Q>(), Q, false, pkv::mfma::NoEmit, false, true, 1>(
            sh, min(P, Lj), Lj, sq, sok, sp, Lj - 1, a.scale_log2, lds.k[w], lds.v[w], rs,
            lds.s[w]);
        if (ok) pkv::mfma::store_piece<D>(rs[0], suf->acc[i], &suf->ml[i]);
      }
    }
  }
  // Wave w walks tiles [w * per, (w + 1) * per) of the prefix, alone (no
  // workgroup barrier inside: the eighths may differ in length).  kFused:
  // the prefix is cut so that the waves' walks even out, a prefix tile (two
  // row groups) counting twice a suffix tile (one): wave w takes prefix
  // tiles in proportion to max(0, C - S_w), S_w its suffix tiles and C the
  // workgroup's total over the waves.
  const int tiles = (len + kKT - 1) / kKT;
  const int per = (tiles + kW - 1) / kW;
  int t_lo = min(w * per * kKT, len), t_hi = min((w + 1) * per * kKT, len);
  if constexpr (kFused) {
    int sw[kW];
#pragma unroll
    for (int u = 0; u < kW; ++u) sw[u] = 0;
    int item = 0;
    for (int j = j_lo; j < j_hi; ++j) {
      const int Lj = clamp_len(a.seq_lens[first + j], a.len_cap);
      const int st = (Lj - min(P, Lj) + kKT - 1) / kKT;
      const int ra = max(j * G - r0, 0);
      const int rb = min(min((j + 1) * G - r0, kPrefixRows), nrows - r0);
      for (int c0 = ra; c0 < rb; c0 += 16, ++item) {
        const int v = item % kW;
#pragma unroll
        for (int u = 0; u < kW; ++u) sw[u] += u == v ? st : 0;
      }
    }
    int tot = 0;
#pragma unroll
    for (int u = 0; u < kW; ++u) tot += sw[u];
    const int C = (2 * tiles + tot + kW - 1) / kW;
    int dsum = 0, before = 0, mine = 0;
#pragma unroll
    for (int u = 0; u < kW; ++u) {
      const int d = max(0, C - sw[u]);
      before += u < w ? d : 0;
      mine = u == w ? d : mine;
      dsum += d;
    }
    if (dsum > 0) {
      const int b0 = static_cast<int>(int64_t(tiles) * before / dsum);
      const int b1 = static_cast<int>(int64_t(tiles) * (before + mine) / dsum);
      t_lo = min(b0 * kKT, len);
      t_hi = min(b1 * kKT, len);
    }
  }
  pkv::mfma::RowAcc<D> r[kPrefixRG];
#pragma unroll
  for (int rg = 0; rg < kPrefixRG; ++rg) pkv::mfma::start(r[rg]);
  // one tile of registers in flight for every kind: two row groups fill the
  // register budget
  pkv::mfma::attend_rows<D, 1, 1, Q, false, pkv::mfma::NoEmit, false, true, kPrefixRG>(
      hist, t_lo, t_hi, qrow, row_ok, p_row, lmin - 1, a.scale_log2, lds.k[w], lds.v[w], r,
      lds.s[w]);
  // The wave's states to its own areas (its walk is over): row group 0 in
  // its K area, 1 in its V area, each [row][D] weighted sums, then
  // (reference, sum) per row.
#pragma unroll
  for (int rg = 0; rg < kPrefixRG; ++rg) {
    float* st = reinterpret_cast<float*>(rg == 0 ? lds.k[w] : lds.v[w]);
    pkv::mfma::store_piece<D>(r[rg], st + (lane & 15) * D,
                              reinterpret_cast<float2*>(st + 16 * D) + (lane & 15));
  }
  __syncthreads();
  // Thread t combines row t / 16, elements (t % 16) * D / 16 .. + D / 16 - 1:
  // the eight waves' states and the member's suffix pieces (the suffix
  // kernel ran before), by log-sum-exp, into the result.
  constexpr int kE = D / 16;
  static_assert(64 * kW == 16 * kPrefixRows, "one thread per (row, sixteenth of a row)");
  const int t = threadIdx.x;
  const int crow = t >> 4, d0 = (t & 15) * kE;
  const int crg = r0 + crow;
  if (crg >= nrows) return;
  const int cj = crg / G, ch = crg - cj * G;
  const int cs = first + cj;
  const int cL = clamp_len(a.seq_lens[cs], a.len_cap);
  const int cP = P < cL ? P : cL;
  // (a member with nothing to attend, cL = 0, was written whole by the
  // suffix kernel)
  if (cP == 0) return;
  const int np_suf =
      kFused || cL <= cP ? 0 : min(a.suf_parts, (cL - cP + a.suf_tokens - 1) / a.suf_tokens);
  const int64_t cqh = int64_t(cs) * a.num_q_heads + g * G + ch;
  const int64_t base = cqh * a.suf_parts;
  const int cgrp = crow >> 4, crl = crow & 15;
  const auto state = [&](int v) {
    return reinterpret_cast<const float*>(cgrp == 0 ? lds.k[v] : lds.v[v]);
  };
  float M = -INFINITY;
#pragma unroll
  for (int v = 0; v < kW; ++v)
    M = fmaxf(M, reinterpret_cast<const float2*>(state(v) + 16 * D)[crl].x);
  for (int p = 0; p < np_suf; ++p) M = fmaxf(M, a.ws_ml[base + p].x);
  if constexpr (kFused) M = fmaxf(M, suf->ml[crow].x);
  float lsum = 0.f, acc[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) acc[e] = 0.f;
  if constexpr (kFused) {
    const float2 ml = suf->ml[crow];
    const float wgt = pkv::fast_exp2(ml.x - M);
    lsum = ml.y * wgt;
#pragma unroll
    for (int e = 0; e < kE; ++e) acc[e] = wgt * suf->acc[crow][d0 + e];
  }
#pragma unroll
  for (int v = 0; v < kW; ++v) {
    const float* sv = state(v);
    const float2 ml = reinterpret_cast<const float2*>(sv + 16 * D)[crl];
    const float wgt = pkv::fast_exp2(ml.x - M);
    lsum = fmaf(wgt, ml.y, lsum);
#pragma unroll
    for (int e = 0; e < kE; ++e) acc[e] = fmaf(wgt, sv[crl * D + d0 + e], acc[e]);
  }
  for (int p = 0; p < np_suf; ++p) {
    const float2 ml = a.ws_ml[base + p];
    const float wgt = pkv::fast_exp2(ml.x - M);
    lsum = fmaf(wgt, ml.y, lsum);
    const float* src = a.ws_acc + (base + p) * D + d0;
#pragma unroll
    for (int e = 0; e < kE; ++e) acc[e] = fmaf(wgt, src[e], acc[e]);
  }
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  uint16_t* dst = a.out + cqh * D + d0;
#pragma unroll
  for (int e = 0; e < kE; e += 2)
    *reinterpret_cast<uint32_t*>(dst + e) = pkv::pack_bf16x2(acc[e] * inv, acc[e + 1] * inv);
}

// Suffix role: wave item i = (row group, part, KV head, sequence), row group
// fastest: query heads 16 rg .. 16 rg + 15 of the KV head's group, positions
// P + part * suf_tokens .. of the sequence's own (part, part + suf_parts, ...:
// a suffix longer than the grid was sized for is folded into the same
// piece).  A sequence without a shared prefix is attended whole by its part
// 0 items, which write the result.
template <int D, int Q>
__device__ void suffix_role(const SharedArgs& a, int64_t item, uint16_t* k_lds, uint16_t* v_lds,
                            float* s_lds) {
  const int lane = threadIdx.x & 63;
  const int rgs = (a.group + 15) / 16;
  const int rgi = static_cast<int>(item % rgs);
  const int part = static_cast<int>((item / rgs) % a.suf_parts);
  const int g = static_cast<int>((item / (int64_t(rgs) * a.suf_parts)) % a.num_kv_heads);
  const int64_t s64 = item / (int64_t(rgs) * a.suf_parts * a.num_kv_heads);
  if (s64 >= a.num_seqs) return;
  const int s = static_cast<int>(s64);
  const int L = clamp_len(a.seq_lens[s], a.len_cap);
  const int P = seq_prefix(a, s, L);
  const bool whole = P == 0;
  if (!whole && a.fused) return;  // the prefix kernel walks this member's positions
  if (whole ? part > 0 : P + part * a.suf_tokens >= L) return;

  const int G = a.group;
  const int hh = 16 * rgi + (lane & 15);
  const bool row_ok = hh < G;
  const int64_t qh = int64_t(s) * a.num_q_heads + g * G + (row_ok ? hh : 0);
  const pkv::mfma::History hist{a.k_cache,      a.v_cache,     a.block_tables + int64_t(s) * a.max_blocks,
                                L,              g,             a.block_elems,
                                a.row_elems,    a.num_blocks,  a.block_shift,
                                a.num_kv_heads, a.v_scale,     a.k_scales,
                                a.v_scales};
  pkv::mfma::RowAcc<D> r;
  pkv::mfma::start(r);
  constexpr int kPD = shared_pd<Q>();
  if (whole) {
    pkv::mfma::attend<D, 1, kPD, Q, false, pkv::mfma::NoEmit, false, true>(
        hist, 0, L, a.q + qh * D, row_ok, L - 1, L - 1, a.scale_log2, k_lds, v_lds, r, s_lds);
    if (row_ok) pkv::mfma::store_row_bf16<D>(r, a.out + qh * D);
    return;
  }
  for (int t_lo = P + part * a.suf_tokens; t_lo < L; t_lo += a.suf_parts * a.suf_tokens)
    pkv::mfma::attend<D, 1, kPD, Q, false, pkv::mfma::NoEmit, false, true>(
        hist, t_lo, min(t_lo + a.suf_tokens, L), a.q + qh * D, row_ok, L - 1, L - 1,
        a.scale_log2, k_lds, v_lds, r, s_lds);
  if (!row_ok) return;
  const int64_t slot = qh * a.suf_parts + part;
  pkv::mfma::store_piece<D>(r, a.ws_acc + slot * D, a.ws_ml + slot);
}

// grid = pre_blocks, eight waves (one workgroup per CU by LDS).
template <int D, int Q>
__global__ void __launch_bounds__(64 * kSharedWaves)
__attribute__((amdgpu_waves_per_eu(2)))
attn_prefix_kernel(SharedArgs a) {
  __shared__ __align__(16) SharedLds<D, Q, kSharedWaves> lds;
  prefix_role<D, Q, false>(a, static_cast<int>(blockIdx.x), lds, nullptr);
}

// The same with the members' suffixes walked in the workgroup (kFused).
// grid = pre_blocks + whole_blocks: the workgroups past the prefix ones take
// the sequences that share nothing (suffix items of part 0, round robin over
// their waves; the others return at once), so one launch does the step.
template <int D, int Q>
__global__ void __launch_bounds__(64 * kSharedWaves)
__attribute__((amdgpu_waves_per_eu(2)))
attn_prefix_fused_kernel(SharedArgs a) {
  __shared__ __align__(16) SharedLds<D, Q, kSharedWaves> lds;
  __shared__ __align__(16) SuffixStates<D> suf;
  const int x = static_cast<int>(blockIdx.x);
  if (x < a.pre_blocks) {
    prefix_role<D, Q, true>(a, x, lds, &suf);
    return;
  }
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t items = int64_t(a.num_seqs) * a.num_kv_heads * ((a.group + 15) / 16);
  const int64_t stride = int64_t(gridDim.x - a.pre_blocks) * kSharedWaves;
  for (int64_t it = int64_t(x - a.pre_blocks) * kSharedWaves + w; it < items; it += stride)
    suffix_role<D, Q>(a, it, lds.k[w], lds.v[w], lds.s[w]);
}

// grid = suffix items, one wave each.
template <int D, int Q>
__global__ void __launch_bounds__(64)
attn_suffix_kernel(SharedArgs a) {
  __shared__ __align__(16) SharedLds<D, Q, 1> lds;
  suffix_role<D, Q>(a, int64_t(blockIdx.x), lds.k[0], lds.v[0], lds.s[0]);
}

int64_t round_up_to(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

struct SharedPlan {
  int row_blocks, pre_blocks;
  int fused;
  int suf_parts, suf_tokens;
  int64_t suf_blocks;
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
  // 32 (member, query head) rows per prefix workgroup
  pl->row_blocks = static_cast<int>((int64_t(mg) * G + kPrefixRows - 1) / kPrefixRows);
  const int seq_len = max_seq_len > 0 ? max_seq_len : 1;
  // Suffix partitions from the longest suffix (a hint: longer suffixes are
  // folded into the grid's pieces): short critical paths, about 4096 items.
  const int suf_len = max_suffix_len > 0 && max_suffix_len < seq_len ? max_suffix_len : seq_len;
  const int64_t suf_items = int64_t(num_seqs) * g->num_kv_heads;
  const int64_t want = suf_items >= 4096 ? 1 : (4096 + suf_items - 1) / (suf_items > 0 ? suf_items : 1);
  int64_t spt = round_up_to((suf_len + want - 1) / want, kKT);
  if (spt < 64) spt = 64;
  pl->suf_tokens = static_cast<int>(spt);
  pl->suf_parts = static_cast<int>((suf_len + spt - 1) / spt);
  // Suffixes no longer than kFusedSuffix (by the hint): the prefix kernel
  // walks its members' suffixes itself, and the suffix kernel only the
  // sequences that share nothing (whole, in part 0).
  pl->fused = max_suffix_len > 0 && max_suffix_len <= kFusedSuffix && max_group_size >= 2 &&
              max_prefix_len > 0;
  if (pl->fused) {
    pl->suf_parts = 1;
    pl->suf_tokens = static_cast<int>(round_up_to(seq_len, kKT));
  }
  const int64_t pre_blocks = int64_t(num_groups) * g->num_kv_heads * pl->row_blocks;
  const int64_t wave_items = int64_t(num_seqs) * g->num_kv_heads * pl->suf_parts * ((G + 15) / 16);
  pl->suf_blocks = wave_items;
  if (pre_blocks + pl->suf_blocks > 2147483647LL)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: too many work items", who);
  pl->pre_blocks = static_cast<int>(pre_blocks);
  const size_t slots = size_t(num_seqs) * num_q_heads * pl->suf_parts;
  pl->ws_ml_off = slots * g->head_dim * sizeof(float);
  pl->ws_bytes = pl->ws_ml_off + slots * sizeof(float2);
  return PKV_OK;
}

template <int D, int Q>
hipError_t launch_shared(const SharedPlan& pl, const SharedArgs& a, hipStream_t st) {
  if (a.fused) {
    // whole sequences: about 8 (sequence, KV head) items per wave
    const int64_t whole = (pl.suf_blocks + 8 * kSharedWaves - 1) / (8 * kSharedWaves);
    hipLaunchKernelGGL((attn_prefix_fused_kernel<D, Q>),
                       dim3(static_cast<uint32_t>(a.pre_blocks + whole)), dim3(64 * kSharedWaves), 0,
                       st, a);
    return hipSuccess;
  }
  if (pl.suf_blocks > 0)
    hipLaunchKernelGGL((attn_suffix_kernel<D, Q>), dim3(static_cast<uint32_t>(pl.suf_blocks)),
                       dim3(64), 0, st, a);
  if (a.pre_blocks > 0)
    hipLaunchKernelGGL((attn_prefix_kernel<D, Q>), dim3(static_cast<uint32_t>(a.pre_blocks)),
                       dim3(64 * kSharedWaves), 0, st, a);
  return hipSuccess;
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
  a.suf_parts = pl.suf_parts;
  a.row_blocks = pl.row_blocks;
  a.pre_blocks = a.max_prefix > 0 ? pl.pre_blocks : 0;
  a.suf_tokens = pl.suf_tokens;
  a.fused = pl.fused && a.pre_blocks > 0;
  a.scale_log2 = static_cast<float>(double(scale) * 1.4426950408889634 *
                                    (kind == pkv::mfma::kFp8 ? double(scales->k_scale) : 1.0));
  a.v_scale = kind == pkv::mfma::kFp8 ? scales->v_scale : 1.f;
  a.k_scales = kind == pkv::mfma::kInt8 ? scales->k_scales : nullptr;
  a.v_scales = kind == pkv::mfma::kInt8 ? scales->v_scales : nullptr;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (kind == pkv::mfma::kFp8)
    e = launch_shared<128, pkv::mfma::kFp8>(pl, a, st);
  else if (kind == pkv::mfma::kInt8)
    e = launch_shared<128, pkv::mfma::kInt8>(pl, a, st);
  else if (geom->head_dim == 128)
    e = launch_shared<128, pkv::mfma::kBf16>(pl, a, st);
  else
    e = launch_shared<64, pkv::mfma::kBf16>(pl, a, st);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess)
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
