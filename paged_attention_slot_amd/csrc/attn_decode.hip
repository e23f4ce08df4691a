// Block-table-driven decode attention for gfx950 (pkv_attention_decode).
//
// What is computed ([KVM §19.2.3] paged attention with block-wise online
// softmax and Fig. 19-5; [KVX §01] new-token attention equation; [KVX §02] and
// [KVX §03] grouped-query heads; page keys in include/pkv.h): for sequence s and
// query head h of KV group g = h / G,
//     out[s][h] = sum_t softmax_t(scale * q[s][h] . K_s[t]) V_s[t],  t < L_s,
// with position t stored in physical block block_tables[s][t / B] at offset
// t % B ([SLOT §locate]).
//
// How (MI355X design, not taken from the pages):
//  * A "stream" is the K/V history of one (sequence, KV head).  A wave walks a
//    stretch of it in tiles of 16 positions for GW query heads of the group, so
//    each K/V byte feeds all of those heads.  When the group has more heads than
//    one wave carries, sibling waves of one workgroup walk the same tiles (the
//    repeated reads hit that CU's L1 / the XCD's L2).
//  * Lanes form 8 sub-streams of 8 lanes: sub-stream r owns positions r and r+8
//    of each tile, lane c of it holds 16-byte chunks c, c+8, ... of those K and
//    V rows, so one load instruction reads 8 full 128-byte row segments.
//  * q.k: bf16 pairs through v_dot2_f32_bf16 (fp32 accumulate) and a sum over
//    the 8 lanes with three DPP adds.  Online softmax per sub-stream in log2
//    units; the reference m only moves when a tile's maximum exceeds it by more
//    than 8 (softmax does not depend on the reference, so the result is the
//    running-max form's).  At the end the sub-streams are merged with DPP
//    row_ror:8 and the gfx950 permlane16/permlane32 swaps.
//  * Tiles sit in a ring of P register buffers (P-1 tiles in flight while one is
//    consumed); block ids come from a VGPR cache of 64 table entries read with
//    v_readlane, so each load has a scalar base and a fixed lane offset.
//  * Balanced mode (default): a persistent grid of as many wave groups as the
//    GPU holds at once, followed by more workgroups.  All streams, sequence by
//    sequence, form one global sequence of tiles, cut into intervals: first
//    one equal static share per resident wave group (85 % of the tiles), then
//    small chunks, one per wave group of the workgroups that follow.  The
//    hardware dispatches those as resident workgroups retire, so CUs that
//    finish their shares early take more chunks.  An interval that covers a
//    whole stream writes the output; otherwise it writes a (reference, sum,
//    weighted sum) piece, and attn_merge_balanced_kernel combines the pieces
//    of each stream by log-sum-exp rescaling.  Equal shares alone do not finish
//    together: the SIMD issues memory instructions oldest wave first and XCDs
//    draw different bandwidth, so (a) a wave raises its priority (s_setprio) in
//    proportion to the part of its share still ahead of it, and (b) the
//    dispatched chunks absorb what still differs between CUs and XCDs.
//  * Partition mode (explicit partition_tokens, or batches past the balanced
//    limits): one work item per (sequence, partition, KV head); the partition
//    states are merged by attn_merge_kernel.
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>
#include <cstdlib>
#include <mutex>
#include <unordered_map>

#include "geom.h"
#include "lse_merge.h"
#include "mfma_attend.h"
#include "mfma_route.h"
#include "pkv_device.h"

namespace {

constexpr int kTile = 16;               // positions per tile (8 sub-streams x 2)
constexpr int kMaxWavesPerBlock = 8;    // workgroup <= 512 threads
constexpr float kRescaleSlack = 8.0f;   // log2 units before the reference moves
constexpr float kRefInit = -1e30f;      // reference of a sub-stream with no position yet
constexpr int kMaxBalancedSeqs = 4096;  // per-sequence prefix sums live in LDS
constexpr int kMaxWaveGroups = 8192;    // the workspace is sized for this many groups
constexpr int kDynamicPerMille = 150;   // balanced split: tiles handed out dynamically
constexpr int kMinChunkTiles = 4;       // smallest dynamic chunk
constexpr int kMaxChunks = 8192;        // the workspace is sized for this many chunks
// The matrix-core balanced split: at most this many static workgroups (one
// wave each; about 2048 are resident on 256 CUs), and so at most as many
// dynamic chunks (a chunk count never exceeds the static count).
constexpr int kMaxMatrixGroups = 3072;

enum Mode : int { kPartitionMode = 0, kBalancedMode = 1, kMatrixMode = 2, kMatrixBalancedMode = 3 };

struct AttnArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  void* out;
  float* ws_acc;            // rows of D floats (unnormalised weighted sums)
  float2* ws_ml;            // (reference, sum) per row of ws_acc
  int32_t* ws_span;         // balanced: first and last interval of each stream [N*H_kv][2]
  int64_t block_bytes;
  int32_t row_bytes;
  int32_t max_blocks;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;            // G = Hq / Hkv
  int32_t waves_per_group;  // waves sharing one KV head (G / heads per wave)
  int32_t waves_per_block;  // waves of one workgroup
  int32_t num_blocks;
  int32_t block_shift;
  int32_t len_cap;
  // partition mode
  int32_t waves_per_item;   // H_kv * waves_per_group
  int32_t part_tokens;
  int32_t num_parts;        // workspace rows per (sequence, query head)
  int32_t piece_tokens;     // positions per workspace row: part_tokens, or the
                            // matrix-core route's run (pkv::decode_runs)
  // balanced mode
  int32_t groups_per_block; // wave groups per workgroup
  int32_t num_groups;       // W: wave groups of the static (resident) part of the grid
  int32_t static_blocks;    // workgroups of the static part; the rest run dynamic chunks
  float scale_log2;
  // quantized caches: per-tensor scales (FP8) or fp32 scale pools
  // [num_blocks * block_size][num_kv_heads] (INT8)
  float k_scale, v_scale;
  const float* k_scales;
  const float* v_scales;
  // fused append (pkv_attention_decode_append), else null: the new token of
  // sequence s is k_new/v_new row s ([num_seqs][num_kv_heads][D]), stored to
  // slot new_slots[s] of the pools by the wave that attends it
  const void* k_new;
  const void* v_new;
  const int32_t* new_slots;
  void* k_dst;   // the pools again, writable (the appended rows' destination)
  void* v_dst;
  int32_t stream_kv;  // 1: non-temporal K/V loads; 0: cacheable (shared blocks)
  int32_t merge_lanes;  // balanced merge: piece lanes per (head, column)
  int32_t merge_heads;  // balanced merge: query heads per workgroup
};

// One-byte cache element types ([KVM §19.2.4], [PFX] "KV Cache 量化"): OCP e4m3
// codes with a per-tensor scale, and INT8 codes with one scale per (token, KV
// head).  Queries and outputs of these caches are bf16.
struct fp8_e4m3 { uint8_t bits; };
struct int8_code { int8_t bits; };
template <typename T> constexpr bool kQuant = sizeof(T) == 1;
template <typename T> constexpr bool kInt8 = std::is_same<T, int8_code>::value;
template <typename T> using OutT = typename std::conditional<kQuant<T>, uint16_t, T>::type;

template <typename T, int D>
struct Shape {
  static constexpr int kES = sizeof(T);
  static constexpr int kEPC = 16 / kES;        // elements per 16-byte chunk
  static constexpr int kCPR = D * kES / 16;    // chunks per row
  static constexpr int kCPL = kCPR / 8;        // chunks per lane
  static constexpr int kNE = kCPL * kEPC;      // elements per lane
  static_assert(kCPR % 8 == 0, "row must be a multiple of 8 chunks");
};

template <typename T, int D>
struct TileBuf {
  uint4 k[2][Shape<T, D>::kCPL];
  uint4 v[2][Shape<T, D>::kCPL];
  float ks[2], vs[2];  // INT8: scales of this lane's two positions
};

struct TileInfo {
  int start;      // first position of the tile
  int nvalid;     // valid positions in the tile (1..16)
};

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

// The wave's index in its workgroup, as a wave-uniform (scalar) value: every
// quantity derived from it (sequence, head, bounds, block addresses) then lives
// in SGPRs, and loops over tiles are uniform branches.
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
}

template <typename T>
__device__ __forceinline__ void unpack(const uint4& x, float (&f)[16 / sizeof(T)]) {
  if constexpr (sizeof(T) == 2) {
    f[0] = pkv::bf16lo(x.x); f[1] = pkv::bf16hi(x.x);
    f[2] = pkv::bf16lo(x.y); f[3] = pkv::bf16hi(x.y);
    f[4] = pkv::bf16lo(x.z); f[5] = pkv::bf16hi(x.z);
    f[6] = pkv::bf16lo(x.w); f[7] = pkv::bf16hi(x.w);
  } else {
    f[0] = __uint_as_float(x.x); f[1] = __uint_as_float(x.y);
    f[2] = __uint_as_float(x.z); f[3] = __uint_as_float(x.w);
  }
}

template <typename T>
__device__ __forceinline__ float dot_chunk(const uint4& q, const uint4& k, float acc) {
  if constexpr (sizeof(T) == 2) {
    acc = pkv::dot2_bf16(q.x, k.x, acc);
    acc = pkv::dot2_bf16(q.y, k.y, acc);
    acc = pkv::dot2_bf16(q.z, k.z, acc);
    acc = pkv::dot2_bf16(q.w, k.w, acc);
  } else {
    acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
    acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
    acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
    acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
  }
  return acc;
}

template <typename T>
__device__ __forceinline__ uint4 pack_chunk(const float* f) {
  uint4 o;
  if constexpr (sizeof(T) == 2) {
    o.x = pkv::pack_bf16x2(f[0], f[1]);
    o.y = pkv::pack_bf16x2(f[2], f[3]);
    o.z = pkv::pack_bf16x2(f[4], f[5]);
    o.w = pkv::pack_bf16x2(f[6], f[7]);
  } else {
    o.x = __float_as_uint(f[0]); o.y = __float_as_uint(f[1]);
    o.z = __float_as_uint(f[2]); o.w = __float_as_uint(f[3]);
  }
  return o;
}

// Wave issue priority 0..3 (s_setprio takes an immediate; lv is wave-uniform).
__device__ __forceinline__ void set_priority(int lv) {
  if (lv >= 3) __builtin_amdgcn_s_setprio(3);
  else if (lv == 2) __builtin_amdgcn_s_setprio(2);
  else if (lv == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// 16 one-byte codes -> 16 floats (exact): e4m3 through the gfx950 packed
// fp8 -> f32 conversion, INT8 by sign extension.
template <typename T>
__device__ __forceinline__ void decode16(const uint4& x, float (&f)[16]) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (kInt8<T>) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        f[4 * i + j] = static_cast<float>(static_cast<int8_t>((w[i] >> (8 * j)) & 0xFFu));
    } else {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), true);
      f[4 * i] = lo[0];
      f[4 * i + 1] = lo[1];
      f[4 * i + 2] = hi[0];
      f[4 * i + 3] = hi[1];
    }
  }
}

// Two floats that bf16 holds exactly -> one bf16 pair (lo in the low half).
__device__ __forceinline__ uint32_t bf16_pair_exact(float lo, float hi) {
  // the high halves of both words in one byte permute (v_perm_b32)
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// One wave's attention over a stretch [start, end) of one stream.  kAppend:
// the fused-append variant (pkv_attention_decode_append), bf16/f32 only.
// kStream: the K/V tiles are read with non-temporal loads (each byte read
// once per call); off for batches whose sequences share blocks and for
// groups split over sibling waves (which walk the same tiles), so the
// re-read blocks stay cacheable.
template <typename T, int D, int GW, int P, bool kAppend = false, bool kStream = true>
struct Wave {
  static_assert(!kAppend || !kQuant<T>, "the fused append takes bf16 or f32 pools");
  using S = Shape<T, D>;
  static constexpr int kCPL = S::kCPL, kEPC = S::kEPC, kNE = S::kNE;
  // Queries and outputs: the cache type, or bf16 for one-byte codes (lane c
  // then holds row elements 16c .. 16c+15, i.e. two bf16 chunks).
  static constexpr int kQES = kQuant<T> ? 2 : S::kES;
  static constexpr int kQC = kQuant<T> ? 2 : kCPL;

  const AttnArgs& a;
  int lane, r, c;
  const int32_t* trow;   // the sequence's block-table row
  int blk_last;          // last block index this stretch may read
  int tcache_base;       // first block index held in tcache
  int tcache;            // lane i: block id of index tcache_base + i
  int64_t head_off;      // byte offset of the KV head inside a pool row
  int blk[2];

  uint4 q[GW][kQC];
  int kvh_;              // the KV head (INT8 scale column)
  // Fused append: position newpos_ of this stretch is the new token, read
  // from the k_new/v_new row at new_row_off_ instead of the pools; the writer
  // wave also stores it to slot new_slot_.  newpos_ < 0: no new token here.
  int newpos_ = -1;
  bool writer_ = false;
  int new_slot_ = -1;
  int64_t new_row_off_ = 0;
  float m[GW], l[GW], acc[GW][kNE];
  float M[GW], lt[GW];   // after run(): merged reference and sum

  __device__ explicit Wave(const AttnArgs& args) : a(args) {
    lane = threadIdx.x & 63;
    r = lane >> 3;
    c = lane & 7;
  }

  // Physical block of position ``pos`` (uniform).  Ids out of the pool are
  // redirected to block 0: memory stays in bounds, the values read for them
  // are unspecified.
  __device__ __forceinline__ int block_id(int pos) {
    const int idx = pos >> a.block_shift;
    if (idx - tcache_base >= 64) {
      tcache_base = idx;
      tcache = (idx + lane <= blk_last) ? trow[idx + lane] : 0;
      // Wait for the reload here, in this rare branch; otherwise every
      // v_readlane below would wait for all loads in flight (tile prefetches
      // included), since the compiler cannot tell which path wrote tcache.
      asm volatile("" ::"v"(tcache));
    }
    const int b = __builtin_amdgcn_readlane(tcache, idx - tcache_base);
    return (b >= 0 && b < a.num_blocks) ? b : 0;
  }

  static __device__ __forceinline__ uint4 kv_load(const char* p) {
    if constexpr (kStream) return pkv::load_stream(p);
    else return *reinterpret_cast<const uint4*>(p);
  }

  __device__ __forceinline__ TileInfo prepare(int tile_start, int end) {
    TileInfo t;
    t.start = tile_start;
    t.nvalid = min(kTile, end - tile_start);
    blk[0] = block_id(tile_start);
    blk[1] = (a.block_shift < 4 && t.nvalid > 8) ? block_id(tile_start + 8) : blk[0];
    return t;
  }

  __device__ __forceinline__ void load(const TileInfo& t, TileBuf<T, D>& b) {
    const int bmask = (1 << a.block_shift) - 1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int pos = t.start + 8 * i;
      const int64_t off = int64_t(blk[i]) * a.block_bytes + int64_t(pos & bmask) * a.row_bytes +
                          head_off;
      const char* kb = static_cast<const char*>(a.k_cache) + off;
      const char* vb = static_cast<const char*>(a.v_cache) + off;
      const int lane_off = r * a.row_bytes + c * 16;
      bool plain = true;
      if constexpr (kAppend) {
        if (newpos_ >= pos && newpos_ < pos + 8) {  // uniform: the new token is in this half
          // its sub-stream's lanes read the new-token row, the others the pool
          const bool mine = pos + r == newpos_;
          const char* kl = mine ? static_cast<const char*>(a.k_new) + new_row_off_ + c * 16
                                : kb + lane_off;
          const char* vl = mine ? static_cast<const char*>(a.v_new) + new_row_off_ + c * 16
                                : vb + lane_off;
#pragma unroll
          for (int j = 0; j < kCPL; ++j) {
            b.k[i][j] = kv_load(kl + 128 * j);
            b.v[i][j] = kv_load(vl + 128 * j);
          }
          plain = false;
        }
      }
      if (plain) {
#pragma unroll
        for (int j = 0; j < kCPL; ++j) {
          b.k[i][j] = kv_load(kb + lane_off + 128 * j);
          b.v[i][j] = kv_load(vb + lane_off + 128 * j);
        }
      }
      if constexpr (kInt8<T>) {
        // scale of this lane's position (sub-stream r): slot * H_kv + head
        const int64_t si = (int64_t(blk[i]) * (bmask + 1) + (pos & bmask) + r) * a.num_kv_heads + kvh_;
        b.ks[i] = a.k_scales[si];
        b.vs[i] = a.v_scales[si];
      }
    }
  }

  // Fused append: the lanes holding the new token (its row, read from the
  // input into this tile buffer) store it to its slot (checked in run()).
  __device__ __forceinline__ void store_new(const TileInfo& t, const TileBuf<T, D>& b) {
    const int bmask = (1 << a.block_shift) - 1;
    const int64_t off = int64_t(new_slot_ >> a.block_shift) * a.block_bytes +
                        int64_t(new_slot_ & bmask) * a.row_bytes + head_off + c * 16;
    char* kd = static_cast<char*>(a.k_dst) + off;
    char* vd = static_cast<char*>(a.v_dst) + off;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (t.start + 8 * i + r == newpos_) {
#pragma unroll
        for (int j = 0; j < kCPL; ++j) {
          *reinterpret_cast<uint4*>(kd + 128 * j) = b.k[i][j];
          *reinterpret_cast<uint4*>(vd + 128 * j) = b.v[i][j];
        }
      }
    }
  }

  template <bool kMasked>
  __device__ __forceinline__ void consume(const TileInfo& t, const TileBuf<T, D>& b) {
    bool valid[2];
    valid[0] = r < t.nvalid;
    valid[1] = r + 8 < t.nvalid;

    float sc[2][GW];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (kQuant<T>) {
        // codes -> exact bf16 pairs, dotted with the bf16 query; the K scale
        // multiplies the score (per tensor for FP8, per position for INT8)
        uint32_t kp[8];
        if constexpr (kInt8<T>) {
          float kf[16];
          decode16<T>(b.k[i][0], kf);
#pragma unroll
          for (int w = 0; w < 8; ++w) kp[w] = bf16_pair_exact(kf[2 * w], kf[2 * w + 1]);
        } else {
          const uint32_t kw[4] = {b.k[i][0].x, b.k[i][0].y, b.k[i][0].z, b.k[i][0].w};
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            kp[2 * w] = pkv::fp8x2_to_bf16x2(kw[w], false);
            kp[2 * w + 1] = pkv::fp8x2_to_bf16x2(kw[w], true);
          }
        }
        const float ksc = kInt8<T> ? a.scale_log2 * b.ks[i] : a.scale_log2 * a.k_scale;
#pragma unroll
        for (int hh = 0; hh < GW; ++hh) {
          const uint32_t qw[8] = {q[hh][0].x, q[hh][0].y, q[hh][0].z, q[hh][0].w,
                                  q[hh][1].x, q[hh][1].y, q[hh][1].z, q[hh][1].w};
          float d = 0.f;
#pragma unroll
          for (int w = 0; w < 8; ++w) d = pkv::dot2_bf16(qw[w], kp[w], d);
          d = pkv::sum8(d) * ksc;
          if constexpr (kMasked) d = valid[i] ? d : -INFINITY;
          sc[i][hh] = d;
        }
      } else {
#pragma unroll
        for (int hh = 0; hh < GW; ++hh) {
          float d = 0.f;
#pragma unroll
          for (int j = 0; j < kCPL; ++j) d = dot_chunk<T>(q[hh][j], b.k[i][j], d);
          d = pkv::sum8(d) * a.scale_log2;
          if constexpr (kMasked) d = valid[i] ? d : -INFINITY;
          sc[i][hh] = d;
        }
      }
    }

    bool need = false;
    float cm[GW];
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
      cm[hh] = fmaxf(sc[0][hh], sc[1][hh]);
      need |= cm[hh] > m[hh] + kRescaleSlack;
    }
    if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
      for (int hh = 0; hh < GW; ++hh) {
        const float mn = cm[hh] > m[hh] + kRescaleSlack ? cm[hh] : m[hh];
        const float alpha = pkv::fast_exp2(m[hh] - mn);
        l[hh] *= alpha;
#pragma unroll
        for (int e = 0; e < kNE; ++e) acc[hh][e] *= alpha;
        m[hh] = mn;
      }
    }

    float p[2][GW];
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
      p[0][hh] = pkv::fast_exp2(sc[0][hh] - m[hh]);
      p[1][hh] = pkv::fast_exp2(sc[1][hh] - m[hh]);
      l[hh] += p[0][hh] + p[1][hh];
    }

#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float vf[kNE];
      if constexpr (kQuant<T>) {
        decode16<T>(b.v[i][0], vf);
        // the V scale rides on the weight p (the sum l keeps the bare p); a
        // masked position's weight is exactly 0 whatever its scale slot holds
        const float vsc = kInt8<T> ? b.vs[i] : a.v_scale;
#pragma unroll
        for (int hh = 0; hh < GW; ++hh) {
          p[i][hh] *= vsc;
          if constexpr (kMasked) p[i][hh] = valid[i] ? p[i][hh] : 0.f;
        }
      } else {
#pragma unroll
        for (int j = 0; j < kCPL; ++j) {
          float tmp[kEPC];
          unpack<T>(b.v[i][j], tmp);
#pragma unroll
          for (int e = 0; e < kEPC; ++e) vf[j * kEPC + e] = tmp[e];
        }
      }
      if constexpr (kMasked) {
        // A masked position may hold any bits (stale slot, foreign block):
        // zero it so that 0 * inf / NaN cannot reach the accumulator.
#pragma unroll
        for (int e = 0; e < kNE; ++e) vf[e] = valid[i] ? vf[e] : 0.f;
      }
#pragma unroll
      for (int hh = 0; hh < GW; ++hh) {
#pragma unroll
        for (int e = 0; e < kNE; ++e) acc[hh][e] = fmaf(p[i][hh], vf[e], acc[hh][e]);
      }
    }
  }

  // Issue-priority feedback (balanced mode): tiles of the wave's static share
  // still ahead at the start of this stretch, and the share's length; 0 = off.
  int prio_rem0 = 0, prio_len = 0;

  // Attention of query heads h0 .. h0+GW-1 of sequence s over positions
  // [start, end) of KV head kvh (start < end).  Leaves the merged state in M,
  // lt and acc (identical in every lane holding a given chunk).  newpos >= 0
  // (fused append, always end - 1): that position is the new token, and a
  // writer wave stores it to the pools.
  __device__ __forceinline__ void run(int s, int kvh, int h0, int start, int end, int newpos = -1,
                                      bool writer = false) {
    if constexpr (kAppend) {
      // a slot outside the pool is not written, so that position is then
      // read from the pool like any other
      newpos_ = -1;
      writer_ = false;
      if (newpos >= 0) {
        const int slot = a.new_slots[s];
        if (slot >= 0 && int64_t(slot) < (int64_t(a.num_blocks) << a.block_shift)) {
          newpos_ = newpos;
          writer_ = writer;
          new_slot_ = slot;
          new_row_off_ = (int64_t(s) * a.num_kv_heads + kvh) * (D * S::kES);
        }
      }
    }
    const char* q_base =
        static_cast<const char*>(a.q) + (int64_t(s) * a.num_q_heads + h0) * (D * kQES);
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
#pragma unroll
      for (int j = 0; j < kQC; ++j)
        q[hh][j] = *reinterpret_cast<const uint4*>(q_base + hh * D * kQES + q_chunk_off(j));
      m[hh] = kRefInit;
      l[hh] = 0.f;
#pragma unroll
      for (int e = 0; e < kNE; ++e) acc[hh][e] = 0.f;
    }

    trow = a.block_tables + int64_t(s) * a.max_blocks;
    blk_last = (end - 1) >> a.block_shift;
    const int blk_first = start >> a.block_shift;
    tcache_base = blk_first;
    tcache = (blk_first + lane <= blk_last) ? trow[blk_first + lane] : 0;
    asm volatile("" ::"v"(tcache));
    head_off = int64_t(kvh) * D * S::kES;
    kvh_ = kvh;

    // Ring of P register tile buffers, unrolled P times so each buffer keeps
    // its registers.  Tiles 0 .. ntiles-2 are full; the tail (the last <= P
    // tiles) runs the masked path.
    const int ntiles = (end - start + kTile - 1) / kTile;
    TileBuf<T, D> buf[P];
    TileInfo info[P];
#pragma unroll
    for (int k = 0; k < P; ++k) {
      if (k < ntiles) {
        info[k] = prepare(start + kTile * k, end);
        load(info[k], buf[k]);
      }
    }
    int t = 0;
    for (; t + P < ntiles; t += P) {
      if (prio_len > 0) set_priority(((prio_rem0 - t) * 4) / (prio_len + 1));
#pragma unroll
      for (int k = 0; k < P; ++k) {
        consume<false>(info[k], buf[k]);
        if (t + k + P < ntiles) {
          info[k] = prepare(start + kTile * (t + k + P), end);
          load(info[k], buf[k]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < P; ++k) {
      if (t + k < ntiles) {
        consume<true>(info[k], buf[k]);
        if constexpr (kAppend)
          if (writer_ && t + k == ntiles - 1) store_new(info[k], buf[k]);
      }
    }

    // Merge the 8 sub-streams (log-sum-exp rescale to the common reference).
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
      M[hh] = pkv::max_across_groups8(m[hh]);
      const float wt = pkv::fast_exp2(m[hh] - M[hh]);
      lt[hh] = pkv::sum_across_groups8(l[hh] * wt);
#pragma unroll
      for (int e = 0; e < kNE; ++e) acc[hh][e] = pkv::sum_across_groups8(acc[hh][e] * wt);
    }
  }

  // Byte offset, inside a query/output row, of this lane's j-th chunk, and
  // the row element of lane-local element e (the lane's elements in order).
  __device__ __forceinline__ int q_chunk_off(int j) const {
    return kQuant<T> ? 32 * c + 16 * j : (c + 8 * j) * 16;
  }
  __device__ __forceinline__ int elem_of(int e) const {
    return kQuant<T> ? 16 * c + e : (c + 8 * (e / kEPC)) * kEPC + e % kEPC;
  }

  // Normalised output rows of heads h0 .. h0+GW-1 (sub-stream 0 stores).
  __device__ __forceinline__ void write_out(int s, int h0) {
    if (r != 0) return;
    using O = OutT<T>;
    constexpr int kOE = 16 / sizeof(O);  // output elements per chunk
    char* out_base = static_cast<char*>(a.out) + (int64_t(s) * a.num_q_heads + h0) * (D * kQES);
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
      const float inv = 1.0f / lt[hh];
#pragma unroll
      for (int j = 0; j < kQC; ++j) {
        float f[kOE];
#pragma unroll
        for (int e = 0; e < kOE; ++e) f[e] = acc[hh][j * kOE + e] * inv;
        *reinterpret_cast<uint4*>(out_base + hh * D * kQES + q_chunk_off(j)) = pack_chunk<O>(f);
      }
    }
  }

  // Zero output rows (empty history).
  __device__ __forceinline__ void write_zero(int s, int h0) {
    if (r != 0) return;
    char* out_base = static_cast<char*>(a.out) + (int64_t(s) * a.num_q_heads + h0) * (D * kQES);
#pragma unroll
    for (int hh = 0; hh < GW; ++hh)
#pragma unroll
      for (int j = 0; j < kQC; ++j)
        *reinterpret_cast<uint4*>(out_base + hh * D * kQES + q_chunk_off(j)) =
            make_uint4(0, 0, 0, 0);
  }

  // Unnormalised state of head hh to workspace row row0 + hh * row_stride.
  __device__ __forceinline__ void write_piece(int64_t row0, int64_t row_stride) {
    if (r != 0) return;
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
      const int64_t row = row0 + hh * row_stride;
      float* dst = a.ws_acc + row * D;
#pragma unroll
      for (int e4 = 0; e4 < kNE; e4 += 4)
        *reinterpret_cast<float4*>(dst + elem_of(e4)) =
            make_float4(acc[hh][e4], acc[hh][e4 + 1], acc[hh][e4 + 2], acc[hh][e4 + 3]);
      if (c == 0) a.ws_ml[row] = make_float2(M[hh], lt[hh]);
    }
  }
};

// ---------------------------------------------------------------------------
// Partition mode: one wave per (sequence, partition, KV head, head subset).
// ---------------------------------------------------------------------------
template <typename T, int D, int GW, int P, bool kAppend, bool kStream>
__global__ void __launch_bounds__(64 * kMaxWavesPerBlock)
attn_partition_kernel(AttnArgs a) {
  // The waves of one (sequence, partition) are numbered consecutively and
  // packed into workgroups.
  const int wi = blockIdx.x * a.waves_per_block + wave_index();
  if (wi >= a.waves_per_item) return;
  const int kvh = wi / a.waves_per_group;
  const int sub = wi - kvh * a.waves_per_group;
  const int part = blockIdx.y;
  const int s = blockIdx.z;
  const int h0 = kvh * a.group + sub * GW;

  Wave<T, D, GW, P, kAppend, kStream> w(a);
  const int Lraw = a.seq_lens[s];
  const int L = clamp_len(Lraw, a.len_cap);
  const int start = part * a.part_tokens;
  if (start >= L) {
    // Empty history (L == 0): the output is zero.  With more than one
    // partition the merge kernel writes it instead.
    if (part == 0 && a.num_parts == 1) w.write_zero(s, h0);
    return;
  }
  const int end = min(start + a.part_tokens, L);
  const bool app = kAppend && end == L && L == Lraw;  // holds the new token
  w.run(s, kvh, h0, start, end, app ? L - 1 : -1, sub == 0);
  if (a.num_parts == 1) {
    w.write_out(s, h0);
  } else {
    const int64_t row0 = (int64_t(s) * a.num_q_heads + h0) * a.num_parts + part;
    w.write_piece(row0, a.num_parts);
  }
}

// ---------------------------------------------------------------------------
using pkv::kMergeThreads;
using pkv::merge_rows;

// Partition mode merge: one workgroup per (query head, sequence).
template <typename T, int D>
__global__ void __launch_bounds__(kMergeThreads)
attn_merge_kernel(AttnArgs a) {
  const int h = blockIdx.x, s = blockIdx.y;
  const int L = clamp_len(a.seq_lens[s], a.len_cap);
  const int np = (L + a.piece_tokens - 1) / a.piece_tokens;
  const int64_t row0 = (int64_t(s) * a.num_q_heads + h) * a.num_parts;
  char* dst = static_cast<char*>(a.out) + ((int64_t(s) * a.num_q_heads + h) * D) * sizeof(T);
  merge_rows<T, D>(a.ws_acc, a.ws_ml, np, row0, 1, dst);
}

// The append of pkv_attention_decode_append where the attention kernel does
// not fold it in (waves of three or more query heads, whose issue slots the
// attention already fills): one workgroup per sequence copies the new K and V
// rows to the slot, under the same conditions as the folded store (a slot in
// the pool, 1 <= L_s <= len_cap).
constexpr int kAppendThreads = 256;

__global__ void __launch_bounds__(kAppendThreads)
append_rows_kernel(const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
                   const int32_t* __restrict__ slots, const int32_t* __restrict__ seq_lens,
                   uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, int32_t row_chunks,
                   int64_t num_slots, int32_t len_cap) {
  const int s = blockIdx.x;
  const int L = seq_lens[s];
  const int slot = slots[s];
  if (L < 1 || L > len_cap || slot < 0 || slot >= num_slots) return;
  const int64_t src = int64_t(s) * row_chunks, dst = int64_t(slot) * row_chunks;
  for (int i = threadIdx.x; i < 2 * row_chunks; i += kAppendThreads) {
    if (i < row_chunks) k_cache[dst + i] = k_new[src + i];
    else v_cache[dst + i - row_chunks] = v_new[src + i - row_chunks];
  }
}

// ---------------------------------------------------------------------------
// Balanced mode.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int stream_tiles(const AttnArgs& a, int s) {
  return (clamp_len(a.seq_lens[s], a.len_cap) + kTile - 1) / kTile;
}

// Share of wave group w in a global order of T tiles cut into W shares:
// [floor(T*w/W), floor(T*(w+1)/W)).  With W <= T every share is non-empty.
__device__ __forceinline__ int64_t share_lo(int64_t T, int64_t w, int64_t W) { return T * w / W; }


// The balanced split's intervals over the global tile order (all streams,
// sequence by sequence, KV head by KV head): intervals 0 .. Ws-1 are the static
// shares of [0, S), intervals Ws .. Ws+K-1 the dynamic chunks of [S, T).
struct Intervals {
  int64_t T, S;
  int Ws, K;
  __device__ Intervals(int64_t total, int W) : T(total) {
    const int64_t dyn = total * kDynamicPerMille / 1000;
    S = total - dyn;
    Ws = static_cast<int>(S < W ? S : W);
    // one chunk per static group, of at least kMinChunkTiles tiles
    int64_t k = (dyn + kMinChunkTiles - 1) / kMinChunkTiles;
    if (k > W) k = W;
    K = static_cast<int>(k < kMaxChunks ? k : kMaxChunks);
  }
  // First tile of interval j (0 <= j <= Ws + K; lo(Ws) = S, lo(Ws + K) = T).
  __device__ int64_t lo(int j) const {
    return j <= Ws ? share_lo(S, j, Ws) : S + share_lo(T - S, j - Ws, K);
  }
};

__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

// Attention over global tiles [lo, hi) of interval `iv`, stream by stream.
template <typename T, int D, int GW, int P, bool kAppend, bool kStream>
__device__ __forceinline__ void run_interval(Wave<T, D, GW, P, kAppend, kStream>& w,
                                             const AttnArgs& a,
                                             const int32_t* base, int64_t lo, int64_t hi, int iv,
                                             int sub) {
  const int N = a.num_seqs, Hkv = a.num_kv_heads;
  int64_t cur = lo;
  while (cur < hi) {
    // The sequence holding global tile `cur`: the largest s with base[s] <= cur.
    int lo_s = 0, hi_s = N - 1;
    while (lo_s < hi_s) {
      const int mid = (lo_s + hi_s + 1) >> 1;
      if (base[mid] <= cur) lo_s = mid;
      else hi_s = mid - 1;
    }
    const int s = lo_s;
    const int nt = (base[s + 1] - base[s]) / Hkv;
    const int rel = static_cast<int>(cur - base[s]);
    const int kvh = rel / nt;
    const int t0 = rel - kvh * nt;
    const int seg = static_cast<int>(min(hi - cur, int64_t(nt - t0)));
    const int Lraw = a.seq_lens[s];
    const int L = clamp_len(Lraw, a.len_cap);
    const int h0 = kvh * a.group + sub * GW;
    // the stream's last tile holds the new token (fused append)
    const bool app = kAppend && t0 + seg == nt && L == Lraw;
    w.run(s, kvh, h0, t0 * kTile, min((t0 + seg) * kTile, L), app ? L - 1 : -1, sub == 0);
    // the stream's first and last intervals, for the merge
    const int64_t ks = int64_t(s) * Hkv + kvh;
    if (sub == 0 && w.lane == 0) {
      if (t0 == 0) a.ws_span[2 * ks] = iv;
      if (t0 + seg == nt) a.ws_span[2 * ks + 1] = iv;
    }
    if (t0 == 0 && seg == nt) {
      w.write_out(s, h0);  // the whole stream in one interval
    } else {
      // piece of stream k from interval iv -> row group (k + iv): unique,
      // since streams and intervals are both contiguous and in the same order.
      const int64_t k = int64_t(s) * Hkv + kvh;
      w.write_piece((k + iv) * a.group + sub * GW, 1);
    }
    if (w.prio_len > 0) w.prio_rem0 -= seg;
    cur += seg;
  }
}

template <typename T, int D, int GW, int P, bool kAppend, bool kStream>
__global__ void __launch_bounds__(64 * kMaxWavesPerBlock)
attn_balanced_kernel(AttnArgs a) {
  __shared__ int32_t base[kMaxBalancedSeqs + 1];
  __shared__ int32_t wave_tot[kMaxWavesPerBlock];
  const int N = a.num_seqs, Hkv = a.num_kv_heads;
  const int tid = threadIdx.x, nth = blockDim.x, lane = tid & 63, wv = wave_index();

  // base[s] = sum over s' < s of H_kv * tiles(s'): every thread sums a
  // contiguous run of sequences, then a block-wide exclusive scan.
  const int per = (N + nth - 1) / nth;
  const int s0 = tid * per;
  int tsum = 0;
  for (int i = 0; i < per; ++i)
    if (s0 + i < N) tsum += Hkv * stream_tiles(a, s0 + i);
  const int incl = wave_incl_scan(tsum);
  if (lane == 63) wave_tot[wv] = incl;
  __syncthreads();
  int off = 0, total = 0;
  for (int k = 0; k < (nth >> 6); ++k) {
    off += k < wv ? wave_tot[k] : 0;
    total += wave_tot[k];
  }
  int run = off + incl - tsum;
  for (int i = 0; i < per; ++i) {
    if (s0 + i < N) {
      base[s0 + i] = run;
      run += Hkv * stream_tiles(a, s0 + i);
    }
  }
  if (tid == 0) base[N] = total;
  __syncthreads();

  const int grp = wv / a.waves_per_group;
  const int sub = wv - grp * a.waves_per_group;
  if (grp >= a.groups_per_block || total == 0) return;
  const Intervals ivs(total, a.num_groups);
  Wave<T, D, GW, P, kAppend, kStream> w(a);
  if (static_cast<int>(blockIdx.x) < a.static_blocks) {
    const int gidx = blockIdx.x * a.groups_per_block + grp;
    if (gidx >= ivs.Ws) return;
    const int64_t lo = ivs.lo(gidx), hi = ivs.lo(gidx + 1);
    w.prio_len = static_cast<int>(hi - lo);
    w.prio_rem0 = w.prio_len;
    run_interval(w, a, base, lo, hi, gidx, sub);
    return;
  }
  const int j = (blockIdx.x - a.static_blocks) * a.groups_per_block + grp;
  if (j >= ivs.K) return;
  const int iv = ivs.Ws + j;
  run_interval(w, a, base, ivs.lo(iv), ivs.lo(iv + 1), iv, sub);
}

// Balanced mode merge: one workgroup per (stream, block of its query heads).
// Its threads are (piece lane pp, head, float4 column): after one round trip
// for the length and the stream's first and last interval (as the attention
// kernel recorded them), piece lane pp folds pieces pp, pp + P, ... of its
// head's rows, issuing the loads of kMergeBatch of them at once, so up to
// P * kMergeBatch pieces take one more round trip; the P partial states then
// meet in LDS and are combined in a fixed order.  Nothing to do when one
// interval held the whole stream (the attention kernel wrote the rows); zeros
// for an empty history.
constexpr int kMergeBalancedThreads = 256;
constexpr int kMergeBatch = 8;

// grid = (ceil(G / heads per block), num_seqs * H_kv)
template <typename T, int D>
__global__ void __launch_bounds__(kMergeBalancedThreads)
__attribute__((amdgpu_waves_per_eu(1, 4)))  // registers for a whole batch in flight
attn_merge_balanced_kernel(AttnArgs a) {
  constexpr int kQ = D / 4;  // float4 columns per row
  __shared__ float part[kMergeBalancedThreads][6];  // (reference, sum, 4 columns)
  const int G = a.group;
  const int HB = a.merge_heads;  // blockDim.x = HB * kQ * P <= 256
  const int cols = HB * kQ;
  const int P = a.merge_lanes;  // piece lanes: blockDim.x = cols * P <= 256
  const int tid = threadIdx.x;
  const int col = tid % cols, pp = tid / cols;
  const int hl = col / kQ, q = col % kQ;
  const int j = blockIdx.x * HB + hl;  // head within the group
  const int64_t k = blockIdx.y;        // stream: s * H_kv + g
  const int s = static_cast<int>(k / a.num_kv_heads);
  const int g = static_cast<int>(k - int64_t(s) * a.num_kv_heads);
  const bool live = pp < P && j < G;
  // the length and the record in one round trip (the record is stale, and
  // unused, for an empty history)
  const int Lraw = a.seq_lens[s];
  const int2 span = reinterpret_cast<const int2*>(a.ws_span)[k];
  asm volatile("" ::"v"(span.x), "v"(span.y));  // issued before the branch
  const int nt = (clamp_len(Lraw, a.len_cap) + kTile - 1) / kTile;
  char* dst = static_cast<char*>(a.out) +
              ((int64_t(s) * a.num_q_heads + g * G + j) * D + 4 * q) * sizeof(T);
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  float M = -INFINITY, lsum = 0.f;
  if (nt > 0) {  // uniform over the workgroup
    const int i0 = span.x, i1 = span.y;
    if (i0 == i1) return;  // the attention kernel wrote these rows
    const int n = i1 - i0 + 1;
    // row indices fit in 32 bits (the workspace holds fewer than 2^31 / D rows)
    const int row0 = static_cast<int>((k + i0) * G) + (j < G ? j : 0);
    const float4* acc4 = reinterpret_cast<const float4*>(a.ws_acc) + q;
    for (int p0 = pp; live && p0 < n; p0 += P * kMergeBatch) {
      // pieces past the last one re-read it and weigh 0
      float2 ml[kMergeBatch];
      float4 x[kMergeBatch];
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) {
        const int row = row0 + min(p0 + i * P, n - 1) * G;
        ml[i] = a.ws_ml[row];
        x[i] = acc4[row * kQ];
      }
      float Mn = M;
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) Mn = fmaxf(Mn, ml[i].x);
      const float al = M == -INFINITY ? 0.f : pkv::fast_exp2(M - Mn);
      lsum *= al;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] *= al;
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) {
        const float wgt = p0 + i * P < n ? pkv::fast_exp2(ml[i].x - Mn) : 0.f;
        lsum = fmaf(wgt, ml[i].y, lsum);
        o[0] = fmaf(wgt, x[i].x, o[0]);
        o[1] = fmaf(wgt, x[i].y, o[1]);
        o[2] = fmaf(wgt, x[i].z, o[2]);
        o[3] = fmaf(wgt, x[i].w, o[3]);
      }
      M = Mn;
    }
    if (P > 1) {
      part[tid][0] = M;
      part[tid][1] = lsum;
#pragma unroll
      for (int e = 0; e < 4; ++e) part[tid][2 + e] = o[e];
      __syncthreads();
      if (pp != 0) return;
      // lane 0's state rescaled with the others, lanes in order
      float Mt = M;
      for (int r = 1; r < P; ++r) Mt = fmaxf(Mt, part[r * cols + col][0]);
      const float w0 = M == -INFINITY ? 0.f : pkv::fast_exp2(M - Mt);
      lsum *= w0;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] *= w0;
      for (int r = 1; r < P; ++r) {
        const float* pr = part[r * cols + col];
        const float wr = pr[0] == -INFINITY ? 0.f : pkv::fast_exp2(pr[0] - Mt);
        lsum = fmaf(wr, pr[1], lsum);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = fmaf(wr, pr[2 + e], o[e]);
      }
    }
  } else if (pp != 0) {
    return;
  }
  if (j >= G) return;
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<uint2*>(dst) =
        make_uint2(pkv::pack_bf16x2(o[0] * inv, o[1] * inv), pkv::pack_bf16x2(o[2] * inv, o[3] * inv));
  } else {
    *reinterpret_cast<float4*>(dst) = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
  }
}

// ---------------------------------------------------------------------------
// Balanced split on the matrix cores: the balanced split's intervals over the
// batch's global order of cut units (32-position tiles, or partitions of
// partition_tokens positions when the caller gives one), each walked by a
// one-wave workgroup with the matrix-core pass of the multi-token kernel
// (pkv::mfma::attend): the G <= 16 query heads of a KV head are the rows of
// the 16-row products, so q.k and p.v run on the matrix cores and only the
// softmax stays on the vector units.  For one-byte codes the vector kernels
// are bound by instruction issue (decoding the codes, then a multiply-add per
// (element, position, head)), while here a 32-position tile of all G heads
// costs 24 matrix instructions and the softmax of one tile.  Pieces and
// records are the balanced split's, so attn_merge_balanced_kernel merges
// them.
// ---------------------------------------------------------------------------
// Cut units of a stream (a.part_tokens positions each, a multiple of 32).
__device__ __forceinline__ int stream_units(const AttnArgs& a, int s) {
  return (clamp_len(a.seq_lens[s], a.len_cap) + a.part_tokens - 1) / a.part_tokens;
}

// grid = static workgroups (the resident ones) + dynamic chunks, 64 threads;
// dynamic LDS: (num_seqs + 1) int32 prefix sums.  kAppend (bf16): the step's
// append folded in, as on the vector kernels: the wave walking a stream's last
// tile reads the newest position from the new-token rows and stores it to its
// slot.
template <int Q, bool kStream, bool kAppend = false>
__global__ void __launch_bounds__(64)
attn_mfma_balanced_kernel(AttnArgs a) {
  constexpr int D = 128;
  extern __shared__ int32_t base[];
  __shared__ __align__(16) uint16_t k_lds[pkv::mfma::k_lds_elems<D, 1>()];
  __shared__ __align__(16) uint16_t v_lds[pkv::mfma::v_lds_elems<D, 1>()];
  __shared__ float s_lds[pkv::mfma::s_lds_elems<Q, 1>()];
  const int N = a.num_seqs, Hkv = a.num_kv_heads;
  const int lane = threadIdx.x & 63;

  // base[s] = sum over s' < s of H_kv * tiles(s'): each lane sums a run of
  // sequences, then a wave scan.
  const int per = (N + 63) / 64;
  const int s0 = lane * per;
  int tsum = 0;
  for (int i = 0; i < per; ++i)
    if (s0 + i < N) tsum += Hkv * stream_units(a, s0 + i);
  const int incl = wave_incl_scan(tsum);
  const int total = __shfl(incl, 63, 64);
  int run = incl - tsum;
  for (int i = 0; i < per; ++i) {
    if (s0 + i < N) {
      base[s0 + i] = run;
      run += Hkv * stream_units(a, s0 + i);
    }
  }
  if (lane == 0) base[N] = total;
  __syncthreads();
  if (total == 0) return;
  const Intervals ivs(total, a.num_groups);
  int iv;
  if (static_cast<int>(blockIdx.x) < a.static_blocks) {
    // Workgroups go to the 8 XCDs round robin (workgroup b to XCD b % 8);
    // each XCD takes a contiguous eighth of the static intervals, so the
    // KV heads of one sequence (consecutive streams) run side by side on one
    // XCD: the INT8 scales, [slot][KV head] with one 32-byte sector per slot,
    // then reach HBM once per slot instead of once per head.
    const int B = a.static_blocks, b = blockIdx.x;
    const int c = b & 7, q8 = B >> 3, r8 = B & 7;
    iv = c * q8 + min(c, r8) + (b >> 3);
    if (iv >= ivs.Ws) return;
  } else {
    const int j = blockIdx.x - a.static_blocks;
    if (j >= ivs.K) return;
    iv = ivs.Ws + j;
  }
  const int64_t lo = ivs.lo(iv), hi = ivs.lo(iv + 1);

  const int G = a.group;
  const int row = lane & 15;
  const bool row_ok = row < G;
  constexpr int kEB = Q == pkv::mfma::kBf16 ? 2 : 1;
  const float scale_log2 = Q == pkv::mfma::kFp8 ? a.scale_log2 * a.k_scale : a.scale_log2;
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  uint16_t* out = static_cast<uint16_t*>(a.out);
  int64_t cur = lo;
  while (cur < hi) {
    // the sequence holding global tile cur: the largest s with base[s] <= cur
    int lo_s = 0, hi_s = N - 1;
    while (lo_s < hi_s) {
      const int mid = (lo_s + hi_s + 1) >> 1;
      if (base[mid] <= cur) lo_s = mid;
      else hi_s = mid - 1;
    }
    const int s = lo_s;
    const int nt = (base[s + 1] - base[s]) / Hkv;
    const int rel = static_cast<int>(cur - base[s]);
    const int kvh = rel / nt;
    const int t0 = rel - kvh * nt;
    const int seg = static_cast<int>(min(hi - cur, int64_t(nt - t0)));
    const int Lraw = a.seq_lens[s];
    const int L = clamp_len(Lraw, a.len_cap);
    pkv::mfma::NewRow nr{nullptr, nullptr, nullptr, nullptr, -1};
    if constexpr (kAppend) {
      // the stream's last tile holds the new token; a slot outside the pool
      // is not written, and that position is then read from the pool
      const int slot = a.new_slots[s];
      if (t0 + seg == nt && L == Lraw && slot >= 0 &&
          int64_t(slot) < (int64_t(a.num_blocks) << a.block_shift)) {
        const int64_t row = (int64_t(s) * Hkv + kvh) * D;
        const int64_t dst = int64_t(slot) * (a.row_bytes / 2) + int64_t(kvh) * D;
        nr = {static_cast<const uint16_t*>(a.k_new) + row, static_cast<const uint16_t*>(a.v_new) + row,
              static_cast<uint16_t*>(a.k_dst) + dst, static_cast<uint16_t*>(a.v_dst) + dst, L - 1};
      }
    }
    const pkv::mfma::History hist{a.k_cache,      a.v_cache,    a.block_tables + int64_t(s) * a.max_blocks,
                                  L,              kvh,          a.block_bytes / kEB,
                                  a.row_bytes / kEB, a.num_blocks, a.block_shift,
                                  Hkv,            a.v_scale,    a.k_scales,
                                  a.v_scales};
    const int64_t qh = int64_t(s) * a.num_q_heads + kvh * G + (row_ok ? row : 0);
    pkv::mfma::RowAcc<D> r;
    pkv::mfma::start(r);
    // one-byte tiles are half the registers: two in flight ahead of the one
    // being computed, at the same occupancy
    constexpr int kPD = Q == pkv::mfma::kBf16 ? 1 : 2;
    const int U = a.part_tokens;
    pkv::mfma::attend<D, 1, kPD, Q, kStream, pkv::mfma::NoEmit, kAppend>(
        hist, t0 * U, min((t0 + seg) * U, L), q + qh * D, row_ok, L - 1, L - 1, scale_log2,
        k_lds, v_lds, r, s_lds, 0, pkv::mfma::NoEmit(), nr);
    const int64_t k = int64_t(s) * Hkv + kvh;
    if (lane == 0) {  // the stream's first and last intervals, for the merge
      if (t0 == 0) a.ws_span[2 * k] = iv;
      if (t0 + seg == nt) a.ws_span[2 * k + 1] = iv;
    }
    if (t0 == 0 && seg == nt) {
      if (row_ok) pkv::mfma::store_row_bf16<D>(r, out + qh * D);
    } else if (row_ok) {
      // row group (k + iv), as on the vector kernels' balanced split
      const int64_t prow = (k + iv) * G + row;
      pkv::mfma::store_piece<D>(r, a.ws_acc + prow * D, a.ws_ml + prow);
    }
    cur += seg;
  }
}

// ---------------------------------------------------------------------------
// Host side: planning, validation, dispatch.
// ---------------------------------------------------------------------------

// Tuning knobs (pkv_set_tuning in include/pkv.h; the environment is read once
// per process).  0 = the heuristic.
int knob_heads_per_wave() { return pkv::tuning(pkv::kKnobHeadsPerWave); }
int knob_prefetch() { return pkv::tuning(pkv::kKnobPrefetch); }
// 1 partitions, 2 balanced, 3 matrix cores
int knob_mode() { return pkv::tuning(pkv::kKnobMode); }
int knob_append() { return pkv::tuning(pkv::kKnobAppend); }  // 1 copy kernel, 2 folded
int knob_waves_per_block() { return pkv::tuning(pkv::kKnobWavesPerBlock); }

// Query heads per wave: the largest of 4, 3, 2, 1 dividing the group size that
// fits the register file without spilling (fp32 rows of 128 hold twice the
// registers of bf16 ones: one head per wave).
int heads_per_wave(int G, int dtype, int head_dim) {
  int cap = (dtype == PKV_F32 && head_dim == 128) ? 1 : 4;
  if (const int k = knob_heads_per_wave()) cap = k < cap ? k : cap;
  for (int gw : {4, 3, 2, 1})
    if (gw <= cap && G % gw == 0) return gw;
  return 1;
}

// Deepest register ring that fits without spilling at head_dim 128 (bf16):
// four tiles for one head per wave, three for two, two beyond.
template <int GW>
constexpr int max_prefetch() { return GW >= 3 ? 2 : (GW == 2 ? 3 : 4); }

// Tiles per wave in the register ring.  Two (one in flight while one is
// consumed) measured best with the balanced split; fixed partitions with few
// heads per wave gain a little from three.
int prefetch_depth(int gw, int dtype, bool balanced) {
  if (dtype == PKV_F32) return 2;
  // one-byte codes: half-size tiles, so up to 4 fit beside any head count
  const int cap = pkv::is_quant(dtype) ? 4 : (gw >= 3 ? 2 : (gw == 2 ? 3 : 4));
  int p = (!balanced && gw <= 2) ? 3 : 2;
  if (pkv::is_quant(dtype) && balanced && gw >= 4) p = 4;  // measured: 3 % on 4-head waves
  if (const int k = knob_prefetch()) p = k;
  return p < cap ? p : cap;
}

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Default split-KV partition of partition mode: 256 positions up to 4096-long
// contexts, 512 beyond; no split when one partition covers the longest one.
int auto_partition(int32_t max_seq_len, int32_t block_size) {
  const int unit = block_size > kTile ? block_size : kTile;
  int64_t t = max_seq_len <= 4096 ? 256 : 512;
  t = round_up(t, unit);
  if (max_seq_len <= t) return static_cast<int>(round_up(max_seq_len > 0 ? max_seq_len : 1, unit));
  return static_cast<int>(t);
}

struct Plan {
  int mode;
  int gw, prefetch, waves_per_group, waves_per_block;
  int len_cap;
  // partition mode
  int waves_per_item, blocks_per_item, part_tokens, num_parts;
  // matrix mode: how runs of workgroups cut each history
  pkv::DecodeRuns runs;
  // balanced mode
  int groups_per_block;
  int64_t rows;  // workspace rows of D floats
  size_t ws_bytes, ws_ml_off, ws_span_off;
  int max_chunks;  // balanced: upper bound of the dynamic chunks
};

pkv_status make_plan(int32_t num_seqs, int32_t num_q_heads, int32_t max_seq_len,
                     int32_t max_blocks, int32_t partition_tokens, const pkv_geom* g,
                     const char* who, Plan* pl) {
  if (pkv_status st = pkv::check_geom(g, who)) return st;
  if (num_seqs < 0 || num_q_heads <= 0 || max_seq_len < 0 || max_blocks < 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: negative size", who);
  if (num_q_heads % g->num_kv_heads != 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: num_q_heads %d is not a multiple of num_kv_heads %d",
                     who, num_q_heads, g->num_kv_heads);
  if (pkv::is_quant(g->dtype) && g->head_dim != 128)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "%s: head_dim %d (quantized caches: 128)", who,
                     g->head_dim);
  if (g->head_dim != 64 && g->head_dim != 128)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "%s: head_dim %d (built: 64, 128)", who, g->head_dim);
  if (g->block_size < 8)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "%s: block_size %d < 8", who, g->block_size);
  const int G = num_q_heads / g->num_kv_heads;
  if (G > 64) return pkv::fail(PKV_ERR_UNSUPPORTED, "%s: more than 64 query heads per group", who);
  if (num_seqs > 65535) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: more than 65535 sequences", who);
  if (partition_tokens < 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: partition_tokens < 0", who);
  if (partition_tokens > 0 && (partition_tokens % kTile != 0 || partition_tokens % g->block_size != 0))
    return pkv::fail(PKV_ERR_INVALID_ARG,
                     "%s: partition_tokens %d must be a multiple of 16 and of block_size %d", who,
                     partition_tokens, g->block_size);
  pl->gw = heads_per_wave(G, g->dtype, g->head_dim);
  pl->waves_per_group = G / pl->gw;
  const int64_t cap = int64_t(max_blocks) * g->block_size;
  pl->len_cap = static_cast<int>(max_seq_len < cap ? max_seq_len : cap);
  const int64_t stream_tiles_max = (int64_t(pl->len_cap) + kTile - 1) / kTile;
  const int wpg = pl->waves_per_group;
  const bool balanced_ok = partition_tokens == 0 && num_seqs <= kMaxBalancedSeqs &&
                           (wpg == 1 || wpg == 2 || wpg == 4 || wpg == 8) &&
                           int64_t(num_seqs) * g->num_kv_heads * stream_tiles_max < (int64_t(1) << 31);
  const int km = knob_mode();
  // Groups of 8 or more query heads per KV head belong on the matrix cores:
  // the vector kernels are bound by instruction issue there (a wave carries
  // at most 4 heads), while the matrix-core pass does the q.k and p.v
  // products for 16 heads at once and keeps only the softmax on the vector
  // units (the fixed-partition route below takes those the balanced split
  // does not).
  const bool matrix_ok = g->head_dim == 128 && (g->dtype == PKV_BF16 || pkv::is_quant(g->dtype)) &&
                         partition_tokens % 32 == 0 && g->num_kv_heads <= 65535;
  // 2 to 16 query heads per KV head (head_dim 128, bf16 or one-byte codes,
  // automatic partitions): the balanced split on the matrix cores.  For
  // one-byte codes the vector kernels are issue-bound decoding the codes; for
  // bf16 the matrix cores match them on unshared batches (the llama3-8b
  // layer: 718 against 720 us, the qwen layer: 91.7 against 95.4 us) and beat
  // them where blocks are shared (the shared-prefix config: 153.5 against
  // 177.0 us) and on long histories with 8 heads per group (the 70b layer:
  // 334 against 360 us on the fixed-partition matrix route).  The cut unit
  // stays one tile: partitions given by the caller take the fixed-partition
  // routes.
  const int unit = 32;
  const int64_t units_max = (int64_t(pl->len_cap) + unit - 1) / unit;
  const bool mbal_ok = matrix_ok && partition_tokens == 0 && num_seqs <= kMaxBalancedSeqs &&
                       G <= 16 && int64_t(num_seqs) * g->num_kv_heads * units_max < (int64_t(1) << 31);
  if (mbal_ok && (km == 4 || (km == 0 && G >= 2))) {
    pl->mode = kMatrixBalancedMode;
    pl->gw = G;
    pl->waves_per_group = 1;
    pl->prefetch = 0;
    pl->waves_per_block = 1;
    pl->waves_per_item = pl->blocks_per_item = 0;
    pl->groups_per_block = 1;
    pl->num_parts = 0;
    pl->part_tokens = unit;  // the cut unit
    pl->rows = (int64_t(num_seqs) * g->num_kv_heads + 2 * kMaxMatrixGroups) * G;
    const size_t acc = size_t(pl->rows) * g->head_dim * sizeof(float);
    pl->ws_ml_off = acc;
    pl->ws_span_off = acc + size_t(pl->rows) * sizeof(float2);
    pl->ws_bytes = pl->ws_span_off + round_up(int64_t(num_seqs) * g->num_kv_heads * 8, 256);
    const int64_t tmax = int64_t(num_seqs) * g->num_kv_heads * units_max;
    const int64_t kb = (tmax * kDynamicPerMille / 1000 + kMinChunkTiles - 1) / kMinChunkTiles;
    pl->max_chunks = static_cast<int>(kb < kMaxMatrixGroups ? kb : kMaxMatrixGroups);
    return PKV_OK;
  }
  if (matrix_ok && (km == 3 || (km == 0 && G >= 8))) {
    pl->mode = kMatrixMode;
    pl->prefetch = 0;
    pl->waves_per_block = pl->waves_per_item = pl->blocks_per_item = 0;
    pl->groups_per_block = 0;
    pl->max_chunks = 0;
    // automatic partitions: about 3072 (sequence, KV head, partition) items
    // of at least 256 positions
    const int64_t len = pl->len_cap > 0 ? pl->len_cap : 1;
    int64_t pt = partition_tokens;
    if (pt == 0) {
      const int64_t items = int64_t(num_seqs) * g->num_kv_heads;
      const int64_t parts = items >= 2048 ? 1 : (3072 + items - 1) / (items > 0 ? items : 1);
      pt = round_up((len + parts - 1) / parts, 32);
      if (pt < 256) pt = 256;
      if (pt > round_up(len, 32)) pt = round_up(len, 32);
    }
    const int64_t np = (len + pt - 1) / pt;
    if (np > 65535) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: more than 65535 partitions", who);
    pl->part_tokens = static_cast<int>(pt);
    pl->num_parts = static_cast<int>(np);
    pl->runs = pkv::decode_runs(num_seqs, g->num_kv_heads, pl->len_cap, pl->part_tokens,
                                pl->num_parts, 2048);
    if (pl->runs.runs > 1) {
      pl->rows = int64_t(num_seqs) * num_q_heads * pl->runs.runs;
      pl->ws_ml_off = size_t(pl->rows) * g->head_dim * sizeof(float);
      pl->ws_span_off = 0;
      pl->ws_bytes = pl->ws_ml_off + size_t(pl->rows) * sizeof(float2);
    } else {
      pl->rows = 0;
      pl->ws_ml_off = pl->ws_span_off = 0;
      pl->ws_bytes = 0;
    }
    return PKV_OK;
  }
  pl->mode = (balanced_ok && km != 1) ? kBalancedMode : kPartitionMode;
  pl->prefetch = prefetch_depth(pl->gw, g->dtype, pl->mode == kBalancedMode);

  if (pl->mode == kBalancedMode) {
    pl->waves_per_block = wpg <= 4 ? 4 : 8;
    pl->groups_per_block = pl->waves_per_block / wpg;
    // piece rows: (stream + interval) over N * H_kv streams and at most
    // kMaxWaveGroups static shares + kMaxChunks dynamic chunks
    pl->rows = (int64_t(num_seqs) * g->num_kv_heads + kMaxWaveGroups + kMaxChunks) * G;
    pl->num_parts = 0;
    pl->part_tokens = 0;
    const size_t acc = size_t(pl->rows) * g->head_dim * sizeof(float);
    pl->ws_ml_off = acc;
    pl->ws_span_off = acc + size_t(pl->rows) * sizeof(float2);
    pl->ws_bytes = pl->ws_span_off + round_up(int64_t(num_seqs) * g->num_kv_heads * 8, 256);
    // dynamic chunks: at most kMaxChunks, at least kMinChunkTiles tiles each,
    // out of kDynamicPerMille of all tiles (bounded here by max_seq_len)
    const int64_t tmax = int64_t(num_seqs) * g->num_kv_heads * stream_tiles_max;
    const int64_t kb = (tmax * kDynamicPerMille / 1000 + kMinChunkTiles - 1) / kMinChunkTiles;
    pl->max_chunks = static_cast<int>(kb < kMaxChunks ? kb : kMaxChunks);
    return PKV_OK;
  }

  pl->waves_per_item = g->num_kv_heads * wpg;
  int wpb = knob_waves_per_block();
  if (!wpb) wpb = wpg > 1 ? kMaxWavesPerBlock : 1;  // siblings of a group share a CU
  pl->waves_per_block = pl->waves_per_item < wpb ? pl->waves_per_item : wpb;
  pl->blocks_per_item = (pl->waves_per_item + pl->waves_per_block - 1) / pl->waves_per_block;
  pl->part_tokens = partition_tokens ? partition_tokens : auto_partition(pl->len_cap, g->block_size);
  const int64_t np =
      pl->len_cap == 0 ? 1 : (int64_t(pl->len_cap) + pl->part_tokens - 1) / pl->part_tokens;
  if (np > 65535) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: more than 65535 partitions", who);
  pl->num_parts = static_cast<int>(np);
  pl->groups_per_block = 0;
  pl->max_chunks = 0;
  if (pl->num_parts > 1) {
    pl->rows = int64_t(num_seqs) * num_q_heads * pl->num_parts;
    pl->ws_ml_off = size_t(pl->rows) * g->head_dim * sizeof(float);
    pl->ws_span_off = 0;
    pl->ws_bytes = pl->ws_ml_off + size_t(pl->rows) * sizeof(float2);
  } else {
    pl->rows = 0;
    pl->ws_ml_off = pl->ws_span_off = 0;
    pl->ws_bytes = 0;
  }
  return PKV_OK;
}

// Workgroups of ``kernel`` (at ``threads`` per group) one CU holds at once,
// times the CU count of the current device; cached per (device, kernel).
int resident_blocks(const void* kernel, int threads, size_t dyn_lds = 0) {
  static std::mutex mu;
  static std::unordered_map<uint64_t, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const uint64_t key = (uint64_t(reinterpret_cast<uintptr_t>(kernel)) << 8) ^ uint64_t(dev) ^
                       (uint64_t(dyn_lds) << 40);
  {
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, dyn_lds) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  const int v = per_cu * cus;
  std::lock_guard<std::mutex> lk(mu);
  cache[key] = v;
  return v;
}

// The balanced split's merge (both balanced kernels).  Piece lanes from the
// average pieces per stream (intervals plus streams over streams): about two
// batches' worth per lane group, so most streams take one round trip, without
// idle lanes on batches whose streams are cut into a few pieces only.
// a.num_groups is the static part's wave groups.
template <typename O, int D>
void launch_balanced_merge(const Plan& pl, AttnArgs& a, int num_seqs, hipStream_t st) {
  constexpr int kQ = D / 4;
  const int64_t streams = int64_t(num_seqs) * a.num_kv_heads;
  const int64_t chunks = pl.max_chunks < a.num_groups ? pl.max_chunks : a.num_groups;
  const int64_t avg = (a.num_groups + chunks + streams + streams - 1) / streams;
  // lanes first (few streams cut into many pieces: up to 256 / kQ lanes, the
  // heads then spread over more workgroups), then as many heads per
  // workgroup as the 256 threads hold
  int lanes = 1;
  while (lanes * kMergeBatch < 2 * avg && 2 * lanes * kQ <= kMergeBalancedThreads) lanes *= 2;
  int hb = kMergeBalancedThreads / (kQ * lanes);
  if (hb > a.group) hb = a.group;
  if (hb < 1) hb = 1;
  a.merge_lanes = lanes;
  a.merge_heads = hb;
  hipLaunchKernelGGL((attn_merge_balanced_kernel<O, D>),
                     dim3((a.group + hb - 1) / hb, num_seqs * a.num_kv_heads),
                     dim3(hb * kQ * lanes), 0, st, a);
}

// The matrix-core balanced kernel of a cache kind, streaming or cacheable
// K/V loads, with the append folded in (bf16 only) or not.
template <int Q, bool kStream, bool kAppend>
const void* mbal_ptr() {
  return reinterpret_cast<const void*>(&attn_mfma_balanced_kernel<Q, kStream, kAppend>);
}

const void* mfma_balanced_kernel_of(int kind, bool stream, bool append) {
  using pkv::mfma::kBf16;
  using pkv::mfma::kFp8;
  if (kind == kFp8) return stream ? mbal_ptr<kFp8, true, false>() : mbal_ptr<kFp8, false, false>();
  if (kind == pkv::mfma::kInt8)
    return stream ? mbal_ptr<pkv::mfma::kInt8, true, false>() : mbal_ptr<pkv::mfma::kInt8, false, false>();
  if (append) return stream ? mbal_ptr<kBf16, true, true>() : mbal_ptr<kBf16, false, true>();
  return stream ? mbal_ptr<kBf16, true, false>() : mbal_ptr<kBf16, false, false>();
}

template <int Q, bool kStream, bool kAppend>
void launch_mbal(int grid, size_t lds, hipStream_t st, const AttnArgs& a) {
  hipLaunchKernelGGL((attn_mfma_balanced_kernel<Q, kStream, kAppend>), dim3(grid), dim3(64), lds,
                     st, a);
}

void launch_mfma_balanced(int kind, bool stream, bool append, int grid, size_t lds,
                          hipStream_t st, const AttnArgs& a) {
  using pkv::mfma::kBf16;
  using pkv::mfma::kFp8;
  if (kind == kFp8) {
    if (stream) launch_mbal<kFp8, true, false>(grid, lds, st, a);
    else launch_mbal<kFp8, false, false>(grid, lds, st, a);
  } else if (kind == pkv::mfma::kInt8) {
    if (stream) launch_mbal<pkv::mfma::kInt8, true, false>(grid, lds, st, a);
    else launch_mbal<pkv::mfma::kInt8, false, false>(grid, lds, st, a);
  } else if (append) {
    if (stream) launch_mbal<kBf16, true, true>(grid, lds, st, a);
    else launch_mbal<kBf16, false, true>(grid, lds, st, a);
  } else {
    if (stream) launch_mbal<kBf16, true, false>(grid, lds, st, a);
    else launch_mbal<kBf16, false, false>(grid, lds, st, a);
  }
}

template <typename T, int D, int GW, int P, bool kAppend, bool kStream = true>
pkv_status launch_main(const Plan& pl, AttnArgs& a, int num_seqs, hipStream_t st) {
  if (pl.mode == kBalancedMode) {
    const void* k =
        reinterpret_cast<const void*>(&attn_balanced_kernel<T, D, GW, P, kAppend, kStream>);
    const int threads = 64 * pl.waves_per_block;
    int blocks = resident_blocks(k, threads);
    if (blocks <= 0)
      return pkv::fail(PKV_ERR_HIP, "pkv_attention_decode: occupancy query failed");
    const int max_blocks = kMaxWaveGroups / pl.groups_per_block;
    if (blocks > max_blocks) blocks = max_blocks;
    a.num_groups = blocks * pl.groups_per_block;
    a.static_blocks = blocks;
    const int chunks = pl.max_chunks < a.num_groups ? pl.max_chunks : a.num_groups;
    const int tail = (chunks + pl.groups_per_block - 1) / pl.groups_per_block;
    hipLaunchKernelGGL((attn_balanced_kernel<T, D, GW, P, kAppend, kStream>), dim3(blocks + tail),
                       dim3(threads), 0,
                       st, a);
  } else {
    const dim3 grid(pl.blocks_per_item, pl.num_parts, num_seqs);
    hipLaunchKernelGGL((attn_partition_kernel<T, D, GW, P, kAppend, kStream>), grid,
                       dim3(64 * pl.waves_per_block),
                       0, st, a);
  }
  if (hipError_t e = hipGetLastError())
    return pkv::fail(PKV_ERR_HIP, "pkv_attention_decode: launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

// Ring depths instantiated for (T, GW): 2 always; 3 and 4 for bf16 where
// max_prefetch allows, up to 4 for one-byte codes (prefetch_depth never asks
// for more).
template <typename T, int GW, int P>
constexpr bool ring_built() {
  return P == 2 || (sizeof(T) == 1 && P <= 4) || (sizeof(T) == 2 && P <= max_prefetch<GW>());
}

template <typename T, int D, int GW, bool kAppend>
pkv_status launch_main_p(const Plan& pl, AttnArgs& a, int num_seqs, hipStream_t st) {
  if constexpr (ring_built<T, GW, 4>())
    if (pl.prefetch == 4) return launch_main<T, D, GW, 4, kAppend>(pl, a, num_seqs, st);
  if constexpr (ring_built<T, GW, 3>())
    if (pl.prefetch == 3) return launch_main<T, D, GW, 3, kAppend>(pl, a, num_seqs, st);
  return launch_main<T, D, GW, 2, kAppend>(pl, a, num_seqs, st);
}

// The grid of the balanced merge depends on W, which the main launch fixes;
// a phase-2-only call recomputes it the same way.
template <typename T, int D, int GW, bool kAppend, bool kStream = true>
int balanced_groups(const Plan& pl) {
  const void* k =
      reinterpret_cast<const void*>(&attn_balanced_kernel<T, D, GW, 2, kAppend, kStream>);
  if constexpr (kStream && ring_built<T, GW, 4>())
    if (pl.prefetch == 4)
      k = reinterpret_cast<const void*>(&attn_balanced_kernel<T, D, GW, 4, kAppend, true>);
  if constexpr (kStream && ring_built<T, GW, 3>())
    if (pl.prefetch == 3)
      k = reinterpret_cast<const void*>(&attn_balanced_kernel<T, D, GW, 3, kAppend, true>);
  int blocks = resident_blocks(k, 64 * pl.waves_per_block);
  const int max_blocks = kMaxWaveGroups / pl.groups_per_block;
  if (blocks > max_blocks) blocks = max_blocks;
  return blocks * pl.groups_per_block;
}

template <typename T, int D, int GW>
pkv_status dispatch_gw(int phases, const Plan& pl, AttnArgs& a, int num_seqs, int num_q_heads,
                       hipStream_t st) {
  // the fused-append variant (bf16/f32 pools only) and the cacheable-load
  // variant (ring of 2, no fused append) have their own occupancy, so a
  // phase-2-only call derives W from the same variant as phase 1
  const bool append = !kQuant<T> && a.k_new != nullptr;
  const bool cached = !a.stream_kv;
  if (phases & 1) {
    pkv_status s;
    if (cached)
      s = launch_main<T, D, GW, 2, false, false>(pl, a, num_seqs, st);
    else if constexpr (!kQuant<T>)
      s = append ? launch_main_p<T, D, GW, true>(pl, a, num_seqs, st)
                 : launch_main_p<T, D, GW, false>(pl, a, num_seqs, st);
    else
      s = launch_main_p<T, D, GW, false>(pl, a, num_seqs, st);
    if (s) return s;
  } else if (pl.mode == kBalancedMode) {
    if (cached)
      a.num_groups = balanced_groups<T, D, GW, false, false>(pl);
    else if constexpr (!kQuant<T>)
      a.num_groups = append ? balanced_groups<T, D, GW, true>(pl)
                            : balanced_groups<T, D, GW, false>(pl);
    else
      a.num_groups = balanced_groups<T, D, GW, false>(pl);
    if (a.num_groups <= 0)
      return pkv::fail(PKV_ERR_HIP, "pkv_attention_decode: occupancy query failed");
  }
  if (phases & 2) {
    if (pl.mode == kBalancedMode) {
      launch_balanced_merge<OutT<T>, D>(pl, a, num_seqs, st);
    } else if (pl.num_parts > 1) {
      hipLaunchKernelGGL((attn_merge_kernel<OutT<T>, D>), dim3(num_q_heads, num_seqs),
                         dim3(kMergeThreads), 0, st, a);
    }
    if (hipError_t e = hipGetLastError())
      return pkv::fail(PKV_ERR_HIP, "pkv_attention_decode: merge launch failed: %s",
                       hipGetErrorString(e));
  }
  return PKV_OK;
}

template <typename T, int D>
pkv_status dispatch(int phases, const Plan& pl, AttnArgs& a, int num_seqs, int num_q_heads,
                    hipStream_t st) {
  if constexpr (sizeof(T) == 4 && D == 128) {  // heads_per_wave() gives 1 here
    return dispatch_gw<T, D, 1>(phases, pl, a, num_seqs, num_q_heads, st);
  } else {
    switch (pl.gw) {
      case 4: return dispatch_gw<T, D, 4>(phases, pl, a, num_seqs, num_q_heads, st);
      case 3: return dispatch_gw<T, D, 3>(phases, pl, a, num_seqs, num_q_heads, st);
      case 2: return dispatch_gw<T, D, 2>(phases, pl, a, num_seqs, num_q_heads, st);
      default: return dispatch_gw<T, D, 1>(phases, pl, a, num_seqs, num_q_heads, st);
    }
  }
}

}  // namespace

// Whether the vector kernels stream K/V with non-temporal loads: only when
// every cached byte is read once, i.e. no block is shared between sequences
// and one wave carries a KV head's whole query group.  Sibling waves of a
// split group walk the same tiles just apart; the second read is served by
// the L1 or the L2 only if the first left the lines cacheable (streaming
// them cost 15 % on groups of 8 split over two waves).
bool streams_kv(const Plan& pl, bool kv_shared) {
  return !kv_shared && pl.waves_per_group == 1;
}

// Whether pkv_attention_decode_append stores the new rows from inside the
// attention kernel: on the vector routes for waves of up to two query heads
// (with more the kernel is issue-bound and a copy launch costs less), and
// only where the kernel streams K/V: the cacheable-load kernels are built
// without the folded store.
bool folds_append(const Plan& pl, bool kv_shared) {
  if (pl.mode == kMatrixBalancedMode) return knob_append() != 1;  // bf16: folded unless asked
  if (!streams_kv(pl, kv_shared) || pl.mode == kMatrixMode) return false;
  const int ka = knob_append();
  return ka ? ka == 2 : pl.gw <= 2;
}

extern "C" {

int32_t pkv_attention_partition_tokens(int32_t num_seqs, int32_t num_q_heads,
                                       int32_t max_seq_len, const pkv_geom* geom) {
  Plan pl;
  const int32_t max_blocks =
      geom && geom->block_size > 0 ? (max_seq_len + geom->block_size - 1) / geom->block_size : 0;
  if (make_plan(num_seqs, num_q_heads, max_seq_len, max_blocks, 0, geom,
                "pkv_attention_partition_tokens", &pl) != PKV_OK)
    return 0;
  if (pl.mode == kBalancedMode || pl.mode == kMatrixBalancedMode)  // shares, not partitions
    return 0;
  return pl.part_tokens;
}

int32_t pkv_attention_piece_tokens(int32_t num_seqs, int32_t num_q_heads, int32_t max_seq_len,
                                   int32_t partition_tokens, const pkv_geom* geom) {
  Plan pl;
  const int32_t max_blocks =
      geom && geom->block_size > 0 ? (max_seq_len + geom->block_size - 1) / geom->block_size : 0;
  if (make_plan(num_seqs, num_q_heads, max_seq_len, max_blocks, partition_tokens, geom,
                "pkv_attention_piece_tokens", &pl) != PKV_OK)
    return 0;
  if (pl.mode == kBalancedMode || pl.mode == kMatrixBalancedMode) return 0;
  if (pl.mode == kMatrixMode) return pl.runs.run_tokens;
  return pl.part_tokens;
}

int32_t pkv_attention_decode_route(int32_t num_seqs, int32_t num_q_heads, int32_t max_seq_len,
                                   int32_t partition_tokens, const pkv_geom* geom) {
  Plan pl;
  const int32_t max_blocks =
      geom && geom->block_size > 0 ? (max_seq_len + geom->block_size - 1) / geom->block_size : 0;
  if (make_plan(num_seqs, num_q_heads, max_seq_len, max_blocks, partition_tokens, geom,
                "pkv_attention_decode_route", &pl) != PKV_OK)
    return -1;
  return pl.mode == kMatrixMode           ? PKV_ROUTE_MATRIX
         : pl.mode == kMatrixBalancedMode ? PKV_ROUTE_MATRIX_BALANCED
         : pl.mode == kBalancedMode       ? PKV_ROUTE_BALANCED
                                          : PKV_ROUTE_PARTITIONS;
}

int32_t pkv_attention_decode_append_folded(int32_t num_seqs, int32_t num_q_heads,
                                           int32_t max_seq_len, int32_t partition_tokens,
                                           int32_t kv_shared, const pkv_geom* geom) {
  Plan pl;
  const int32_t max_blocks =
      geom && geom->block_size > 0 ? (max_seq_len + geom->block_size - 1) / geom->block_size : 0;
  if (make_plan(num_seqs, num_q_heads, max_seq_len, max_blocks, partition_tokens, geom,
                "pkv_attention_decode_append_folded", &pl) != PKV_OK)
    return -1;
  if (pkv::is_quant(geom->dtype)) {
    pkv::fail(PKV_ERR_UNSUPPORTED,
              "pkv_attention_decode_append_folded: the fused append takes bf16 or f32 pools");
    return -1;
  }
  return folds_append(pl, kv_shared != 0) ? 1 : 0;
}

size_t pkv_attention_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t max_seq_len,
                                     int32_t partition_tokens, const pkv_geom* geom) {
  Plan pl;
  const int32_t max_blocks =
      geom && geom->block_size > 0 ? (max_seq_len + geom->block_size - 1) / geom->block_size : 0;
  if (make_plan(num_seqs, num_q_heads, max_seq_len, max_blocks, partition_tokens, geom,
                "pkv_attention_workspace_bytes", &pl) != PKV_OK)
    return static_cast<size_t>(-1);
  return pl.ws_bytes;
}

}  // extern "C"

namespace {

// New token of the fused append (pkv_attention_decode_append), else all null.
struct NewToken {
  bool on = false;
  const void* k = nullptr;
  const void* v = nullptr;
  const int32_t* slots = nullptr;
  void* k_cache = nullptr;  // the pools, writable
  void* v_cache = nullptr;
};

pkv_status attention_impl(const char* who, int32_t phases, const void* q, const void* k_cache,
                          const void* v_cache, const pkv_kv_scales* scales,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* seq_lens, float scale, void* out, int32_t num_seqs,
                          int32_t num_q_heads, int32_t max_seq_len, int32_t partition_tokens,
                          void* workspace, size_t workspace_bytes, const pkv_geom* geom,
                          void* stream, const NewToken& nt = NewToken()) {
  if ((phases & ~(3 | PKV_KV_SHARED)) || !(phases & 3))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: phases must be 1, 2 or 3 (optionally | PKV_KV_SHARED)",
                     who);
  const bool kv_shared = (phases & PKV_KV_SHARED) != 0;
  phases &= 3;
  Plan pl;
  if (pkv_status st = make_plan(num_seqs, num_q_heads, max_seq_len, max_blocks_per_seq,
                                partition_tokens, geom, who, &pl))
    return st;
  if (!std::isfinite(scale)) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: scale is not finite", who);
  const bool quant = pkv::is_quant(geom->dtype);
  const bool append = nt.on;
  if (append && quant)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "%s: quantized pools (write with pkv_write_quant)", who);
  if (quant) {
    if (!scales) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: null scales", who);
    if (geom->dtype == PKV_FP8_E4M3 &&
        !(std::isfinite(scales->k_scale) && scales->k_scale > 0.0f &&
          std::isfinite(scales->v_scale) && scales->v_scale > 0.0f))
      return pkv::fail(PKV_ERR_INVALID_ARG, "%s: FP8 scales must be finite and > 0", who);
    if (geom->dtype == PKV_INT8 && num_seqs > 0 &&
        (!scales->k_scales || !scales->v_scales ||
         (reinterpret_cast<uintptr_t>(scales->k_scales) & 3u) ||
         (reinterpret_cast<uintptr_t>(scales->v_scales) & 3u)))
      return pkv::fail(PKV_ERR_INVALID_ARG, "%s: INT8 scale pools null or misaligned", who);
  }
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !out)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: null pointer", who);
  if (append && (!nt.k || !nt.v || !nt.slots || !pkv::aligned16(nt.k) || !pkv::aligned16(nt.v) ||
                 (reinterpret_cast<uintptr_t>(nt.slots) & 3u)))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: new-token pointer null or misaligned", who);
  if (!pkv::aligned16(q) || !pkv::aligned16(out) || !pkv::aligned16(k_cache) ||
      !pkv::aligned16(v_cache) || (reinterpret_cast<uintptr_t>(block_tables) & 3u) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: misaligned pointer", who);
  if (pl.ws_bytes > 0) {
    if (!workspace || workspace_bytes < pl.ws_bytes)
      return pkv::fail(PKV_ERR_INVALID_ARG, "%s: workspace of %zu bytes needed, %zu given", who,
                       pl.ws_bytes, workspace ? workspace_bytes : size_t(0));
    if (!pkv::aligned16(workspace))
      return pkv::fail(PKV_ERR_INVALID_ARG, "%s: misaligned workspace", who);
  }
  const int es = pkv::elem_size(geom->dtype);
  AttnArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.out = out;
  char* ws = static_cast<char*>(workspace);
  a.ws_acc = pl.ws_bytes ? reinterpret_cast<float*>(ws) : nullptr;
  a.ws_ml = pl.ws_bytes ? reinterpret_cast<float2*>(ws + pl.ws_ml_off) : nullptr;
  a.ws_span = (pl.ws_bytes && (pl.mode == kBalancedMode || pl.mode == kMatrixBalancedMode))
                  ? reinterpret_cast<int32_t*>(ws + pl.ws_span_off)
                  : nullptr;
  a.row_bytes = geom->num_kv_heads * geom->head_dim * es;
  a.block_bytes = int64_t(geom->block_size) * a.row_bytes;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = geom->num_kv_heads;
  a.group = num_q_heads / geom->num_kv_heads;
  a.waves_per_group = pl.waves_per_group;
  a.waves_per_block = pl.waves_per_block;
  a.num_blocks = geom->num_blocks;
  a.block_shift = pkv::log2_exact(geom->block_size);
  a.len_cap = pl.len_cap;
  a.waves_per_item = pl.waves_per_item;
  a.part_tokens = pl.part_tokens;
  a.num_parts = pl.mode == kMatrixMode ? pl.runs.runs : pl.num_parts;
  a.piece_tokens = pl.mode == kMatrixMode ? pl.runs.run_tokens : pl.part_tokens;
  a.groups_per_block = pl.groups_per_block;
  a.num_groups = 0;
  a.static_blocks = 0;
  a.scale_log2 = static_cast<float>(double(scale) * 1.4426950408889634);
  a.k_scale = quant ? scales->k_scale : 1.0f;
  a.v_scale = quant ? scales->v_scale : 1.0f;
  a.k_scales = quant ? scales->k_scales : nullptr;
  a.v_scales = quant ? scales->v_scales : nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool fold = append && folds_append(pl, kv_shared);
  a.stream_kv = streams_kv(pl, kv_shared) ? 1 : 0;
  a.k_new = fold ? nt.k : nullptr;
  a.v_new = fold ? nt.v : nullptr;
  a.new_slots = fold ? nt.slots : nullptr;
  a.k_dst = fold ? nt.k_cache : nullptr;
  a.v_dst = fold ? nt.v_cache : nullptr;
  if (append && !fold && (phases & 1)) {
    hipLaunchKernelGGL(append_rows_kernel, dim3(num_seqs), dim3(kAppendThreads), 0, st,
                       static_cast<const uint4*>(nt.k), static_cast<const uint4*>(nt.v), nt.slots,
                       seq_lens, static_cast<uint4*>(nt.k_cache),
                       static_cast<uint4*>(nt.v_cache), a.row_bytes / 16,
                       int64_t(geom->num_blocks) * geom->block_size, pl.len_cap);
    if (hipError_t e = hipGetLastError())
      return pkv::fail(PKV_ERR_HIP, "%s: append launch failed: %s", who, hipGetErrorString(e));
  }
  if (pl.mode == kMatrixBalancedMode) {
    const int kind = geom->dtype == PKV_FP8_E4M3 ? pkv::mfma::kFp8
                     : (geom->dtype == PKV_INT8 ? pkv::mfma::kInt8 : pkv::mfma::kBf16);
    const size_t lds = size_t(num_seqs + 1) * sizeof(int32_t);
    const bool folded = a.k_new != nullptr;
    const void* kern = mfma_balanced_kernel_of(kind, a.stream_kv != 0, folded);
    int blocks = resident_blocks(kern, 64, lds);
    if (blocks <= 0)
      return pkv::fail(PKV_ERR_HIP, "%s: occupancy query failed", who);
    if (blocks > kMaxMatrixGroups) blocks = kMaxMatrixGroups;
    a.num_groups = blocks;
    a.static_blocks = blocks;
    if (phases & 1) {
      const int chunks = pl.max_chunks < a.num_groups ? pl.max_chunks : a.num_groups;
      launch_mfma_balanced(kind, a.stream_kv != 0, folded, blocks + chunks, lds, st, a);
    }
    if (phases & 2) launch_balanced_merge<uint16_t, 128>(pl, a, num_seqs, st);
    if (hipError_t e = hipGetLastError())
      return pkv::fail(PKV_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
    return PKV_OK;
  }
  if (pl.mode == kMatrixMode) {
    if (phases & 1) {
      const int kind = geom->dtype == PKV_FP8_E4M3 ? 1 : (geom->dtype == PKV_INT8 ? 2 : 0);
      if (pkv_status e = pkv::mfma_decode(q, k_cache, v_cache, kind, a.k_scale, a.v_scale,
                                          a.k_scales, a.v_scales, block_tables,
                                          max_blocks_per_seq, seq_lens, scale, out, num_seqs,
                                          num_q_heads, pl.len_cap, pl.part_tokens, pl.num_parts,
                                          pl.runs, a.ws_acc, a.ws_ml, !kv_shared, geom, st))
        return e;
    }
    if ((phases & 2) && pl.runs.runs > 1) {
      hipLaunchKernelGGL((attn_merge_kernel<uint16_t, 128>), dim3(num_q_heads, num_seqs),
                         dim3(kMergeThreads), 0, st, a);
      if (hipError_t e = hipGetLastError())
        return pkv::fail(PKV_ERR_HIP, "%s: merge launch failed: %s", who, hipGetErrorString(e));
    }
    return PKV_OK;
  }
  if (geom->dtype == PKV_FP8_E4M3)
    return dispatch<fp8_e4m3, 128>(phases, pl, a, num_seqs, num_q_heads, st);
  if (geom->dtype == PKV_INT8)
    return dispatch<int8_code, 128>(phases, pl, a, num_seqs, num_q_heads, st);
  if (geom->dtype == PKV_BF16) {
    return geom->head_dim == 128 ? dispatch<uint16_t, 128>(phases, pl, a, num_seqs, num_q_heads, st)
                                 : dispatch<uint16_t, 64>(phases, pl, a, num_seqs, num_q_heads, st);
  }
  return geom->head_dim == 128 ? dispatch<float, 128>(phases, pl, a, num_seqs, num_q_heads, st)
                               : dispatch<float, 64>(phases, pl, a, num_seqs, num_q_heads, st);
}

}  // namespace

extern "C" {

pkv_status pkv_attention_decode_phase(int32_t phases, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                      float scale, void* out, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t max_seq_len,
                                      int32_t partition_tokens, void* workspace,
                                      size_t workspace_bytes, const pkv_geom* geom,
                                      void* stream) {
  const char* who = "pkv_attention_decode";
  if (geom && pkv::is_quant(geom->dtype))
    return pkv::fail(PKV_ERR_INVALID_ARG,
                     "%s: quantized pools need scales (pkv_attention_decode_quant)", who);
  return attention_impl(who, phases, q, k_cache, v_cache, nullptr, block_tables,
                        max_blocks_per_seq, seq_lens, scale, out, num_seqs, num_q_heads,
                        max_seq_len, partition_tokens, workspace, workspace_bytes, geom, stream);
}

pkv_status pkv_attention_decode_quant(int32_t phases, const void* q, const void* k_cache,
                                      const void* v_cache, const pkv_kv_scales* scales,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* seq_lens, float scale, void* out,
                                      int32_t num_seqs, int32_t num_q_heads, int32_t max_seq_len,
                                      int32_t partition_tokens, void* workspace,
                                      size_t workspace_bytes, const pkv_geom* geom,
                                      void* stream) {
  const char* who = "pkv_attention_decode_quant";
  if (geom && !pkv::is_quant(geom->dtype))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: dtype %d is not a quantized cache type", who,
                     geom->dtype);
  return attention_impl(who, phases, q, k_cache, v_cache, scales, block_tables,
                        max_blocks_per_seq, seq_lens, scale, out, num_seqs, num_q_heads,
                        max_seq_len, partition_tokens, workspace, workspace_bytes, geom, stream);
}

pkv_status pkv_attention_decode_append(int32_t phases, const void* q, const void* k_new,
                                       const void* v_new, const int32_t* slot_mapping,
                                       void* k_cache, void* v_cache, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                       float scale, void* out, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t max_seq_len,
                                       int32_t partition_tokens, void* workspace,
                                       size_t workspace_bytes, const pkv_geom* geom,
                                       void* stream) {
  NewToken nt;
  nt.on = true;
  nt.k = k_new;
  nt.v = v_new;
  nt.slots = slot_mapping;
  nt.k_cache = k_cache;
  nt.v_cache = v_cache;
  return attention_impl("pkv_attention_decode_append", phases, q, k_cache, v_cache, nullptr,
                        block_tables, max_blocks_per_seq, seq_lens, scale, out, num_seqs,
                        num_q_heads, max_seq_len, partition_tokens, workspace, workspace_bytes,
                        geom, stream, nt);
}

pkv_status pkv_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* seq_lens, float scale, void* out,
                                int32_t num_seqs, int32_t num_q_heads, int32_t max_seq_len,
                                int32_t partition_tokens, void* workspace,
                                size_t workspace_bytes, const pkv_geom* geom, void* stream) {
  return pkv_attention_decode_phase(3, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                                    seq_lens, scale, out, num_seqs, num_q_heads, max_seq_len,
                                    partition_tokens, workspace, workspace_bytes, geom, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// pkv_attention_decode_noalloc: pkv_attention_decode with its workspace in a
// file-scope device array instead of a caller's buffer, for callers that
// cannot allocate.  Each device holds its own copy of the array from module
// load to process end.  In host code ``scratch`` names a host-side stand-in,
// not device memory: the kernels get the array's device address, looked up
// once per device with that device current.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The device address of ``scratch`` on the current device, looked up on the
// first call there.
pkv_status scratch_on_current_device(const char* who, void** out) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev))
    return pkv::fail(PKV_ERR_HIP, "%s: hipGetDevice failed: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "%s: device %d beyond the %d the scratch table holds",
                     who, dev, kMaxScratchDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)))
      return pkv::fail(PKV_ERR_HIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s",
                       who, dev, hipGetErrorString(e));
    if (!ptr)
      return pkv::fail(PKV_ERR_HIP, "%s: no device address for scratch on device %d", who, dev);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_attention_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* seq_lens, float scale, void* out,
                                        int32_t num_seqs, int32_t num_q_heads,
                                        int32_t max_seq_len, int32_t partition_tokens,
                                        const pkv_geom* geom, void* stream) {
  const char* who = "pkv_attention_decode_noalloc";
  if (geom && pkv::is_quant(geom->dtype))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: quantized pools are not taken here", who);
  Plan pl;
  if (pkv_status st = make_plan(num_seqs, num_q_heads, max_seq_len, max_blocks_per_seq,
                                partition_tokens, geom, who, &pl))
    return st;
  if (pl.ws_bytes > kScratchBytes)
    return pkv::fail(PKV_ERR_INVALID_ARG,
                     "%s: these sizes need %zu bytes of workspace, beyond the %zu bytes of the "
                     "library's scratch (use pkv_attention_decode with a workspace)",
                     who, pl.ws_bytes, kScratchBytes);
  void* ws = nullptr;
  if (pl.ws_bytes > 0 && num_seqs > 0)
    if (pkv_status st = scratch_on_current_device(who, &ws)) return st;
  return attention_impl(who, 3, q, k_cache, v_cache, nullptr, block_tables, max_blocks_per_seq,
                        seq_lens, scale, out, num_seqs, num_q_heads, max_seq_len,
                        partition_tokens, ws, ws ? kScratchBytes : 0, geom, stream);
}

}  // extern "C"
