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
//  * Work item = (sequence, KV head, partition of the sequence's positions).
//    One wave handles GW query heads of the group against that KV head, so
//    each K/V byte feeds all of those heads; when the group is larger than GW,
//    the group's head subsets run as sibling waves of one workgroup (same CU,
//    so the duplicate K/V reads hit the CU's L1 / the XCD's L2).
//  * A wave consumes tiles of 16 positions.  Lanes form 8 "streams" of 8
//    lanes; stream r owns positions r and r+8 of each tile, and lane c of a
//    stream holds the 16-byte chunks c, c+8, ... of those K and V rows.  Each
//    load instruction therefore reads 8 full 128-byte row segments; rows of
//    one block and KV head are 16 B-chunk contiguous, blocks are reached
//    through the table (contiguous within a block, indirect across blocks).
//  * q.k: bf16 pairs through v_dot2_f32_bf16 (fp32 accumulate), then a sum over
//    the 8 lanes of the stream with three DPP adds.
//  * Online softmax per stream, in log2 units (scale folded with log2 e):
//    the running reference m is only raised when a tile's maximum exceeds it by
//    more than 8, so the accumulator is rescaled rarely; since softmax does not
//    depend on the reference, the result equals the running-max form.
//  * At the end the 8 streams are merged with DPP row_ror:8 and the gfx950
//    permlane16/permlane32 swaps (log-sum-exp rescale), then either the
//    normalised output is written or, with split-KV, the partition's
//    (reference, sum, weighted sum) go to the workspace for attn_merge_kernel.
//  * Tiles are double-buffered in registers (loads of tile t+1 are in flight
//    while tile t is computed); the partition's block ids are fetched once per
//    64 blocks into a VGPR and read with v_readlane, so every K/V load has a
//    scalar base and a loop-invariant per-lane offset.
#include <hip/hip_runtime.h>

#include <cmath>

#include "geom.h"
#include "pkv_device.h"

namespace {

constexpr int kTile = 16;              // positions per tile (8 streams x 2)
constexpr int kMaxWavesPerBlock = 4;   // workgroup <= 256 threads
constexpr float kRescaleSlack = 8.0f;  // log2 units before the reference moves
constexpr float kRefInit = -1e30f;     // reference of a stream with no position yet

struct AttnArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  void* out;
  float* ws_acc;      // [N][Hq][P][D]
  float* ws_ml;       // [N][Hq][P][2] = (reference, sum)
  int64_t block_bytes;
  int32_t row_bytes;
  int32_t max_blocks;
  int32_t num_q_heads;
  int32_t group;      // G = Hq / Hkv
  int32_t waves_per_group;
  int32_t waves_per_block;
  int32_t blocks_per_group;
  int32_t num_blocks;
  int32_t block_shift;
  int32_t len_cap;
  int32_t part_tokens;
  int32_t num_parts;
  float scale_log2;
};

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
};

struct TileInfo {
  int start;      // first position of the tile
  int nvalid;     // valid positions in the tile (1..16)
  bool ok0, ok1;  // block of positions start+[0,8) / start+[8,16) is in the pool
};

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

template <typename T, int D, int GW>
struct Wave {
  using S = Shape<T, D>;
  static constexpr int kCPL = S::kCPL, kEPC = S::kEPC, kNE = S::kNE;

  const AttnArgs& a;
  int lane, r, c;
  const int32_t* trow;   // this sequence's block-table row
  int blk_last;          // last block index this work item may read
  int tcache_base;       // first block index held in tcache
  int tcache;            // lane i: block id of index tcache_base + i
  int64_t head_off;      // byte offset of this KV head inside a pool row

  uint4 q[GW][kCPL];
  float m[GW], l[GW], acc[GW][kNE];

  __device__ Wave(const AttnArgs& args) : a(args) {}

  __device__ __forceinline__ int block_id(int pos) {
    const int idx = pos >> a.block_shift;
    if (idx - tcache_base >= 64) {
      tcache_base = idx;
      tcache = (idx + lane <= blk_last) ? trow[idx + lane] : -1;
    }
    return __builtin_amdgcn_readlane(tcache, idx - tcache_base);
  }

  __device__ __forceinline__ TileInfo prepare(int tile_start, int end) {
    TileInfo t;
    t.start = tile_start;
    t.nvalid = min(kTile, end - tile_start);
    const int b0 = block_id(tile_start);
    t.ok0 = b0 >= 0 && b0 < a.num_blocks;
    int b1 = b0;
    t.ok1 = t.ok0;
    if (a.block_shift < 4 && t.nvalid > 8) {  // block_size 8: second block
      b1 = block_id(tile_start + 8);
      t.ok1 = b1 >= 0 && b1 < a.num_blocks;
    }
    blk[0] = t.ok0 ? b0 : 0;
    blk[1] = t.ok1 ? b1 : 0;
    return t;
  }
  int blk[2];

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
#pragma unroll
      for (int j = 0; j < kCPL; ++j) {
        b.k[i][j] = *reinterpret_cast<const uint4*>(kb + lane_off + 128 * j);
        b.v[i][j] = *reinterpret_cast<const uint4*>(vb + lane_off + 128 * j);
      }
    }
  }

  template <bool kMasked>
  __device__ __forceinline__ void consume(const TileInfo& t, const TileBuf<T, D>& b) {
    bool valid[2];
    valid[0] = r < t.nvalid && t.ok0;
    valid[1] = r + 8 < t.nvalid && t.ok1;

    float sc[2][GW];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
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
#pragma unroll
      for (int j = 0; j < kCPL; ++j) {
        float tmp[kEPC];
        unpack<T>(b.v[i][j], tmp);
#pragma unroll
        for (int e = 0; e < kEPC; ++e) vf[j * kEPC + e] = tmp[e];
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

  __device__ __forceinline__ void run_tile(const TileInfo& t, const TileBuf<T, D>& b) {
    if (t.nvalid == kTile && t.ok0 && t.ok1) consume<false>(t, b);
    else consume<true>(t, b);
  }
};

template <typename T, int D, int GW>
__global__ void __launch_bounds__(256)
attn_partition_kernel(AttnArgs a) {
  using S = Shape<T, D>;
  constexpr int kCPL = S::kCPL, kEPC = S::kEPC, kNE = S::kNE;
  const int kvh = blockIdx.x / a.blocks_per_group;
  const int sub = blockIdx.x - kvh * a.blocks_per_group;
  const int wave = sub * a.waves_per_block + (threadIdx.x >> 6);
  if (wave >= a.waves_per_group) return;
  const int part = blockIdx.y;
  const int s = blockIdx.z;

  Wave<T, D, GW> w(a);
  w.lane = threadIdx.x & 63;
  w.r = w.lane >> 3;
  w.c = w.lane & 7;

  int L = a.seq_lens[s];
  L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
  const int start = part * a.part_tokens;
  const int h0 = kvh * a.group + wave * GW;
  char* out_base = static_cast<char*>(a.out) + (int64_t(s) * a.num_q_heads + h0) * (D * S::kES);

  if (start >= L) {
    // Empty history (L == 0): the output is zero.  With split-KV the merge
    // kernel writes it instead.
    if (part == 0 && a.num_parts == 1 && w.r == 0) {
#pragma unroll
      for (int hh = 0; hh < GW; ++hh)
#pragma unroll
        for (int j = 0; j < kCPL; ++j)
          *reinterpret_cast<uint4*>(out_base + hh * D * S::kES + (w.c + 8 * j) * 16) =
              make_uint4(0, 0, 0, 0);
    }
    return;
  }
  const int end = min(start + a.part_tokens, L);

  const char* q_base =
      static_cast<const char*>(a.q) + (int64_t(s) * a.num_q_heads + h0) * (D * S::kES);
#pragma unroll
  for (int hh = 0; hh < GW; ++hh) {
#pragma unroll
    for (int j = 0; j < kCPL; ++j)
      w.q[hh][j] = *reinterpret_cast<const uint4*>(q_base + hh * D * S::kES + (w.c + 8 * j) * 16);
    w.m[hh] = kRefInit;
    w.l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < kNE; ++e) w.acc[hh][e] = 0.f;
  }

  w.trow = a.block_tables + int64_t(s) * a.max_blocks;
  w.blk_last = (end - 1) >> a.block_shift;
  const int blk_first = start >> a.block_shift;
  w.tcache_base = blk_first;
  w.tcache = (blk_first + w.lane <= w.blk_last) ? w.trow[blk_first + w.lane] : -1;
  w.head_off = int64_t(kvh) * D * S::kES;

  const int ntiles = (end - start + kTile - 1) / kTile;
  TileBuf<T, D> b0, b1;
  TileInfo t0 = w.prepare(start, end);
  w.load(t0, b0);
  for (int t = 0;;) {
    TileInfo t1;
    const bool has1 = t + 1 < ntiles;
    if (has1) {
      t1 = w.prepare(start + kTile * (t + 1), end);
      w.load(t1, b1);
    }
    w.run_tile(t0, b0);
    if (!has1) break;
    ++t;
    const bool has2 = t + 1 < ntiles;
    if (has2) {
      t0 = w.prepare(start + kTile * (t + 1), end);
      w.load(t0, b0);
    }
    w.run_tile(t1, b1);
    if (!has2) break;
    ++t;
  }

  // Merge the 8 streams (log-sum-exp rescale to the common reference).
  float lt[GW], M[GW];
#pragma unroll
  for (int hh = 0; hh < GW; ++hh) {
    M[hh] = pkv::max_across_groups8(w.m[hh]);
    const float wt = pkv::fast_exp2(w.m[hh] - M[hh]);
    lt[hh] = pkv::sum_across_groups8(w.l[hh] * wt);
#pragma unroll
    for (int e = 0; e < kNE; ++e) w.acc[hh][e] = pkv::sum_across_groups8(w.acc[hh][e] * wt);
  }
  if (w.r != 0) return;

  if (a.num_parts == 1) {
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
      const float inv = 1.0f / lt[hh];
#pragma unroll
      for (int j = 0; j < kCPL; ++j) {
        float f[kEPC];
#pragma unroll
        for (int e = 0; e < kEPC; ++e) f[e] = w.acc[hh][j * kEPC + e] * inv;
        *reinterpret_cast<uint4*>(out_base + hh * D * S::kES + (w.c + 8 * j) * 16) =
            pack_chunk<T>(f);
      }
    }
  } else {
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
      const int64_t row = (int64_t(s) * a.num_q_heads + h0 + hh) * a.num_parts + part;
      float* dst = a.ws_acc + row * D;
#pragma unroll
      for (int j = 0; j < kCPL; ++j) {
#pragma unroll
        for (int e4 = 0; e4 < kEPC; e4 += 4) {
          const int elem = (w.c + 8 * j) * kEPC + e4;
          const int src = j * kEPC + e4;
          *reinterpret_cast<float4*>(dst + elem) =
              make_float4(w.acc[hh][src], w.acc[hh][src + 1], w.acc[hh][src + 2],
                          w.acc[hh][src + 3]);
        }
      }
      if (w.c == 0) *reinterpret_cast<float2*>(a.ws_ml + row * 2) = make_float2(M[hh], lt[hh]);
    }
  }
}

// Split-KV merge: one workgroup (4 waves) per (sequence, query head).  Wave w
// folds partitions w, w+4, ...; the 4 partial results meet in LDS.
template <typename T, int D>
__global__ void __launch_bounds__(256)
attn_merge_kernel(AttnArgs a) {
  constexpr int kDPL = D / 64;  // dims per lane
  const int h = blockIdx.x, s = blockIdx.y;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int L = a.seq_lens[s];
  L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
  const int np = (L + a.part_tokens - 1) / a.part_tokens;
  const int64_t row0 = (int64_t(s) * a.num_q_heads + h) * a.num_parts;
  const float* ml = a.ws_ml + row0 * 2;
  const float* accp = a.ws_acc + row0 * D;

  __shared__ float red_m[4];
  __shared__ float red_l[4];
  __shared__ float red_o[4][D];

  float Mw = -INFINITY;
  for (int p = wv; p < np; p += 4) Mw = fmaxf(Mw, ml[2 * p]);
  if (lane == 0) red_m[wv] = Mw;
  __syncthreads();
  const float M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));

  float ls = 0.f, o[kDPL];
#pragma unroll
  for (int d = 0; d < kDPL; ++d) o[d] = 0.f;
  for (int p = wv; p < np; p += 4) {
    const float wt = pkv::fast_exp2(ml[2 * p] - M);
    ls = fmaf(wt, ml[2 * p + 1], ls);
    const float* src = accp + int64_t(p) * D + lane * kDPL;
#pragma unroll
    for (int d = 0; d < kDPL; ++d) o[d] = fmaf(wt, src[d], o[d]);
  }
  if (lane == 0) red_l[wv] = ls;
#pragma unroll
  for (int d = 0; d < kDPL; ++d) red_o[wv][lane * kDPL + d] = o[d];
  __syncthreads();
  if (wv != 0) return;
  const float lsum = red_l[0] + red_l[1] + red_l[2] + red_l[3];
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;  // np == 0: zeros
  char* dst = static_cast<char*>(a.out) + ((int64_t(s) * a.num_q_heads + h) * D) * sizeof(T);
  float f[kDPL];
#pragma unroll
  for (int d = 0; d < kDPL; ++d) {
    const int e = lane * kDPL + d;
    f[d] = ((red_o[0][e] + red_o[1][e]) + (red_o[2][e] + red_o[3][e])) * inv;
  }
  if constexpr (sizeof(T) == 2) {
    if constexpr (kDPL == 2) {
      reinterpret_cast<uint32_t*>(dst)[lane] = pkv::pack_bf16x2(f[0], f[1]);
    } else {
      reinterpret_cast<uint16_t*>(dst)[lane] = uint16_t(pkv::f32_to_bf16_bits(f[0]));
    }
  } else {
#pragma unroll
    for (int d = 0; d < kDPL; ++d) reinterpret_cast<float*>(dst)[lane * kDPL + d] = f[d];
  }
}

// ---------------------------------------------------------------------------
// Host side: planning, validation, dispatch.
// ---------------------------------------------------------------------------

struct Plan {
  int gw, waves_per_group, waves_per_block, blocks_per_group;
  int len_cap, part_tokens, num_parts;
  size_t ws_bytes;
};

int heads_per_wave(int G) {
  for (int gw : {4, 3, 2, 1})
    if (G % gw == 0) return gw;
  return 1;
}

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Default split-KV partition: 256 positions up to 4096-long contexts, 512
// beyond; no split when one partition covers the longest sequence.
int auto_partition(int32_t max_seq_len, int32_t block_size) {
  const int unit = block_size > kTile ? block_size : kTile;
  int64_t t = max_seq_len <= 4096 ? 256 : 512;
  t = round_up(t, unit);
  if (max_seq_len <= t) return static_cast<int>(round_up(max_seq_len > 0 ? max_seq_len : 1, unit));
  return static_cast<int>(t);
}

pkv_status make_plan(int32_t num_seqs, int32_t num_q_heads, int32_t max_seq_len,
                     int32_t max_blocks, int32_t partition_tokens, const pkv_geom* g,
                     const char* who, Plan* pl) {
  if (pkv_status st = pkv::check_geom(g, who)) return st;
  if (num_seqs < 0 || num_q_heads <= 0 || max_seq_len < 0 || max_blocks < 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: negative size", who);
  if (num_q_heads % g->num_kv_heads != 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: num_q_heads %d is not a multiple of num_kv_heads %d",
                     who, num_q_heads, g->num_kv_heads);
  if (g->head_dim != 64 && g->head_dim != 128)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "%s: head_dim %d (built: 64, 128)", who, g->head_dim);
  if (g->block_size < 8)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "%s: block_size %d < 8", who, g->block_size);
  const int G = num_q_heads / g->num_kv_heads;
  if (G > 64) return pkv::fail(PKV_ERR_UNSUPPORTED, "%s: more than 64 query heads per group", who);
  if (num_seqs > 65535) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: more than 65535 sequences", who);
  pl->gw = heads_per_wave(G);
  pl->waves_per_group = G / pl->gw;
  pl->waves_per_block =
      pl->waves_per_group < kMaxWavesPerBlock ? pl->waves_per_group : kMaxWavesPerBlock;
  pl->blocks_per_group = (pl->waves_per_group + pl->waves_per_block - 1) / pl->waves_per_block;
  const int64_t cap = int64_t(max_blocks) * g->block_size;
  pl->len_cap = static_cast<int>(max_seq_len < cap ? max_seq_len : cap);
  if (partition_tokens < 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: partition_tokens < 0", who);
  if (partition_tokens == 0) {
    pl->part_tokens = auto_partition(pl->len_cap, g->block_size);
  } else {
    if (partition_tokens % kTile != 0 || partition_tokens % g->block_size != 0)
      return pkv::fail(PKV_ERR_INVALID_ARG,
                       "%s: partition_tokens %d must be a multiple of 16 and of block_size %d", who,
                       partition_tokens, g->block_size);
    pl->part_tokens = partition_tokens;
  }
  const int64_t np = pl->len_cap == 0 ? 1 : (int64_t(pl->len_cap) + pl->part_tokens - 1) / pl->part_tokens;
  if (np > 65535) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: more than 65535 partitions", who);
  pl->num_parts = static_cast<int>(np);
  if (pl->num_parts > 1) {
    pl->ws_bytes = size_t(num_seqs) * num_q_heads * pl->num_parts * (g->head_dim + 2) * sizeof(float);
  } else {
    pl->ws_bytes = 0;
  }
  if (int64_t(g->num_kv_heads) * pl->blocks_per_group > 2147483647)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: grid too large", who);
  return PKV_OK;
}

template <typename T, int D, int GW>
void launch_partition(const dim3& grid, const dim3& block, hipStream_t st, const AttnArgs& a) {
  hipLaunchKernelGGL((attn_partition_kernel<T, D, GW>), grid, block, 0, st, a);
}

template <typename T, int D>
pkv_status dispatch(int phases, const Plan& pl, const AttnArgs& a, int num_kv_heads,
                    int num_seqs, int num_q_heads, hipStream_t st) {
  if (phases & 1) {
    const dim3 grid(num_kv_heads * pl.blocks_per_group, pl.num_parts, num_seqs);
    const dim3 block(64 * pl.waves_per_block);
    switch (pl.gw) {
      case 4: launch_partition<T, D, 4>(grid, block, st, a); break;
      case 3: launch_partition<T, D, 3>(grid, block, st, a); break;
      case 2: launch_partition<T, D, 2>(grid, block, st, a); break;
      default: launch_partition<T, D, 1>(grid, block, st, a); break;
    }
    if (hipError_t e = hipGetLastError())
      return pkv::fail(PKV_ERR_HIP, "pkv_attention_decode: launch failed: %s",
                       hipGetErrorString(e));
  }
  if ((phases & 2) && pl.num_parts > 1) {
    hipLaunchKernelGGL((attn_merge_kernel<T, D>), dim3(num_q_heads, num_seqs), dim3(256), 0, st, a);
    if (hipError_t e = hipGetLastError())
      return pkv::fail(PKV_ERR_HIP, "pkv_attention_decode: merge launch failed: %s",
                       hipGetErrorString(e));
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

int32_t pkv_attention_partition_tokens(int32_t num_seqs, int32_t num_q_heads,
                                       int32_t max_seq_len, const pkv_geom* geom) {
  Plan pl;
  const int32_t max_blocks =
      geom && geom->block_size > 0 ? (max_seq_len + geom->block_size - 1) / geom->block_size : 0;
  if (make_plan(num_seqs, num_q_heads, max_seq_len, max_blocks, 0, geom,
                "pkv_attention_partition_tokens", &pl) != PKV_OK)
    return 0;
  return pl.part_tokens;
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

pkv_status pkv_attention_decode_phase(int32_t phases, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                      float scale, void* out, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t max_seq_len,
                                      int32_t partition_tokens, void* workspace,
                                      size_t workspace_bytes, const pkv_geom* geom,
                                      void* stream) {
  const char* who = "pkv_attention_decode";
  if (phases < 1 || phases > 3)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: phases must be 1, 2 or 3", who);
  Plan pl;
  if (pkv_status st = make_plan(num_seqs, num_q_heads, max_seq_len, max_blocks_per_seq,
                                partition_tokens, geom, who, &pl))
    return st;
  if (!std::isfinite(scale)) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: scale is not finite", who);
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !out)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!pkv::aligned16(q) || !pkv::aligned16(out) || !pkv::aligned16(k_cache) ||
      !pkv::aligned16(v_cache) || (reinterpret_cast<uintptr_t>(block_tables) & 3u) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: misaligned pointer", who);
  if (pl.num_parts > 1) {
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
  a.ws_acc = static_cast<float*>(workspace);
  a.ws_ml = pl.num_parts > 1
                ? static_cast<float*>(workspace) +
                      size_t(num_seqs) * num_q_heads * pl.num_parts * geom->head_dim
                : nullptr;
  a.row_bytes = geom->num_kv_heads * geom->head_dim * es;
  a.block_bytes = int64_t(geom->block_size) * a.row_bytes;
  a.max_blocks = max_blocks_per_seq;
  a.num_q_heads = num_q_heads;
  a.group = num_q_heads / geom->num_kv_heads;
  a.waves_per_group = pl.waves_per_group;
  a.waves_per_block = pl.waves_per_block;
  a.blocks_per_group = pl.blocks_per_group;
  a.num_blocks = geom->num_blocks;
  a.block_shift = pkv::log2_exact(geom->block_size);
  a.len_cap = pl.len_cap;
  a.part_tokens = pl.part_tokens;
  a.num_parts = pl.num_parts;
  a.scale_log2 = static_cast<float>(double(scale) * 1.4426950408889634);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int hkv = geom->num_kv_heads;
  if (geom->dtype == PKV_BF16) {
    return geom->head_dim == 128
               ? dispatch<uint16_t, 128>(phases, pl, a, hkv, num_seqs, num_q_heads, st)
               : dispatch<uint16_t, 64>(phases, pl, a, hkv, num_seqs, num_q_heads, st);
  }
  return geom->head_dim == 128
             ? dispatch<float, 128>(phases, pl, a, hkv, num_seqs, num_q_heads, st)
             : dispatch<float, 64>(phases, pl, a, hkv, num_seqs, num_q_heads, st);
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
