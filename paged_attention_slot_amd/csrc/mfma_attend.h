// One workgroup's pass of paged attention on the gfx950 matrix cores: up to
// 16 query rows per wave against the K/V of one KV head over a range of
// positions read through one block-table row ([KVM §19.2.3] paged attention;
// [KVX §01] the attention of one query; page keys in include/pkv.h).  Shared
// by the multi-token kernel and the shared-prefix kernels.
//
//  * K/V arrive in tiles of 32 positions, staged in LDS by the whole
//    workgroup as [position][d] rows, read back as MFMA operands: K with
//    plain 16-byte reads, V through gfx950's transposing LDS read
//    (ds_read_b64_tr_b16), which hands each lane the 4 positions of one d
//    that the V^T operand needs.  With several waves two LDS buffers each of
//    K and V are used in turn and the walk is software-pipelined (a tile's
//    scores are computed one step ahead of its weights, K staged two tiles
//    ahead and V one), with one barrier per tile; a single wave's LDS
//    accesses run in order, so it uses one buffer.  Tiles' global loads are
//    issued two tiles ahead of their staging, and the barrier waits only for
//    LDS, so they stay in flight; bf16 rows of 128 on eight waves (or four
//    of two row groups) load straight into four LDS buffers instead.
//  * A wave carries RG groups of 16 query rows (attend_rows): each K/V
//    operand read from LDS feeds RG matrix instructions.
//  * Scores as S^T = K Q^T with v_mfma_f32_16x16x32_bf16: a lane's result
//    fragment holds 8 positions of one query row (its lane & 15), so the
//    online softmax (log2 units) needs only the ^16 and ^32 lane exchanges,
//    and the weights P land directly in the operand layout of O^T += V^T P^T
//    (positions ordered 16(j/4) + 4q + j%4 in both operands).  P enters as
//    two bf16 terms (hi + lo), so the product keeps fp32-like weights.
//  * A row sees positions t <= p_row inside [t_lo, t_hi), which callers keep
//    below the history's length; past it tiles load zeros for V (finite
//    products) and leave K as it was (its scores are masked by selection).
//  * One-byte caches ([KVM §19.2.4] precision table; [PFX] "KV Cache 量化"):
//    FP8 e4m3 and INT8 codes are decoded exactly to bf16 pairs when a tile is
//    staged, so the matrix work is the bf16 one.  The FP8 K scale is folded
//    into the score scale by the caller and the V scale multiplies the
//    weights; INT8's per-(slot, head) K scale multiplies each score and its V
//    scale each weight (the sum of weights keeps the bare weights).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "pkv_device.h"

namespace pkv {
namespace mfma {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kKT = 32;             // positions per K/V tile
constexpr float kRefInit = -1e30f;  // reference of a row with no position yet

// LDS of one workgroup of NW waves: K/V tile buffers (two each for several
// waves: tiles ahead are staged into one while the other is read; one
// wave's LDS accesses run in order, so it needs one), and for INT8 the
// tiles' position scales (three slots for several waves).
// Row strides in LDS (bf16 elements): V rows padded by 32 bytes, so the
// transposing reads (4 rows x 4 eight-byte columns per 16 lanes) fall in
// different banks.  K rows by 32 bytes too with several waves: a 16-byte
// pad left the operand reads conflicting (the bank-conflict counter read
// about one cycle per LDS instruction on 512-token prefill; 0 with 32), but
// single-wave workgroups keep 16 bytes, where the larger tile would cost
// one resident workgroup per CU.
template <int D, int NW> constexpr int k_stride() { return NW == 1 ? D + 8 : D + 16; }
template <int D> constexpr int v_stride() { return D + 16; }
template <int NW> constexpr int lds_tiles() { return NW == 1 ? 1 : 2; }

// Element kinds of the cache pools.
enum Kind : int { kBf16 = 0, kFp8 = 1, kInt8 = 2 };

// Passes over bf16 pools with head_dim 128 on eight waves, or on four waves
// of two row groups, load tiles straight into LDS (gfx950's
// global_load_lds_dwordx4: each lane's 16 bytes land at the wave's LDS base
// + 16 * lane, no registers and no LDS stores), into four buffers each of K
// and V in the padded row layout.
template <int D, int NW, int Q, int RG = 1> constexpr bool direct_lds() {
  return Q == kBf16 && D == 128 && (NW == 8 || (NW == 4 && RG == 2));
}
constexpr int kDirectBufs = 4;

// One direct-to-LDS load: this lane's 16 bytes at base + off (base the same
// in every lane) go to LDS byte lds_base + 16 * lane (lds_base the same in
// every lane).  Written in asm so the compiler's wait insertion, which
// cannot tell the tile buffers apart, adds no wait for it before the LDS
// reads; the walk waits for these loads itself (vmcnt).  M0 (the LDS base)
// is saved and restored around it, with the wait state an M0 write needs
// before an LDS DMA.  No VGPR is written.
__device__ __forceinline__ void load_to_lds16(const char* base, int off, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory");
}

template <int D, int NW, int Q = kBf16, int RG = 1> constexpr int k_lds_elems() {
  return (direct_lds<D, NW, Q, RG>() ? kDirectBufs : lds_tiles<NW>()) * kKT * k_stride<D, NW>();
}
template <int D, int NW, int Q = kBf16, int RG = 1> constexpr int v_lds_elems() {
  return (direct_lds<D, NW, Q, RG>() ? kDirectBufs : lds_tiles<NW>()) * kKT * v_stride<D>();
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));

// Two floats to packed bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2v_t));
}

// ds_read_b64_tr_b16 (lane layout checked with a one-wave probe): within each
// group of 16 lanes, lane j receives element j % 4 of the 8-byte words that
// lanes j / 4, j / 4 + 4, j / 4 + 8, j / 4 + 12 address.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& x) {
  return __builtin_bit_cast(bf16x8_t, x);
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS accesses,
// not for its global loads, so the next tile's loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int Q, int NW> constexpr int s_lds_elems() {
  return Q == kInt8 ? (NW == 1 ? 1 : 3) * 2 * kKT : 1;
}

// The K/V history a workgroup reads: one KV head through one table row.
struct History {
  const void* k_cache;   // pools of the element kind (bf16 bits or one-byte codes)
  const void* v_cache;
  const int32_t* trow;   // block table row
  int32_t len;           // positions < len are in the table; zeros past it
  int32_t g;             // KV head
  int64_t block_elems;
  int32_t row_elems;
  int32_t num_blocks;
  int32_t block_shift;
  int32_t num_kv_heads;
  float v_scale;             // FP8: the V tensor scale
  const float* k_scales;     // INT8: fp32 [slot][num_kv_heads]
  const float* v_scales;
};

// Sixteen one-byte codes -> sixteen floats (exact).
template <int Q>
__device__ __forceinline__ void decode_codes(const uint4& x, float (&f)[16]) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (Q == kInt8) {
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

// Two floats that bf16 holds exactly (decoded codes) -> one bf16 pair.
__device__ __forceinline__ uint32_t bf16_pair_exact(float lo, float hi) {
  // the high halves of both words in one byte permute (v_perm_b32)
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// A row's running state in log2 units: reference m, sum of weights lsum, and
// the unnormalised weighted sum as this lane's fragment: o[dt][i] holds
// d = 16 dt + 4 (lane >> 4) + i of row (lane & 15).
template <int D>
struct RowAcc {
  float m;
  float lsum;
  f32x4_t o[D / 16];
};

// An empty state (no position seen).
template <int D>
__device__ __forceinline__ void start(RowAcc<D>& r) {
  r.m = kRefInit;
  r.lsum = 0.f;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) r.o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// The NW waves of the workgroup walk positions [t_lo, t_hi) of ``h`` together
// (every wave must call this with the same range), folding them into ``r``
// (start() it first; further calls continue the same online softmax).
// ``q`` points at this lane's query row (D bf16, 16-byte aligned); it is read
// only if row_ok.  k_lds / v_lds hold k_lds_elems<D, NW>() elements.  Q is
// the pools' element kind; INT8 needs ``s_lds`` (s_lds_elems<Q, NW>() floats
// of LDS) for the tiles' scales.  p_all (the same in every lane) is a position every live
// row of the workgroup sees: tiles entirely at or before it, and inside
// [t_lo, t_hi), skip the per-score mask (p_all < h.len or t_hi <= h.len,
// so tiles reaching past the history are masked).  t_lo must be a multiple of 8 (a
// lane's positions of a tile then lie in one block).  PD tiles are in flight
// ahead of the one being computed (PD register buffers of K/V per thread).
//
// The reference m of a row moves lazily: only when some lane of the wave
// holds a score more than kSlack (log2 units) above its row's reference is
// the state rescaled (to the rows' maxima), so weights stay <= 2^kSlack and
// most tiles skip both the rescale and the cross-lane maximum.  The sum of
// weights is kept per lane (each lane's positions of its row) and reduced
// over the row's four lanes only where a state is handed out.
//
// Segments: with an ``emit`` functor, [t_lo, t_hi) is cut at the multiples
// of ``seg`` (t_lo and seg multiples of the tile): after a segment's last
// tile emit(t, r) receives the start t of that tile and the segment's state,
// and the state starts afresh, while the tile stream (loads
// in flight, LDS buffers) runs on across the boundary.  One workgroup can so
// produce the pieces of several split-KV partitions in one pass.
struct NoEmit {
  template <class R> __device__ void operator()(int, R&, int) const {}
};

// The step's append folded into the pass (bf16 pools; kAppend): position
// ``pos`` of the history is the new token, whose K/V row for this KV head is
// read from ``k``/``v`` (D bf16 each) instead of the pools, and stored to the
// pools at ``k_dst``/``v_dst`` (the row of its slot for this KV head) when
// its tile is staged.  pos < 0: nothing to do.
struct NewRow {
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* k_dst;
  uint16_t* v_dst;
  int pos;
};

template <int D, int NW, int PD = 1, int Q = kBf16, bool kStream = false, class Emit = NoEmit,
          bool kAppend = false, bool kWaveOnly = false, int RG = 1>
__device__ __forceinline__ void attend_rows(const History& h, int t_lo, int t_hi,
                                            const uint16_t* const (&q)[RG],
                                            const bool (&row_ok)[RG], const int (&p_row)[RG],
                                            int p_all, float scale_log2, uint16_t* k_lds,
                                            uint16_t* v_lds, RowAcc<D> (&r)[RG],
                                            float* s_lds = nullptr, int seg = 0,
                                            const Emit& emit = Emit(),
                                            const NewRow& nr = NewRow()) {
  static_assert(!kAppend || Q == kBf16, "the folded append takes bf16 pools");
  static_assert(!kAppend || NW == 1, "the folded append runs in single-wave passes");
  static_assert(NW == 1 || PD == 2, "several waves keep two tiles of registers in flight");
  static_assert(!kWaveOnly || NW == 1, "a wave-only walk is a single wave's");
  // A single wave's LDS accesses run in order: it waits for its own and
  // needs the workgroup barrier only when its workgroup is one wave.  A
  // wave-only walk (kWaveOnly: one of several independent walks in a
  // workgroup, possibly of different lengths) never touches the barrier.
  const auto sync_lds = [] {
    if constexpr (kWaveOnly) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    else lds_barrier();
  };
  constexpr bool kDirect = direct_lds<D, NW, Q, RG>();
  constexpr float kSlack = 8.0f;
  constexpr int kEB = Q == kBf16 ? 2 : 1;   // bytes per element
  constexpr int kKS = D / 32;            // k-steps of the score product
  constexpr int kDT = D / 16;            // 16-wide d tiles of the output
  constexpr int kKStride = k_stride<D, NW>();  // K rows in LDS, bf16 elements
  constexpr int kVStride = v_stride<D>();  // V rows
  constexpr int kEPC = 16 / kEB;         // elements per 16-byte chunk
  constexpr int kChunksPerRow = D / kEPC;  // 16-byte chunks per K/V row
  constexpr int kChunks = kKT * kChunksPerRow;
  // (a single-wave walk uses its lane only: it may be one of several walks
  // in a workgroup)
  const int tid = NW == 1 ? static_cast<int>(threadIdx.x & 63) : static_cast<int>(threadIdx.x);
  const int lane = tid & 63;
  const int quad = lane >> 4;

  // The query rows as the score product's B operand (zeros for rows not
  // live); the scale enters with the exponent's fma.
  uint4 qf[RG][kKS];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
      qf[g][ks] = row_ok[g] ? *reinterpret_cast<const uint4*>(q[g] + 32 * ks + 8 * quad)
                            : make_uint4(0, 0, 0, 0);

  const int L = h.len;
  const int bmask = (1 << h.block_shift) - 1;
  // Chunks of a tile this thread moves: the same kEPC-element d slice (chunk cc)
  // of kPer consecutive positions pg * kPer .. + kPer - 1 (the global loads
  // stay coalesced: 16 lanes read one contiguous K/V row).
  constexpr int kPer = kChunks / (64 * NW);
  static_assert(kChunks % (64 * NW) == 0, "tile chunks must split evenly");
  const int cc = tid % kChunksPerRow;
  const int pg = tid / kChunksPerRow;
  // Register sets of tiles in flight: K/V chunks, and INT8's position scales
  // (lanes < 32), which travel with K.
  uint4 nk[PD][kPer], nv[PD][kPer];
  float nks[PD], nvs[PD];
  // The tile's (at most 4, block_size >= 8) block ids come from a window of
  // 64 table entries held one per lane (tcache: entry tcache_base + lane) and
  // read with v_readlane, so a tile's loads do not wait for a table read:
  // the window is reloaded only when a tile reaches past it.
  const int last_idx = L > 0 ? (L - 1) >> h.block_shift : -1;
  // Window of 64 entries from table index base: entries past the history, or
  // naming no block of the pool, read as block 0 (only zero-filled or masked
  // positions use them).  The asm waits for the window where it is loaded;
  // otherwise the first v_readlane would wait for every load in flight, since
  // the compiler cannot tell which path wrote it.
  const auto window = [&](int base) {
    int b = base + lane <= last_idx ? h.trow[base + lane] : 0;
    b = (b >= 0 && b < h.num_blocks) ? b : 0;
    asm volatile("" ::"v"(b));
    return b;
  };
  int tcache_base = t_lo >> h.block_shift;
  int tcache = window(tcache_base);
  // Byte offsets: this lane's d slice of KV head g, a position's row in its
  // block, a block.
  const int lane_pos = pg * kPer;
  const int lane_off = (h.g * D + cc * kEPC) * kEB;
  const int row_bytes = h.row_elems * kEB;
  const uint32_t block_bytes = static_cast<uint32_t>(h.block_elems * kEB);  // < 2^31
  // K/V tile loads: non-temporal when the caller reads each byte once
  const auto kv_load = [](const char* p) {
    if constexpr (kStream) return load_stream(p);
    else return *reinterpret_cast<const uint4*>(p);
  };
  // Issue the K loads (and INT8 scales) of the tile at t0 into register set j;
  // returns the tile's byte offset in the pools for its V loads.  Past the
  // history K is left as it was (its scores are masked by selection).
  auto fetch_k = [&](int j, int t0) -> uint64_t {
    const int b0 = t0 >> h.block_shift;
    if (b0 + 3 - tcache_base >= 64) {  // uniform, rare: move the window to b0
      tcache_base = b0;
      tcache = window(b0);
    }
    int ids[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) ids[k] = __builtin_amdgcn_readlane(tcache, b0 + k - tcache_base);
    // This lane's kPer positions p0 .. p0 + kPer - 1 lie in one block (t0 is
    // a multiple of 8, kPer divides 8 and the block size).
    const int p0 = t0 + lane_pos;
    const int k = (p0 >> h.block_shift) - b0;
    const int blk = k == 0 ? ids[0] : (k == 1 ? ids[1] : (k == 2 ? ids[2] : ids[3]));
    const uint64_t off = uint64_t(static_cast<uint32_t>(blk)) * block_bytes +
                         static_cast<uint32_t>((p0 & bmask) * row_bytes + lane_off);
    const char* kb = static_cast<const char*>(h.k_cache) + off;
    if (kAppend && nr.pos >= t0 && nr.pos < t0 + kKT) {  // uniform: the tile holds the new token
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        nk[j][i] = make_uint4(0, 0, 0, 0);
        if (p0 + i == nr.pos) nk[j][i] = kv_load(reinterpret_cast<const char*>(nr.k + cc * kEPC));
        else if (p0 + i < L) nk[j][i] = kv_load(kb + i * row_bytes);
      }
    } else if (t0 + kKT <= L) {  // uniform: the whole tile is history
#pragma unroll
      for (int i = 0; i < kPer; ++i) nk[j][i] = kv_load(kb + i * row_bytes);
    } else {
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (p0 + i < L) nk[j][i] = kv_load(kb + i * row_bytes);
    }
    if constexpr (Q == kInt8) {
      // Lane t < 32 fetches the scales of position t0 + t (0 past the
      // history, so an unwritten slot never reaches a weight).
      nks[j] = 0.f;
      nvs[j] = 0.f;
      const int pos = t0 + tid;
      if (tid < kKT && pos < L) {
        const int kp = (pos >> h.block_shift) - b0;
        const int bp = kp == 0 ? ids[0] : (kp == 1 ? ids[1] : (kp == 2 ? ids[2] : ids[3]));
        const int64_t si = (int64_t(bp) * (1 << h.block_shift) + (pos & bmask)) * h.num_kv_heads + h.g;
        nks[j] = h.k_scales[si];
        nvs[j] = h.v_scales[si];
      }
    }
    return off;
  };
  // Issue the V loads of the tile at t0 (pool offset ``off`` from fetch_k)
  // into register set j: zeros past the history, which keep the products
  // finite.
  auto fetch_v = [&](int j, int t0, uint64_t off) {
    const char* vb = static_cast<const char*>(h.v_cache) + off;
    const int p0 = t0 + lane_pos;
    if (kAppend && nr.pos >= t0 && nr.pos < t0 + kKT) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        nv[j][i] = make_uint4(0, 0, 0, 0);
        if (p0 + i == nr.pos) nv[j][i] = kv_load(reinterpret_cast<const char*>(nr.v + cc * kEPC));
        else if (p0 + i < L) nv[j][i] = kv_load(vb + i * row_bytes);
      }
    } else if (t0 + kKT <= L) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) nv[j][i] = kv_load(vb + i * row_bytes);
    } else {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        nv[j][i] = make_uint4(0, 0, 0, 0);
        if (p0 + i < L) nv[j][i] = kv_load(vb + i * row_bytes);
      }
    }
  };
  // Stage a tile's K (register set j) into LDS tile buffer kbuf as [pos][d]
  // bf16 (codes decoded), and INT8's scales into scale slot ss; its V into
  // buffer vbuf.  With kAppend the new token's chunks go to its slot as well
  // (the loads that read them have completed: their values are staged).
  constexpr int kTileElems = kKT * kKStride;   // one LDS tile buffer of K
  constexpr int kVTileElems = kKT * kVStride;  // and of V
  auto stage_rows = [&](const uint4& x, uint16_t* dst) {
    if constexpr (Q == kBf16) {
      *reinterpret_cast<uint4*>(dst) = x;
    } else if constexpr (Q == kFp8) {
      // code pairs straight to bf16 pairs (packed conversion)
      const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
      uint32_t w[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w[2 * e] = fp8x2_to_bf16x2(xw[e], false);
        w[2 * e + 1] = fp8x2_to_bf16x2(xw[e], true);
      }
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
      *reinterpret_cast<uint4*>(dst + 8) = make_uint4(w[4], w[5], w[6], w[7]);
    } else {
      float f[16];
      uint32_t w[8];
      decode_codes<Q>(x, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = bf16_pair_exact(f[2 * e], f[2 * e + 1]);
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
      *reinterpret_cast<uint4*>(dst + 8) = make_uint4(w[4], w[5], w[6], w[7]);
    }
  };
  auto stage_k = [&](int j, int kbuf, int ss, int t0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      stage_rows(nk[j][i], k_lds + kbuf * kTileElems + (pg * kPer + i) * kKStride + cc * kEPC);
      if constexpr (kAppend)
        if (t0 + pg * kPer + i == nr.pos)
          *reinterpret_cast<uint4*>(nr.k_dst + cc * kEPC) = nk[j][i];
    }
    if constexpr (Q == kInt8) {
      if (tid < kKT) {
        s_lds[2 * kKT * ss + tid] = nks[j];
        s_lds[2 * kKT * ss + kKT + tid] = nvs[j];
      }
    }
  };
  auto stage_v = [&](int j, int vbuf, int t0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      stage_rows(nv[j][i], v_lds + vbuf * kVTileElems + (pg * kPer + i) * kVStride + cc * kEPC);
      if constexpr (kAppend)
        if (t0 + pg * kPer + i == nr.pos)
          *reinterpret_cast<uint4*>(nr.v_dst + cc * kEPC) = nv[j][i];
    }
  };
  // This lane's V^T reads: row 4 (lane >> 4) + (lane & 15) / 4 (+ 16 for the
  // second half of the k dimension), columns 4 ((lane & 15) % 4) .. + 3 of
  // each 16-wide d tile.
  const uint16_t* v_rd = v_lds + (4 * quad + ((lane & 15) >> 2)) * kVStride + 4 * (lane & 3);
  // Last position this lane's row sees (-1: none): the mask of a tile that
  // not every live row sees whole is one compare per score against it.
  int row_lim[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g)
    row_lim[g] = row_ok[g] ? (p_row[g] < t_hi - 1 ? p_row[g] : t_hi - 1) : -1;
  // This lane's part of its row's sum of weights (the state's sum enters
  // through the row's first lane).
  float lpart[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) lpart[g] = quad == 0 ? r[g].lsum : 0.f;

  // A staged tile's scores S^T = K Q^T (LDS tile buffer kbuf): s[pt][i] is
  // position 16 pt + 4 quad + i of the tile for row (lane & 15).
  // Each K operand read serves the RG row groups of the wave.
  auto qk = [&](int kbuf, f32x4_t (&s)[RG][2]) {
    const uint16_t* kt = k_lds + kbuf * kTileElems;
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      f32x4_t acc[RG];
#pragma unroll
      for (int g = 0; g < RG; ++g) acc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        const uint4 ka = *reinterpret_cast<const uint4*>(
            kt + (16 * pt + (lane & 15)) * kKStride + 32 * ks + 8 * quad);
#pragma unroll
        for (int g = 0; g < RG; ++g)
          acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka), as_bf16x8(qf[g][ks]),
                                                           acc[g], 0, 0, 0);
      }
#pragma unroll
      for (int g = 0; g < RG; ++g) s[g][pt] = acc[g];
    }
  };
  // A tile's exponents x = scale * score - m (log2 units, m the row's
  // reference), -inf where the lane's row does not see the position; INT8
  // scores carry their key scales (scale slot ss).  If some lane's x exceeds
  // kSlack, the references move to the rows' maxima (the state rescaled) and
  // the exponents are formed again against them.  The exponents are fresh
  // registers, so the scores' registers are free for the next tile's product.
  auto exps = [&](int t0, const float* st, const f32x4_t (&s)[RG][2], int g, float mref,
                  float (&x)[RG][8]) {
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float c = scale_log2;
        if constexpr (Q == kInt8) c *= st[16 * pt + 4 * quad + i];
        x[g][4 * pt + i] = fmaf(s[g][pt][i], c, -mref);
      }
    // Uniform: some live row does not see every position of the tile.  Score
    // e = 4 pt + i sits at position t0 + 16 pt + 4 quad + i, visible to this
    // lane's row iff 16 pt + i <= vis.
    if (t0 + kKT - 1 > p_all || t0 + kKT > t_hi) {
      const int vis = row_lim[g] - t0 - 4 * quad;
#pragma unroll
      for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          x[g][4 * pt + i] = 16 * pt + i <= vis ? x[g][4 * pt + i] : -INFINITY;
    }
  };
  // (the NaN-propagating maximum: its operands need no quieting first)
  const auto max8 = [](const float (&v)[8]) {
    const auto mx = [](float a, float b) { return __builtin_elementwise_maximum(a, b); };
    return mx(mx(mx(mx(v[0], v[1]), v[2]), mx(mx(v[3], v[4]), v[5])), mx(v[6], v[7]));
  };
  auto prepare = [&](int t0, int ss, const f32x4_t (&s)[RG][2], float (&x)[RG][8]) {
    const float* st = s_lds + 2 * kKT * ss;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      exps(t0, st, s, g, r[g].m, x);
      if (__builtin_amdgcn_ballot_w64(max8(x[g]) > kSlack) != 0) {  // uniform
        exps(t0, st, s, g, 0.f, x);  // the scaled scores themselves
        const float mn = fmaxf(r[g].m, max_across_rows16(max8(x[g])));
        const float alpha = fast_exp2(r[g].m - mn);
        r[g].m = mn;
        lpart[g] *= alpha;
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) r[g].o[dt][i] *= alpha;
        exps(t0, st, s, g, mn, x);
      }
    }
  };
  // The weights of prepared exponents and their P V: vfrag(dt) reads this
  // lane's V^T operand of d tile dt (V^T[16 dt + (lane & 15)][positions
  // 4 quad .. + 3 and 16 + 4 quad .. + 3]); INT8's V scales in slot ss.
  // Each V operand read serves the RG row groups of the wave.
  auto weigh = [&](const auto& vfrag, int ss, const float (&x)[RG][8]) {
    const float* st = s_lds + 2 * kKT * ss;
    // Weights as two bf16 terms, p = hi + lo (hi = bf16(p), lo = bf16(p - hi)):
    // P V then carries p to about 2^-17 relative, like the fp32 sum.
    bf16x8_t pfh[RG], pfl[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      uint32_t ph[4], pl[4];
      float psum;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float p0 = fast_exp2(x[g][2 * k]);
        float p1 = fast_exp2(x[g][2 * k + 1]);
        psum = k == 0 ? p0 + p1 : psum + (p0 + p1);
        // score element e = 2k (+1) sits at tile position 16 (e / 4) + 4 quad + e % 4
        if constexpr (Q == kFp8) {
          p0 *= h.v_scale;
          p1 *= h.v_scale;
        } else if constexpr (Q == kInt8) {
          p0 *= st[kKT + 16 * ((2 * k) >> 2) + 4 * quad + ((2 * k) & 3)];
          p1 *= st[kKT + 16 * ((2 * k + 1) >> 2) + 4 * quad + ((2 * k + 1) & 3)];
        }
        const uint32_t hw = cvt_pk_bf16(p0, p1);
        ph[k] = hw;
        pl[k] = cvt_pk_bf16(p0 - __uint_as_float(hw << 16), p1 - __uint_as_float(hw & 0xFFFF0000u));
      }
      lpart[g] += psum;
      pfh[g] = as_bf16x8(make_uint4(ph[0], ph[1], ph[2], ph[3]));
      pfl[g] = as_bf16x8(make_uint4(pl[0], pl[1], pl[2], pl[3]));
    }
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) {
      const bf16x8_t va = vfrag(dt);
      f32x4_t acc[RG];
#pragma unroll
      for (int g = 0; g < RG; ++g)
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pfh[g], r[g].o[dt], 0, 0, 0);
#pragma unroll
      for (int g = 0; g < RG; ++g)
        r[g].o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pfl[g], acc[g], 0, 0, 0);
    }
  };
  // V^T fragments from the padded layout's buffer vbuf
  auto vfrag_padded = [&](int vbuf) {
    const uint16_t* vt = v_rd + vbuf * kVTileElems;
    return [vt](int dt) {
      const uint2 lo = lds_read_tr16(vt + 16 * dt);
      const uint2 hi = lds_read_tr16(vt + 16 * kVStride + 16 * dt);
      return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
    };
  };
  // Segment end after the tile at t (see above).
  auto segment_end = [&](int t) {
    if constexpr (!std::is_same<Emit, NoEmit>::value) {
      const int te = t + kKT;
      if (te >= t_hi || te % seg == 0) {  // uniform: a segment is complete
#pragma unroll
        for (int g = 0; g < RG; ++g) {
          r[g].lsum = sum_across_rows16(lpart[g]);
          emit(t, r[g], g);
          start(r[g]);
          lpart[g] = 0.f;
        }
      }
    }
  };

#pragma unroll
  for (int j = 0; j < PD; ++j)
#pragma unroll
    for (int i = 0; i < kPer; ++i) nk[j][i] = make_uint4(0, 0, 0, 0);
  if constexpr (NW == 1) {
    // One wave: tile t is staged, its scores and P V computed, in turn; the
    // tile PD ahead is loaded meanwhile.
#pragma unroll
    for (int j = 0; j < PD; ++j)
      if (t_lo + j * kKT < t_hi) fetch_v(j, t_lo + j * kKT, fetch_k(j, t_lo + j * kKT));
    for (int t0 = t_lo; t0 < t_hi; t0 += PD * kKT) {
#pragma unroll
      for (int j = 0; j < PD; ++j) {
        const int t = t0 + j * kKT;
        if (t >= t_hi) break;  // uniform
        stage_k(j, 0, 0, t);
        stage_v(j, 0, t);
        sync_lds();
        // the register set just staged takes the tile PD ahead, in flight
        // meanwhile
        if (t + PD * kKT < t_hi) fetch_v(j, t + PD * kKT, fetch_k(j, t + PD * kKT));
        f32x4_t sv[RG][2];
        float sc[RG][8];
        qk(0, sv);
        prepare(t, 0, sv, sc);
        weigh(vfrag_padded(0), 0, sc);
        segment_end(t);
      }
    }
  } else if constexpr (kDirect) {
    // Tiles loaded straight into LDS (see direct_lds), the same
    // software pipeline as below: iteration i, after one barrier, computes
    // tile i + 1's scores (K buffer (i + 1) % 4) and tile i's weights and
    // P V (V buffer i % 4), and issues tile i + 3's loads into buffers
    // (i + 3) % 4, whose previous tile (i - 1) every wave finished before
    // that barrier.  Before the barrier of iteration i a wave waits for its
    // loads of K(i + 1) and V(i) (every load issued later may stay in
    // flight: loads complete in order).  The history's last tile, if
    // partial, goes through registers with zeros past the history.
    //
    // The buffers keep the padded row layout of the register-staged walk
    // (rows of 18 chunks of 16 bytes, the last two padding).  Wave w loads
    // rows kRW w .. kRW w + kRW - 1 (kRW = 32 / NW: 4 or 8), 18 kRW chunk
    // slots from LDS byte 288 kRW w of the buffer, 64 slots per instruction
    // (the last one partly masked: 72 slots take 2, 144 take 3); padding
    // slots are not loaded.  The kRW rows lie in one block (t0 is a multiple
    // of 8, blocks hold a power of two >= 8), so a tile's block and row
    // offsets are the same in every lane: each lane adds only its slot's
    // fixed offset.
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = (t_hi - t_lo + kKT - 1) / kKT;
    const auto tile = [&](int u) { return t_lo + u * kKT; };
    constexpr int kSlotsPerRow = kKStride * 2 / 16;
    static_assert(kKStride == kVStride && kSlotsPerRow == 18, "rows of 18 chunks");
    constexpr int kRW = kKT / NW;                            // rows per wave
    constexpr int kLI = (kRW * kSlotsPerRow + 63) / 64;     // load instructions per pool
    int srow[kLI], soff[kLI];
    bool sval[kLI];
#pragma unroll
    for (int e = 0; e < kLI; ++e) {
      const int z = 64 * e + lane;  // slot of the wave's 18 kRW
      srow[e] = z / kSlotsPerRow;
      const int x = z - kSlotsPerRow * srow[e];
      sval[e] = z < kRW * kSlotsPerRow && x < 16;
      soff[e] = srow[e] * row_bytes + (h.g * D + 8 * x) * 2;
    }
    typedef __attribute__((address_space(3))) u32x4_native_t lds_u32x4;
    const auto lds_addr = [](uint16_t* q) {  // LDS byte address, in an SGPR
      return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(
          reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint16_t*)(q)))));
    };
    const uint32_t k_lds_a = lds_addr(k_lds), v_lds_a = lds_addr(v_lds);
    const auto uniform_ptr = [](const char* q) {
      const uint64_t v = reinterpret_cast<uint64_t>(q);
      const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
      const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
      return reinterpret_cast<const char*>((uint64_t(hi) << 32) | lo);
    };
    auto issue = [&](int t0, int buf) {
      const int b0 = t0 >> h.block_shift;
      if (b0 + 3 - tcache_base >= 64) {  // uniform, rare: move the window to b0
        tcache_base = b0;
        tcache = window(b0);
      }
      const int p0 = t0 + kRW * w;  // the wave's first row
      const int blk = __builtin_amdgcn_readlane(tcache, (p0 >> h.block_shift) - tcache_base);
      const uint64_t ub = uint64_t(static_cast<uint32_t>(blk)) * block_bytes +
                          static_cast<uint32_t>((p0 & bmask) * row_bytes);
      const char* const kg = uniform_ptr(static_cast<const char*>(h.k_cache) + ub);
      const char* const vg = uniform_ptr(static_cast<const char*>(h.v_cache) + ub);
      const uint32_t kd = k_lds_a + buf * (kTileElems * 2) + w * (kRW * kSlotsPerRow * 16);
      const uint32_t vd = v_lds_a + buf * (kVTileElems * 2) + w * (kRW * kSlotsPerRow * 16);
      if (t0 + kKT <= L) {  // uniform: the whole tile is history
        // K's instructions, then V's (the waits count them in this order)
#pragma unroll
        for (int e = 0; e < kLI; ++e)
          if (sval[e]) load_to_lds16(kg, soff[e], kd + 1024 * e);
#pragma unroll
        for (int e = 0; e < kLI; ++e)
          if (sval[e]) load_to_lds16(vg, soff[e], vd + 1024 * e);
      } else {
        // the history's last tile: through registers (waited for here, so
        // the counts of direct loads stay as the waits assume), zeros past
        // the history
#pragma unroll
        for (int e = 0; e < kLI; ++e) {
          uint4 kx = make_uint4(0, 0, 0, 0), vx = make_uint4(0, 0, 0, 0);
          if (sval[e] && p0 + srow[e] < L) {
            kx = *reinterpret_cast<const uint4*>(kg + soff[e]);
            vx = *reinterpret_cast<const uint4*>(vg + soff[e]);
          }
          if (sval[e]) {
            *(lds_u32x4*)(uintptr_t)(kd + 1024 * e + 16 * lane) = u32x4_native_t{kx.x, kx.y, kx.z, kx.w};
            *(lds_u32x4*)(uintptr_t)(vd + 1024 * e + 16 * lane) = u32x4_native_t{vx.x, vx.y, vx.z, vx.w};
          }
        }
      }
    };
    // Tiles loaded directly (whole tiles of history): their loads (kLI per
    // pool and wave) are the ones the waits count.
    const auto direct = [&](int u) { return u < n && tile(u) + kKT <= L; };
    // This wave's loads but the last kLI * ``later`` (later: 0, 1, 3 or 5).
    const auto wait_loads = [](int later) {
      if constexpr (kLI == 2) {
        switch (later) {
          case 1: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
          case 3: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
          case 5: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
          default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
        }
      } else {
        static_assert(kLI == 3, "two or three load instructions per pool");
        switch (later) {
          case 1: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
          case 3: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
          case 5: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
          default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
        }
      }
    };
#pragma unroll
    for (int u = 0; u < 3; ++u)
      if (u < n) issue(tile(u), u);
    // K(0) is needed: after it come V(0) and both pools' loads of tiles 1, 2
    wait_loads(direct(0) ? 1 + 2 * direct(1) + 2 * direct(2) : 0);
    lds_barrier();
    f32x4_t s_nx[RG][2];
    float sc[RG][8];
    qk(0, s_nx);
    if (n > 0) prepare(tile(0), 0, s_nx, sc);
    for (int i0 = 0; i0 < n; i0 += kDirectBufs) {
#pragma unroll
      for (int b = 0; b < kDirectBufs; ++b) {
        const int i = i0 + b;
        if (i >= n) break;  // uniform
        // K(i + 1) and V(i): after K(i + 1) come V(i + 1), then tile i + 2's
        // (a tile through registers is complete once issued)
        wait_loads(direct(i + 2) ? 3 : (direct(i + 1) ? 1 : 0));
        lds_barrier();
        qk((b + 1) % kDirectBufs, s_nx);      // tile i + 1's scores (unused past the last)
        weigh(vfrag_padded(b), 0, sc);        // tile i's weights and P V
        if (i + 3 < n) issue(tile(i + 3), (b + 3) % kDirectBufs);
        segment_end(tile(i));
        if (i + 1 < n) prepare(tile(i + 1), 0, s_nx, sc);
      }
    }
  } else {
    // Several waves, software-pipelined: while tile i's weights and P V are
    // computed, tile i + 1's scores are already on the matrix cores.  K is
    // staged two tiles ahead, V one: iteration i, after one barrier, reads K
    // buffer (i + 1) & 1 and V buffer i & 1, then stages K(i + 2) into K
    // buffer i & 1 and V(i + 1) into V buffer (i + 1) & 1, whose readers
    // (tile i's scores, tile i - 1's P V) every wave finished before that
    // barrier.  INT8 scales staged with K(u) sit in slot u % 3 until tile u's
    // P V.  Register sets: K(u) and V(u) in set u & 1; V loads trail K's by
    // one tile, so each V load reuses the pool offset its K load computed.
    const int n = (t_hi - t_lo + kKT - 1) / kKT;
    const auto tile = [&](int u) { return t_lo + u * kKT; };
    uint64_t voff = 0;
    if (n > 0) fetch_v(0, tile(0), fetch_k(0, tile(0)));
    if (n > 1) fetch_v(1, tile(1), fetch_k(1, tile(1)));
    if (n > 0) {
      stage_k(0, 0, 0, tile(0));
      stage_v(0, 0, tile(0));
    }
    if (n > 1) stage_k(1, 1, 1, tile(1));
    if (n > 2) fetch_v(0, tile(2), fetch_k(0, tile(2)));
    if (n > 3) voff = fetch_k(1, tile(3));
    lds_barrier();
    f32x4_t s_nx[RG][2];
    float sc[RG][8];
    qk(0, s_nx);
    if (n > 0) prepare(tile(0), 0, s_nx, sc);
    int ss = 0;  // scale slot of tile i
    for (int i0 = 0; i0 < n; i0 += 2) {
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const int i = i0 + par;
        if (i >= n) break;  // uniform
        lds_barrier();
        const int ss1 = ss == 2 ? 0 : ss + 1, ss2 = ss1 == 2 ? 0 : ss1 + 1;
        qk(par ^ 1, s_nx);      // tile i + 1's scores (unused past the last tile)
        weigh(vfrag_padded(par), ss, sc);  // tile i's weights and P V
        if (i + 2 < n) stage_k(par, par, ss2, tile(i + 2));
        if (i + 1 < n) stage_v(par ^ 1, par ^ 1, tile(i + 1));
        if (i + 3 < n) fetch_v(par ^ 1, tile(i + 3), voff);
        if (i + 4 < n) voff = fetch_k(par, tile(i + 4));
        segment_end(tile(i));
        if (i + 1 < n) prepare(tile(i + 1), ss1, s_nx, sc);
        ss = ss1;
      }
    }
  }
#pragma unroll
  for (int g = 0; g < RG; ++g) r[g].lsum = sum_across_rows16(lpart[g]);
  // the caller may reuse the LDS (another pass) right after
  sync_lds();
}


// One row group per wave (the form most walks take).
template <int D, int NW, int PD = 1, int Q = kBf16, bool kStream = false, class Emit = NoEmit,
          bool kAppend = false, bool kWaveOnly = false>
__device__ __forceinline__ void attend(const History& h, int t_lo, int t_hi, const uint16_t* q,
                                       bool row_ok, int p_row, int p_all, float scale_log2,
                                       uint16_t* k_lds, uint16_t* v_lds, RowAcc<D>& r,
                                       float* s_lds = nullptr, int seg = 0,
                                       const Emit& emit = Emit(), const NewRow& nr = NewRow()) {
  const uint16_t* const qs[1] = {q};
  const bool oks[1] = {row_ok};
  const int ps[1] = {p_row};
  attend_rows<D, NW, PD, Q, kStream, Emit, kAppend, kWaveOnly, 1>(
      h, t_lo, t_hi, qs, oks, ps, p_all, scale_log2, k_lds, v_lds,
      *reinterpret_cast<RowAcc<D>(*)[1]>(&r), s_lds, seg, emit, nr);
}

// Store this lane's fragment of a row's state as a piece: D floats of
// weighted sum at acc, (reference, sum) at ml (written by the quad-0 lanes).
template <int D>
__device__ __forceinline__ void store_piece(const RowAcc<D>& r, float* acc, float2* ml) {
  const int quad = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    *reinterpret_cast<float4*>(acc + 16 * dt + 4 * quad) =
        make_float4(r.o[dt][0], r.o[dt][1], r.o[dt][2], r.o[dt][3]);
  if (quad == 0) *ml = make_float2(r.m, r.lsum);
}

// Store a row's normalised result as bf16.
template <int D>
__device__ __forceinline__ void store_row_bf16(const RowAcc<D>& r, uint16_t* dst) {
  const int quad = (threadIdx.x & 63) >> 4;
  const float inv = r.lsum > 0.f ? 1.0f / r.lsum : 0.f;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const int d0 = 16 * dt + 4 * quad;
    *reinterpret_cast<uint2*>(dst + d0) =
        make_uint2(pack_bf16x2(r.o[dt][0] * inv, r.o[dt][1] * inv),
                   pack_bf16x2(r.o[dt][2] * inv, r.o[dt][3] * inv));
  }
}

}  // namespace mfma
}  // namespace pkv
