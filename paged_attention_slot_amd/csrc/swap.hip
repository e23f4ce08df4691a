// Block swap between the device pools and a pool in pinned host memory
// (pkv_swap_out, pkv_swap_in).
//
// A paused request's KV cache moves to CPU memory and back whole blocks at a
// time ([KVM §19.2.6]; [ENG §8.2]: CPU memory as a second-level block pool,
// unseen by attention because only the block table changes).  The block lists
// are scattered on both sides, so instead of one runtime copy request per block
// a single launch moves them all: one workgroup per (pair, pool) reads the
// source block with coalesced 16-byte loads and writes it straight into the
// destination, the host side being reached over the host link through its
// device mapping.  Every lane issues all of its loads before its first store,
// so each workgroup keeps up to 32 KiB of reads in flight, which the link's
// latency needs.  Page keys are listed in include/pkv.h.
#include <hip/hip_runtime.h>

#include "geom.h"

namespace {

constexpr int kSwapThreads = 256;
constexpr int kSwapUnroll = 8;   // 16-byte chunks per lane per round
constexpr int kMaxPools = 4;     // K, V and, for INT8 caches, their scale pools

// A plain vector type: arrays of it stay in registers.
typedef uint32_t chunk16 __attribute__((ext_vector_type(4)));

struct SwapPool {
  const chunk16* src;
  chunk16* dst;
  int32_t chunks;  // 16-byte chunks per block
};

struct SwapArgs {
  const int32_t* pairs;  // [num_pairs][2] = (source block, destination block)
  int32_t src_blocks;
  int32_t dst_blocks;
  SwapPool pool[kMaxPools];
};

// grid = (num_pairs, num_pools).  Pairs naming a block outside either pool
// are skipped.
__global__ void __launch_bounds__(kSwapThreads) swap_blocks_kernel(SwapArgs a) {
  const int32_t s = a.pairs[2 * blockIdx.x];
  const int32_t d = a.pairs[2 * blockIdx.x + 1];
  if (s < 0 || s >= a.src_blocks || d < 0 || d >= a.dst_blocks) return;
  // Uniform select (no dynamic indexing into the argument block).
  const uint32_t w = blockIdx.y;
  const SwapPool p = w == 0 ? a.pool[0] : w == 1 ? a.pool[1] : w == 2 ? a.pool[2] : a.pool[3];
  const chunk16* src = p.src + int64_t(s) * p.chunks;
  chunk16* dst = p.dst + int64_t(d) * p.chunks;
  constexpr int32_t kRound = kSwapThreads * kSwapUnroll;
  const int32_t full = p.chunks - p.chunks % kRound;
  const int32_t t = threadIdx.x;
  for (int32_t r0 = 0; r0 < full; r0 += kRound) {
    chunk16 r[kSwapUnroll];
#pragma unroll
    for (int u = 0; u < kSwapUnroll; ++u) r[u] = src[r0 + u * kSwapThreads + t];
#pragma unroll
    for (int u = 0; u < kSwapUnroll; ++u) dst[r0 + u * kSwapThreads + t] = r[u];
  }
  if (full < p.chunks) {  // last partial round: the same, each chunk guarded
    chunk16 r[kSwapUnroll];
#pragma unroll
    for (int u = 0; u < kSwapUnroll; ++u) {
      const int32_t i = full + u * kSwapThreads + t;
      r[u] = i < p.chunks ? src[i] : chunk16(0);
    }
#pragma unroll
    for (int u = 0; u < kSwapUnroll; ++u) {
      const int32_t i = full + u * kSwapThreads + t;
      if (i < p.chunks) dst[i] = r[u];
    }
  }
}

enum class Kind { kDevice, kPinnedHost, kAny };

// The address a kernel uses for ``p``, after checking that the runtime knows
// it as the expected kind of memory.  Pageable host memory is refused: a
// kernel cannot reach it.
pkv_status mapped(const void* p, Kind want, const char* who, const char* what, const void** out) {
  hipPointerAttribute_t at{};
  const hipError_t e = hipPointerGetAttributes(&at, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // not a launch error: clear it
    return pkv::fail(PKV_ERR_INVALID_ARG,
                     "%s: %s is not memory the runtime knows (pageable host memory?): %s", who,
                     what, hipGetErrorString(e));
  }
  const bool host = at.type == hipMemoryTypeHost;
  const bool dev = at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged;
  if ((want == Kind::kPinnedHost && !host) || (want == Kind::kDevice && !dev) ||
      (want == Kind::kAny && !host && !dev))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: %s must be %s memory (memory type %d)", who, what,
                     want == Kind::kPinnedHost ? "pinned host" : "device", int(at.type));
  *out = host ? at.devicePointer : p;
  if (!*out) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: %s has no device mapping", who, what);
  return PKV_OK;
}

pkv_status swap(bool out, const int32_t* pairs, int32_t num_pairs, const void* k_cache,
                const void* v_cache, const pkv_kv_scales* scales, const pkv_host_pool* host,
                const pkv_geom* geom, void* stream) {
  const char* who = out ? "pkv_swap_out" : "pkv_swap_in";
  if (pkv_status st = pkv::check_geom(geom, who)) return st;
  if (num_pairs < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: num_pairs < 0", who);
  if (!host) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: null host pool", who);
  if (host->num_blocks <= 0 ||
      int64_t(host->num_blocks) * geom->block_size >= (int64_t(1) << 31))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: bad host num_blocks %d", who, host->num_blocks);
  const bool i8 = geom->dtype == PKV_INT8;
  const int64_t block_bytes =
      int64_t(geom->block_size) * geom->num_kv_heads * geom->head_dim * pkv::elem_size(geom->dtype);
  const int64_t scale_bytes = int64_t(geom->block_size) * geom->num_kv_heads * 4;
  if (block_bytes / 16 >= (int64_t(1) << 31))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: block too large", who);
  if (i8 && scale_bytes % 16 != 0)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "%s: block_size * num_kv_heads must be a multiple of 4",
                     who);
  if (num_pairs == 0) return PKV_OK;
  const void* dp[4] = {k_cache, v_cache, i8 && scales ? scales->k_scales : nullptr,
                       i8 && scales ? scales->v_scales : nullptr};
  const void* hp[4] = {host->k, host->v, i8 ? host->k_scales : nullptr,
                       i8 ? host->v_scales : nullptr};
  const int pools = i8 ? 4 : 2;
  if (!pairs) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: null pairs", who);
  if (reinterpret_cast<uintptr_t>(pairs) & 3u)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: misaligned pairs", who);
  if (i8 && !scales) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: null scales", who);
  for (int i = 0; i < pools; ++i) {
    if (!dp[i] || !hp[i]) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: null pool pointer", who);
    if (!pkv::aligned16(dp[i]) || !pkv::aligned16(hp[i]))
      return pkv::fail(PKV_ERR_INVALID_ARG, "%s: misaligned pool pointer", who);
  }
  static const char* dnames[4] = {"k_cache", "v_cache", "k_scales", "v_scales"};
  static const char* hnames[4] = {"host k", "host v", "host k_scales", "host v_scales"};
  const void* pairs_dev = nullptr;
  if (pkv_status st = mapped(pairs, Kind::kAny, who, "pairs", &pairs_dev)) return st;
  SwapArgs a{};
  a.pairs = static_cast<const int32_t*>(pairs_dev);
  a.src_blocks = out ? geom->num_blocks : host->num_blocks;
  a.dst_blocks = out ? host->num_blocks : geom->num_blocks;
  for (int i = 0; i < pools; ++i) {
    const void *d = nullptr, *h = nullptr;
    if (pkv_status st = mapped(dp[i], Kind::kDevice, who, dnames[i], &d)) return st;
    if (pkv_status st = mapped(hp[i], Kind::kPinnedHost, who, hnames[i], &h)) return st;
    const int64_t bytes = i < 2 ? block_bytes : scale_bytes;
    a.pool[i].src = static_cast<const chunk16*>(out ? d : h);
    a.pool[i].dst = static_cast<chunk16*>(const_cast<void*>(out ? h : d));
    a.pool[i].chunks = static_cast<int32_t>(bytes / 16);
  }
  hipLaunchKernelGGL(swap_blocks_kernel, dim3(num_pairs, pools), dim3(kSwapThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  if (hipError_t e = hipGetLastError())
    return pkv::fail(PKV_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_swap_out(const int32_t* pairs, int32_t num_pairs, const void* k_cache,
                        const void* v_cache, const pkv_kv_scales* scales,
                        const pkv_host_pool* host, const pkv_geom* geom, void* stream) {
  return swap(true, pairs, num_pairs, k_cache, v_cache, scales, host, geom, stream);
}

pkv_status pkv_swap_in(const int32_t* pairs, int32_t num_pairs, const pkv_host_pool* host,
                       void* k_cache, void* v_cache, const pkv_kv_scales* scales,
                       const pkv_geom* geom, void* stream) {
  return swap(false, pairs, num_pairs, k_cache, v_cache, scales, host, geom, stream);
}

}  // extern "C"
