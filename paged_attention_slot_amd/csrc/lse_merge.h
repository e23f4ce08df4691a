// Log-sum-exp merge of split-KV pieces into output rows ([KVM §19.2.3]: the
// block-wise online softmax combines partial results by rescaling them to a
// common maximum; page keys in include/pkv.h).  Shared by the decode and the
// multi-token kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "pkv_device.h"

namespace pkv {

// Log-sum-exp merge of n workspace rows row0, row0 + step, ... into one output
// row, by one 256-thread workgroup, in chunks of 64 rows with one memory round
// trip each: every thread (stream, q) loads float4 column q of its rows of the
// chunk (p = stream mod kStreams) while wave 0 loads the chunk's 64 (m, l)
// pairs; wave 0 moves the running reference to M' = max(M, max m_p), puts the
// weights w_p = exp2(m_p - M') and the rescale exp2(M - M') in LDS and keeps
// sum_p w_p l_p; after one barrier every thread rescales its partial row and
// adds its weighted rows.  The partial rows meet in LDS at the end; out = acc /
// l (zeros when n == 0).
// ---------------------------------------------------------------------------
constexpr int kMergeThreads = 256;
constexpr int kMergeRows = 64;  // rows per chunk (one per lane of wave 0)

template <typename T, int D>
__device__ __forceinline__ void merge_rows(const float* ws_acc, const float2* ws_ml, int n,
                                           int64_t row0, int64_t step, char* dst_row) {
  constexpr int kQ = D / 4;                        // float4 columns per row
  constexpr int kStreams = kMergeThreads / kQ;     // rows folded in parallel
  constexpr int kPer = kMergeRows / kStreams;      // rows per thread per chunk
  const int tid = threadIdx.x, lane = tid & 63;
  const bool lead = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6)) == 0;
  const float4* acc4 = reinterpret_cast<const float4*>(ws_acc);

  // double-buffered: wave 0 fills chunk c + 1's weights only after every
  // wave has passed chunk c's barrier, i.e. finished reading chunk c - 1's
  __shared__ float wts[2][kMergeRows];
  __shared__ float rescale[2];
  __shared__ float lsum_sh;
  __shared__ float4 part_out[kStreams][kQ];

  const int stream = tid / kQ, q = tid % kQ;
  float M = -INFINITY, ls = 0.f;  // wave 0's running reference and sum
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  int buf = 0;
  for (int c0 = 0; c0 < n; c0 += kMergeRows, buf ^= 1) {
    float4 x[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int p = c0 + stream + kStreams * k;
      x[k] = p < n ? acc4[(row0 + p * step) * kQ + q] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (lead) {
      const int p = c0 + lane;
      const float2 v = p < n ? ws_ml[row0 + p * step] : make_float2(-INFINITY, 0.f);
      const float Mn = fmaxf(M, wave_max(v.x));
      const float al = M == -INFINITY ? 0.f : fast_exp2(M - Mn);
      const float wt = p < n ? fast_exp2(v.x - Mn) : 0.f;
      ls = ls * al + wave_sum(wt * v.y);
      M = Mn;
      wts[buf][lane] = wt;
      if (lane == 0) rescale[buf] = al;
    }
    __syncthreads();
    const float al = rescale[buf];
    o.x *= al; o.y *= al; o.z *= al; o.w *= al;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const float wt = wts[buf][stream + kStreams * k];
      o.x = fmaf(wt, x[k].x, o.x);
      o.y = fmaf(wt, x[k].y, o.y);
      o.z = fmaf(wt, x[k].z, o.z);
      o.w = fmaf(wt, x[k].w, o.w);
    }
  }
  part_out[stream][q] = o;
  if (lead && lane == 0) lsum_sh = ls;
  __syncthreads();
  if (tid >= kQ) return;
  const float lsum = lsum_sh;
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  float4 rr = part_out[0][q];
#pragma unroll
  for (int k = 1; k < kStreams; ++k) {
    const float4 x = part_out[k][q];
    rr.x += x.x; rr.y += x.y; rr.z += x.z; rr.w += x.w;
  }
  const float f[4] = {rr.x * inv, rr.y * inv, rr.z * inv, rr.w * inv};
  if constexpr (sizeof(T) == 2) {
    reinterpret_cast<uint2*>(dst_row)[q] =
        make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
  } else {
    reinterpret_cast<float4*>(dst_row)[q] = make_float4(f[0], f[1], f[2], f[3]);
  }
}

}  // namespace pkv
