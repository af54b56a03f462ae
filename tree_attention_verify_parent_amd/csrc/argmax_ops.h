// Argmax building blocks shared by the stand-alone per-row argmax and the
// fused verify-step kernel: float32 values, lowest index on ties.
//
// Under greedy verification the target's token at a draft node is the argmax
// of its logits (the target verifies the draft's proposal: Aurora, section 2).
#pragma once

#include "common.h"

namespace spectree {

struct ArgBest {
  float v;
  int i;
};

// b beats a: larger value, or equal value and smaller index.  Float compare,
// so -0.0 == +0.0.
__device__ __forceinline__ ArgBest arg_better(ArgBest a, ArgBest b) {
  const bool take = (b.v > a.v) || (b.v == a.v && b.i < a.i);
  return take ? b : a;
}

// Scan float4 elements [lo4, hi4) of a 16-byte aligned row, NT threads of a
// workgroup together: every pass issues all UNROLL loads before using any
// (the last pass is predicated instead of falling back to one load at a
// time), and each thread visits its indices in increasing order with a
// strict '>', so it keeps its lowest maximal index.
template <int NT, int UNROLL>
__device__ __forceinline__ ArgBest scan_vec4(const float* __restrict__ row, int64_t lo4, int64_t hi4, int tid,
                                             ArgBest best) {
  const f32x4_t* row4 = reinterpret_cast<const f32x4_t*>(row);
  for (int64_t base = lo4; base < hi4; base += (int64_t)NT * UNROLL) {
    f32x4_t x[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t k = base + u * NT + tid;
      x[u] = (k < hi4) ? __builtin_nontemporal_load(&row4[k]) : f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int j = (int)((base + u * NT + tid) << 2);
      if (x[u].x > best.v) { best.v = x[u].x; best.i = j; }
      if (x[u].y > best.v) { best.v = x[u].y; best.i = j + 1; }
      if (x[u].z > best.v) { best.v = x[u].z; best.i = j + 2; }
      if (x[u].w > best.v) { best.v = x[u].w; best.i = j + 3; }
    }
  }
  return best;
}

// Scan elements [lo, hi) one at a time (rows that are not 16-byte aligned,
// and the tail past the last whole float4).
template <int NT>
__device__ __forceinline__ ArgBest scan_scalar(const float* __restrict__ row, int64_t lo, int64_t hi, int tid,
                                               ArgBest best) {
  for (int64_t k = lo + tid; k < hi; k += NT) {
    const float x = row[k];
    if (x > best.v) { best.v = x; best.i = (int)k; }
  }
  return best;
}

// Workgroup-wide best; the result is valid in thread 0.  A thread that saw
// only -inf (or nothing) holds index INT_MAX, so any real element with an
// equal value wins the tie by its smaller index.
template <int NT>
__device__ __forceinline__ ArgBest wg_best(ArgBest best, int tid) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    ArgBest other{__shfl_xor(best.v, o, kWave), __shfl_xor(best.i, o, kWave)};
    best = arg_better(best, other);
  }
  if constexpr (NT == kWave) {
    return best;
  } else {
    __shared__ float sv[NT / kWave];
    __shared__ int si[NT / kWave];
    const int wave = tid / kWave, lane = tid % kWave;
    if (lane == 0) {
      sv[wave] = best.v;
      si[wave] = best.i;
    }
    __syncthreads();
    ArgBest b{sv[0], si[0]};
#pragma unroll
    for (int w = 1; w < NT / kWave; ++w) b = arg_better(b, ArgBest{sv[w], si[w]});
    return b;
  }
}

}  // namespace spectree
