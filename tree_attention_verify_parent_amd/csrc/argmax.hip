// Per-row argmax of float32 logits, lowest index on ties.
//
// Under greedy verification the target's token at a draft node is the argmax
// of its logits (the target verifies the draft's proposal: Aurora, section 2).
// This is a pure HBM stream: one workgroup per row, 16-byte loads, UNROLL
// loads in flight per thread, each thread scanning its indices in increasing
// order with a strict '>' (so it keeps its lowest maximal index), then a wave
// and a workgroup reduction that break value ties by the smaller index.
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

template <int NT, int UNROLL, bool VEC>
__global__ __launch_bounds__(NT) void vocab_argmax_kernel(const float* __restrict__ logits,
                                                          int64_t V, int64_t row_stride,
                                                          int32_t* __restrict__ out_idx) {
  const int64_t r = blockIdx.x;
  const float* row = logits + r * row_stride;
  const int tid = threadIdx.x;
  ArgBest best{-INFINITY, 0x7fffffff};

  if (VEC) {
    const int64_t V4 = V >> 2;
    const f32x4_t* row4 = reinterpret_cast<const f32x4_t*>(row);
    // every pass issues all UNROLL loads before using any; the last pass is
    // predicated instead of falling back to one load at a time
    for (int64_t base = 0; base < V4; base += (int64_t)NT * UNROLL) {
      f32x4_t x[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int64_t k = base + u * NT + tid;
        x[u] = (k < V4) ? __builtin_nontemporal_load(&row4[k]) : f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
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
    for (int64_t k = (V4 << 2) + tid; k < V; k += NT) {
      const float x = row[k];
      if (x > best.v) { best.v = x; best.i = (int)k; }
    }
  } else {
    for (int64_t k = tid; k < V; k += NT) {
      const float x = row[k];
      if (x > best.v) { best.v = x; best.i = (int)k; }
    }
  }
  // A thread that saw only -inf (or nothing) keeps index INT_MAX; any real
  // element with an equal value then wins the tie by its smaller index.

#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    ArgBest other{__shfl_xor(best.v, o, kWave), __shfl_xor(best.i, o, kWave)};
    best = arg_better(best, other);
  }
  __shared__ float sv[NT / kWave];
  __shared__ int si[NT / kWave];
  const int wave = tid / kWave, lane = tid % kWave;
  if (lane == 0) {
    sv[wave] = best.v;
    si[wave] = best.i;
  }
  __syncthreads();
  if (tid == 0) {
    ArgBest b{sv[0], si[0]};
#pragma unroll
    for (int w = 1; w < NT / kWave; ++w) b = arg_better(b, ArgBest{sv[w], si[w]});
    // V >= 1 and logits are finite, so some element was seen
    out_idx[r] = b.i;
  }
}

}  // namespace spectree

using namespace spectree;

extern "C" spec_status spec_vocab_argmax(const float* logits, int64_t rows, int64_t V,
                                         int64_t row_stride, int32_t* out_idx,
                                         hipStream_t stream) {
  if (!logits || !out_idx) return SPEC_ERR_NULL;
  if (rows < 1 || V < 1 || row_stride < V || V > 0x7fffffffLL || rows > 0x7fffffffLL)
    return SPEC_ERR_SHAPE;
  const bool vec = ((reinterpret_cast<uintptr_t>(logits) & 15u) == 0) && (row_stride % 4 == 0);
  // Few rows: wide workgroups so a single row still has enough loads in
  // flight; many rows: 256 threads and several workgroups per CU.
  if (rows < 256) {
    if (vec)
      hipLaunchKernelGGL((vocab_argmax_kernel<1024, 8, true>), dim3((unsigned)rows), dim3(1024), 0,
                         stream, logits, V, row_stride, out_idx);
    else
      hipLaunchKernelGGL((vocab_argmax_kernel<1024, 8, false>), dim3((unsigned)rows), dim3(1024), 0,
                         stream, logits, V, row_stride, out_idx);
  } else {
    if (vec)
      hipLaunchKernelGGL((vocab_argmax_kernel<256, 8, true>), dim3((unsigned)rows), dim3(256), 0,
                         stream, logits, V, row_stride, out_idx);
    else
      hipLaunchKernelGGL((vocab_argmax_kernel<256, 8, false>), dim3((unsigned)rows), dim3(256), 0,
                         stream, logits, V, row_stride, out_idx);
  }
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}
