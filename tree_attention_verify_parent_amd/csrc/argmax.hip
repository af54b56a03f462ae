// Per-row argmax of float32 logits, lowest index on ties, as a stand-alone
// launch (the scan and reductions are in argmax_ops.h).
//
// This is a pure HBM stream: one workgroup per row, 16-byte loads, UNROLL
// loads in flight per thread, then a wave and a workgroup reduction that
// break value ties by the smaller index.
#include "argmax_ops.h"

namespace spectree {

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
    best = scan_vec4<NT, UNROLL>(row, 0, V4, tid, best);
    best = scan_scalar<NT>(row, V4 << 2, V, tid, best);
  } else {
    best = scan_scalar<NT>(row, 0, V, tid, best);
  }
  best = wg_best<NT>(best, tid);
  // V >= 1 and logits are finite, so some element was seen
  if (tid == 0) out_idx[r] = best.i;
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
  hip_clear_error();
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
  return launch_status();
}
