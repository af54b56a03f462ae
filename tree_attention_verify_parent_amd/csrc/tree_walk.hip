// Ancestor-mask build and accept walk as stand-alone launches: one wave per
// request, lane = node (the wave logic is in tree_ops.h).
#include "tree_ops.h"

namespace spectree {

__global__ __launch_bounds__(kWave) void tree_mask_build_kernel(
    const int32_t* __restrict__ parents, int N, uint64_t* __restrict__ anc_mask,
    int32_t* __restrict__ depth, uint32_t* __restrict__ err_word) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const bool live = i < N;
  const int p = live ? parents[(size_t)b * N + i] : 0;
  bool req_bad;
  const uint64_t set = ancestor_set(p, i, live, err_word, &req_bad);
  if (live) {
    const size_t o = (size_t)b * N + i;
    anc_mask[o] = set;
    if (depth) depth[o] = req_bad ? -1 : (__popcll(set) - 1);
  }
}

__global__ __launch_bounds__(kWave) void accept_walk_kernel(
    const int32_t* __restrict__ parents, const uint64_t* __restrict__ anc_mask,
    const int32_t* __restrict__ draft_tokens, const int32_t* __restrict__ target_argmax, int N,
    int V, int32_t* __restrict__ accept_len, int32_t* __restrict__ path_nodes,
    int32_t* __restrict__ out_tokens, uint32_t* __restrict__ err_word) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const bool live = i < N;
  const size_t o = (size_t)b * N + i;
  const int p = live ? parents[o] : 0;
  const uint64_t anc = live ? anc_mask[o] : 0ull;
  const int d = live ? draft_tokens[o] : 0;
  const int t = live ? target_argmax[o] : 0;
  accept_walk_wave(b, i, live, N, V, p, anc, d, t, accept_len, path_nodes, out_tokens, err_word);
}

}  // namespace spectree

using namespace spectree;

extern "C" spec_status spec_tree_mask_build(const int32_t* parents, int B, int N,
                                            uint64_t* anc_mask, int32_t* depth,
                                            uint32_t* err_word, hipStream_t stream) {
  if (!parents || !anc_mask) return SPEC_ERR_NULL;
  if (B < 1 || N < 1 || N > SPEC_MAX_NODES) return SPEC_ERR_SHAPE;
  hip_clear_error();
  hipLaunchKernelGGL(tree_mask_build_kernel, dim3(B), dim3(kWave), 0, stream, parents, N,
                     anc_mask, depth, err_word);
  return launch_status();
}

extern "C" spec_status spec_accept_walk(const int32_t* parents, const uint64_t* anc_mask,
                                        const int32_t* draft_tokens,
                                        const int32_t* target_argmax, int B, int N, int V,
                                        int32_t* accept_len, int32_t* path_nodes,
                                        int32_t* out_tokens, uint32_t* err_word,
                                        hipStream_t stream) {
  if (!parents || !anc_mask || !draft_tokens || !target_argmax || !accept_len || !path_nodes ||
      !out_tokens)
    return SPEC_ERR_NULL;
  if (B < 1 || N < 1 || N > SPEC_MAX_NODES || V < 1) return SPEC_ERR_SHAPE;
  hip_clear_error();
  hipLaunchKernelGGL(accept_walk_kernel, dim3(B), dim3(kWave), 0, stream, parents, anc_mask,
                     draft_tokens, target_argmax, N, V, accept_len, path_nodes, out_tokens,
                     err_word);
  return launch_status();
}

extern "C" const char* spec_status_string(int status) {
  switch (status) {
    case SPEC_OK: return "SPEC_OK";
    case SPEC_ERR_NULL: return "SPEC_ERR_NULL: a required pointer is NULL";
    case SPEC_ERR_SHAPE: return "SPEC_ERR_SHAPE: a size is out of range or inconsistent";
    case SPEC_ERR_DTYPE: return "SPEC_ERR_DTYPE: unsupported dtype or dtype pair";
    case SPEC_ERR_WORKSPACE: return "SPEC_ERR_WORKSPACE: workspace missing or too small";
    case SPEC_ERR_HIP: return "SPEC_ERR_HIP: kernel launch failed";
    case SPEC_ERR_ALIGN: return "SPEC_ERR_ALIGN: pointer not 16-byte aligned";
    case SPEC_ERR_SCRATCH:
      return "SPEC_ERR_SCRATCH: these sizes need more scratch than the library's static buffer holds";
  }
  return "unknown spec_status";
}
