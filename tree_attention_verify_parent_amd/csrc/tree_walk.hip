// Ancestor-mask build and accept walk: one wave per request, lane = node.
//
// The mask is the custom tree-attention mask that follows the speculative
// tree's causal structure (Aurora, section 2, closing paragraph); the walk
// yields the acceptance length, the number of draft tokens the target accepts
// per verification step (Runtime Draft Model Training, "Evaluation").
#include "common.h"

namespace spectree {

// Ancestor-or-self sets by pointer doubling: after round r a node's set holds
// every ancestor within 2^r edges, so six rounds cover N <= 64.
__global__ __launch_bounds__(kWave) void tree_mask_build_kernel(
    const int32_t* __restrict__ parents, int N, uint64_t* __restrict__ anc_mask,
    int32_t* __restrict__ depth, uint32_t* __restrict__ err_word) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const bool live = i < N;
  const int p = live ? parents[(size_t)b * N + i] : 0;

  uint32_t bad = 0;
  if (live) {
    if (i == 0 && p != -1) bad |= SPEC_DERR_ROOT;
    if (i > 0 && (p < 0 || p >= i)) bad |= SPEC_DERR_PARENT;
  }
  // any lane's error marks the whole request
  const bool any_bad = __any(bad != 0);
  if (bad) flag_error(err_word, bad);

  int jump = (i == 0 || !live || bad) ? 0 : p;
  uint64_t set = (1ull << i) | (1ull << jump);
#pragma unroll
  for (int r = 0; r < 6; ++r) {
    set |= shfl_u64(set, jump);
    jump = __shfl(jump, jump, kWave);
  }
  if (live) {
    const size_t o = (size_t)b * N + i;
    anc_mask[o] = any_bad ? (1ull << i) : set;
    if (depth) depth[o] = any_bad ? -1 : (__popcll(set) - 1);
  }
}

// Accept walk.  Node i >= 1 matches when its draft token equals the target's
// argmax at its parent; it is accepted when every node on its root path
// (root excluded) matches, i.e. (anc(i) & ~matched) == 0.  The path ends at
// the accepted node with the largest depth, ties to the lowest index:
// maximise the key depth*64 + (63 - i) over the wave.
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

  uint32_t bad = 0;
  if (live) {
    if (i == 0 && p != -1) bad |= SPEC_DERR_ROOT;
    if (i > 0 && (p < 0 || p >= i)) bad |= SPEC_DERR_PARENT;
    if (i > 0 && (d < 0 || d >= V)) bad |= SPEC_DERR_TOKEN;
    if (t < 0 || t >= V) bad |= SPEC_DERR_TOKEN;
  }
  if (bad) flag_error(err_word, bad);

  const int t_parent = __shfl(t, (p >= 0 && p < kWave) ? p : 0, kWave);
  const bool match = live && i > 0 && d == t_parent;
  const uint64_t matched = __ballot(match) | 1ull;
  const bool accepted = live && (anc & ~matched) == 0ull;
  const int dep = __popcll(anc) - 1;

  int key = accepted ? dep * 64 + (63 - i) : -1;
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) key = max(key, __shfl_xor(key, s, kWave));
  // the root is always accepted, so key >= 63
  const int end = 63 - (key & 63);
  const int L = key >> 6;
  const uint64_t path = shfl_u64(anc, end);

  if (live) {
    // ancestors of the end node write themselves at their depth; the slots
    // past L get -1 from the lane with that index
    if ((path >> i) & 1ull) {
      if (dep >= 0 && dep < N) {
        path_nodes[(size_t)b * N + dep] = i;
        out_tokens[(size_t)b * N + dep] = t;
      }
    }
    if (i > L) {
      path_nodes[o] = -1;
      out_tokens[o] = -1;
    }
    if (i == 0) accept_len[b] = L;
  }
}

}  // namespace spectree

using namespace spectree;

extern "C" spec_status spec_tree_mask_build(const int32_t* parents, int B, int N,
                                            uint64_t* anc_mask, int32_t* depth,
                                            uint32_t* err_word, hipStream_t stream) {
  if (!parents || !anc_mask) return SPEC_ERR_NULL;
  if (B < 1 || N < 1 || N > SPEC_MAX_NODES) return SPEC_ERR_SHAPE;
  hipLaunchKernelGGL(tree_mask_build_kernel, dim3(B), dim3(kWave), 0, stream, parents, N,
                     anc_mask, depth, err_word);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
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
  hipLaunchKernelGGL(accept_walk_kernel, dim3(B), dim3(kWave), 0, stream, parents, anc_mask,
                     draft_tokens, target_argmax, N, V, accept_len, path_nodes, out_tokens,
                     err_word);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

extern "C" const char* spec_status_string(spec_status status) {
  switch (status) {
    case SPEC_OK: return "SPEC_OK";
    case SPEC_ERR_NULL: return "SPEC_ERR_NULL: a required pointer is NULL";
    case SPEC_ERR_SHAPE: return "SPEC_ERR_SHAPE: a size is out of range or inconsistent";
    case SPEC_ERR_DTYPE: return "SPEC_ERR_DTYPE: unsupported dtype or dtype pair";
    case SPEC_ERR_WORKSPACE: return "SPEC_ERR_WORKSPACE: workspace missing or too small";
    case SPEC_ERR_HIP: return "SPEC_ERR_HIP: kernel launch failed";
    case SPEC_ERR_ALIGN: return "SPEC_ERR_ALIGN: pointer not 16-byte aligned";
  }
  return "unknown spec_status";
}
