// Wave-level tree logic shared by the stand-alone mask / walk kernels and the
// fused verify-step kernel: one wave per request, lane i = node i (N <= 64).
//
// The mask is the custom tree-attention mask that follows the speculative
// tree's causal structure (Aurora, section 2, closing paragraph); the walk
// yields the acceptance length, the number of draft tokens the target accepts
// per verification step (Runtime Draft Model Training, "Evaluation").
#pragma once

#include "common.h"

namespace spectree {

// Ancestor-or-self set of node i by pointer doubling: after round r a node's
// set holds every ancestor within 2^r edges, so six rounds cover N <= 64.
// p is node i's parent (lanes at or past N pass live = false).  A request
// with any bad parent gets the self-only set on every lane and *req_bad set;
// its error bits go to err_word when that is non-null.
__device__ __forceinline__ uint64_t ancestor_set(int p, int i, bool live, uint32_t* err_word, bool* req_bad) {
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
  *req_bad = any_bad;
  return any_bad ? (1ull << i) : set;
}

// Accept walk of request b.  Node i >= 1 matches when its draft token d equals
// the target's argmax t at its parent; it is accepted when every node on its
// root path (root excluded) matches, i.e. (anc(i) & ~matched) == 0.  The path
// ends at the accepted node with the largest depth, ties to the lowest index:
// maximise the key depth*64 + (63 - i) over the wave.  Writes accept_len[b],
// path_nodes[b][0..N) and out_tokens[b][0..N) (-1 past the path).
__device__ __forceinline__ void accept_walk_wave(int b, int i, bool live, int N, int V, int p, uint64_t anc,
                                                 int d, int t, int32_t* __restrict__ accept_len,
                                                 int32_t* __restrict__ path_nodes,
                                                 int32_t* __restrict__ out_tokens, uint32_t* err_word) {
  const size_t o = (size_t)b * N + i;
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
