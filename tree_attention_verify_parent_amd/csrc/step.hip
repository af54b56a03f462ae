// The whole verify step in two launches: a "prep" kernel that builds the
// ancestor masks, takes every node's vocabulary argmax and runs each request's
// accept walk, then the tree attention.
//
// The walk needs the argmax and the tree, not the attention's output (under
// greedy verification the target's token at a node is the argmax of its
// logits, and acceptance follows the tree: Aurora, section 2; Runtime Draft
// Model Training, "Evaluation"), so all of it goes ahead of the attention in
// one launch instead of three:
//   * workgroups [0, n_mask_wg): one wave per request builds the ancestor-or-
//     self masks and depths the attention reads;
//   * the rest: workgroup (r, c) scans chunk c of logits row r = b*N + i and
//     folds its best (value, index) into the row's 64-bit key with an atomic
//     unsigned max.  Keys order by value first, then by the smaller index, so
//     the max is the argmax with ties to the lowest index whatever order the
//     chunks land in.  Each chunk then counts itself into its row's counter,
//     and the chunk that completes a row counts the row into its request's
//     counter; the workgroup that completes a request has every key of it
//     final: its first wave swaps the keys back to zero (reading them),
//     recomputes the request's masks in registers and runs the accept walk.
//     Counters are cleared by the workgroup that completes them, so keys and
//     counters start every call at zero, the state in which the caller hands
//     the workspace over the first time.
// Keys and counters are updated with system-scope atomics, which every XCD
// sees at the same coherence point; a chunk's max has returned before the
// chunk counts itself, so the last arrival reads complete keys.
#include "argmax_ops.h"
#include "gfx950.h"
#include "host_api.h"
#include "tree_ops.h"

namespace spectree {

constexpr int kPrepThreads = 256;

#ifndef SPEC_PREP_SCOPE
#define SPEC_PREP_SCOPE __HIP_MEMORY_SCOPE_SYSTEM
#endif

// Unsigned-orderable key of a (value, index) pair: the float's bits mapped so
// that unsigned order is float order (-0.0 taken as +0.0), and the index
// stored as 0xFFFFFFFF - i so that, for equal values, the smaller index has
// the larger key.  Every key of a finite value or of -inf is non-zero, so a
// zeroed key is below all of them.
__device__ __forceinline__ uint64_t arg_key(ArgBest a) {
  uint32_t bits = __float_as_uint(a.v);
  if ((bits << 1) == 0u) bits = 0u;
  const uint32_t ord = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)a.i);
}

template <int UNROLL, bool VEC>
__global__ __launch_bounds__(kPrepThreads) void verify_prep_kernel(
    const int32_t* __restrict__ parents, const int32_t* __restrict__ draft_tokens,
    const float* __restrict__ logits, int64_t V, int64_t row_stride, int B, int N, int n_mask_wg, int chunks,
    int64_t chunk_len, uint64_t* __restrict__ anc_mask, int32_t* __restrict__ depth,
    int32_t* __restrict__ target_argmax, int32_t* __restrict__ accept_len, int32_t* __restrict__ path_nodes,
    int32_t* __restrict__ out_tokens, uint64_t* __restrict__ keys, uint32_t* __restrict__ row_cnt,
    uint32_t* __restrict__ req_cnt, uint32_t* __restrict__ err_word) {
  constexpr int NT = kPrepThreads;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;

  if ((int)blockIdx.x < n_mask_wg) {
    const int b = (int)blockIdx.x * (NT / kWave) + tid / kWave;
    if (b >= B) return;                                // the whole wave leaves; no barrier follows
    const bool live = lane < N;
    const size_t o = (size_t)b * N + lane;
    const int p = live ? parents[o] : 0;
    bool req_bad;
    const uint64_t set = ancestor_set(p, lane, live, err_word, &req_bad);
    if (live) {
      anc_mask[o] = set;
      if (depth) depth[o] = req_bad ? -1 : (__popcll(set) - 1);
    }
    return;
  }

  // chunk c of row r: logits [c * chunk_len, min(V, (c + 1) * chunk_len)),
  // chunk_len a multiple of the NT * UNROLL float4 loads of one pass
  const int u = (int)blockIdx.x - n_mask_wg;
  const int r = u / chunks, c = u - r * chunks;
  const float* row = logits + (int64_t)r * row_stride;
  const int64_t lo = (int64_t)c * chunk_len;
  const int64_t hi = lo + chunk_len < V ? lo + chunk_len : V;
  ArgBest best{-INFINITY, 0x7fffffff};
  if (VEC) {
    const int64_t V4 = V >> 2;
    const int64_t hi4 = (lo + chunk_len) / 4 < V4 ? (lo + chunk_len) / 4 : V4;
    best = scan_vec4<NT, UNROLL>(row, lo / 4, hi4, tid, best);
    if (c == chunks - 1) best = scan_scalar<NT>(row, V4 << 2, V, tid, best);
  } else {
    best = scan_scalar<NT>(row, lo, hi, tid, best);
  }
  best = wg_best<NT>(best, tid);

  // Count in two levels, so that no word takes more than max(chunks, N)
  // atomics (increments of one word are serialised): the last chunk of a row
  // counts the row into its request.
  __shared__ uint32_t s_last;
  const int b = r / N;
  if (tid == 0) {
    const uint64_t prev = __hip_atomic_fetch_max(keys + r, arg_key(best), __ATOMIC_RELAXED, SPEC_PREP_SCOPE);
    asm volatile("" ::"v"(prev));                      // keep the returning form ...
    wait_vmcnt<0>();                                   // ... and wait for its return
    bool row_done = true;
    if (chunks > 1) {
      const uint32_t seen = __hip_atomic_fetch_add(row_cnt + r, 1u, __ATOMIC_RELAXED, SPEC_PREP_SCOPE);
      row_done = seen == (uint32_t)(chunks - 1);
      if (row_done) __hip_atomic_store(row_cnt + r, 0u, __ATOMIC_RELAXED, SPEC_PREP_SCOPE);
    }
    uint32_t last = 0u;
    if (row_done) {
      const uint32_t seen = __hip_atomic_fetch_add(req_cnt + b, 1u, __ATOMIC_RELAXED, SPEC_PREP_SCOPE);
      last = (seen == (uint32_t)(N - 1)) ? 1u : 0u;
    }
    s_last = last;
  }
  __syncthreads();
  if (!s_last || tid >= kWave) return;

  // last row of request b: every key of the request is final
  const bool live = lane < N;
  const size_t o = (size_t)b * N + lane;
  const int p = live ? parents[o] : 0;
  const int d = live ? draft_tokens[o] : 0;
  const uint64_t key = live ? __hip_atomic_exchange(keys + o, 0ull, __ATOMIC_RELAXED, SPEC_PREP_SCOPE) : 0ull;
  const int t = (int)(0xFFFFFFFFu - (uint32_t)key);
  if (live) target_argmax[o] = t;
  bool req_bad;
  const uint64_t anc = ancestor_set(p, lane, live, nullptr, &req_bad);   // the mask workgroup flags errors
  accept_walk_wave(b, lane, live, N, (int)V, p, anc, d, t, accept_len, path_nodes, out_tokens, err_word);
  if (lane == 0) __hip_atomic_store(req_cnt + b, 0u, __ATOMIC_RELAXED, SPEC_PREP_SCOPE);
}

// Argmax work split: UNROLL float4 loads in flight per thread and pass, and
// about kPrepTargetWgs workgroups in all -- rows are cut into chunks (a whole
// number of passes each) only as far as that takes, since every chunk costs
// atomics on its row's key and counter.
constexpr long long kPrepTargetWgs = 1024;

struct PrepPlan {
  int unroll;
  int chunks;
  long long chunk_len;   // logits per chunk
};

static PrepPlan make_prep_plan(long long rows, long long V) {
  PrepPlan pp;
  pp.unroll = 8;
  long long target = kPrepTargetWgs;
#ifdef SPEC_PREP_HOOK
  SPEC_PREP_HOOK(pp.unroll, target);
#endif
  const long long pass = (long long)kPrepThreads * pp.unroll * 4;
  long long want = (target + rows - 1) / rows;
  const long long max_chunks = (V + pass - 1) / pass;
  if (want > max_chunks) want = max_chunks;
  if (want < 1) want = 1;
  const long long per = (V + want - 1) / want;
  pp.chunk_len = ((per + pass - 1) / pass) * pass;
  pp.chunks = (int)((V + pp.chunk_len - 1) / pp.chunk_len);
  return pp;
}

static size_t prep_ws_bytes(int B, int N) {
  const size_t raw = (size_t)B * N * (sizeof(uint64_t) + sizeof(uint32_t)) + (size_t)B * sizeof(uint32_t);
  return (raw + 255) & ~(size_t)255;
}

static bool aligned_to(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace spectree

using namespace spectree;

extern "C" size_t spec_verify_step_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int S_max) {
  if (B < 1 || N < 1 || N > SPEC_MAX_NODES) return 0;
  // the attention's part is never empty for sizes it accepts
  const size_t attn = spec_tree_attn_workspace_bytes(B, N, Hq, Hkv, D, S_max);
  return attn ? prep_ws_bytes(B, N) + attn : 0;
}

extern "C" spec_status spec_verify_step(
    const int32_t* parents, const int32_t* draft_tokens, const int32_t* prefix_lens, const void* q,
    spec_dtype q_dtype, const void* k_cache, const void* v_cache, spec_dtype kv_dtype, const float* k_scale,
    const float* v_scale, const float* logits, int64_t V, int64_t logits_row_stride, int B, int N, int Hq,
    int Hkv, int D, int S_max, float sm_scale, uint64_t* anc_mask, int32_t* depth, void* out, float* lse,
    int32_t* target_argmax, int32_t* accept_len, int32_t* path_nodes, int32_t* out_tokens, void* workspace,
    size_t workspace_bytes, uint32_t* err_word, hipStream_t stream) {
  if (!parents || !draft_tokens || !logits || !anc_mask || !target_argmax || !accept_len || !path_nodes ||
      !out_tokens)
    return SPEC_ERR_NULL;
  if (B < 1 || N < 1 || N > SPEC_MAX_NODES || V < 1 || V > 0x7fffffffLL || logits_row_stride < V)
    return SPEC_ERR_SHAPE;
  const size_t prep_bytes = prep_ws_bytes(B, N);
  // the full size for every dtype (the fp32 attention leaves its part unused)
  if (!workspace || workspace_bytes < spec_verify_step_workspace_bytes(B, N, Hq, Hkv, D, S_max))
    return SPEC_ERR_WORKSPACE;
  if (!aligned_to(workspace, 16)) return SPEC_ERR_ALIGN;
  void* attn_ws = static_cast<char*>(workspace) + prep_bytes;
  const size_t attn_ws_bytes = workspace_bytes - prep_bytes;
  // everything the attention would refuse is refused before the first launch
  const spec_status ast = tree_attn_check(q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, prefix_lens,
                                          anc_mask, B, N, Hq, Hkv, D, S_max, sm_scale, out, attn_ws,
                                          attn_ws_bytes);
  if (ast != SPEC_OK) return ast;

  const long long rows = (long long)B * N;
  const PrepPlan pp = make_prep_plan(rows, V);
  const int n_mask_wg = (B + kPrepThreads / kWave - 1) / (kPrepThreads / kWave);
  const long long grid = n_mask_wg + rows * pp.chunks;
  if (grid >= (1ll << 31)) return SPEC_ERR_SHAPE;

  uint64_t* keys = static_cast<uint64_t*>(workspace);
  uint32_t* row_cnt = reinterpret_cast<uint32_t*>(keys + rows);
  uint32_t* req_cnt = row_cnt + rows;
  const bool vec = aligned_to(logits, 16) && (logits_row_stride % 4 == 0);
#define SPEC_PREP(U_, VEC_)                                                                                   \
  hipLaunchKernelGGL((verify_prep_kernel<U_, VEC_>), dim3((unsigned)grid), dim3(kPrepThreads), 0, stream,     \
                     parents, draft_tokens, logits, V, logits_row_stride, B, N, n_mask_wg, pp.chunks,         \
                     (int64_t)pp.chunk_len, anc_mask, depth, target_argmax, accept_len, path_nodes,           \
                     out_tokens, keys, row_cnt, req_cnt, err_word)
  if (vec) {
    if (pp.unroll == 8) SPEC_PREP(8, true);
    else if (pp.unroll == 4) SPEC_PREP(4, true);
    else SPEC_PREP(2, true);
  } else {
    if (pp.unroll == 8) SPEC_PREP(8, false);
    else if (pp.unroll == 4) SPEC_PREP(4, false);
    else SPEC_PREP(2, false);
  }
#undef SPEC_PREP
  if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
  return spec_tree_attn_verify(q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, prefix_lens, anc_mask,
                               B, N, Hq, Hkv, D, S_max, sm_scale, out, lse, attn_ws, attn_ws_bytes, err_word,
                               stream);
}
