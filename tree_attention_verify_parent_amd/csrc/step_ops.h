// The verify step's "prep" work -- ancestor masks, per-node vocabulary argmax
// and accept walk -- as a workgroup role that the tail workgroups of an
// attention kernel (the split kernel's, or the fp32 kernel's) take on.
//
// The walk needs the argmax and the tree, not the attention's output (under
// greedy verification the target's token at a node is the argmax of its
// logits, and acceptance follows the tree: Aurora, section 2; Runtime Draft
// Model Training, "Evaluation").  Prep workgroups [0, n_mask_wg) build the
// masks, one wave per request; the others each take chunk c of logits row
// r = b*N + i:
//   * the chunk's best (value, index) is folded into the row's 64-bit key with
//     an atomic unsigned max; keys order by value first, then by the smaller
//     index, so the max is the argmax with ties to the lowest index whatever
//     order the chunks land in;
//   * the chunk then counts itself into its request's counter -- or, when a
//     request has many chunks, into its row's counter first, the chunk that
//     completes a row counting the row into its request's (two levels, so
//     that no word takes more than max(chunks, N) increments: increments of
//     one word are serialised);
//   * the workgroup that completes a request has every key of it final: its
//     first wave swaps the keys back to zero (reading them), recomputes the
//     request's masks in registers and runs the accept walk.
// Counters are cleared by the workgroup that completes them, so keys and
// counters start every call at zero, the state in which the caller hands the
// workspace over the first time.  Keys and counters are updated with
// system-scope atomics, which every XCD sees at the same coherence point; a
// chunk's max has been performed (its wave's vector memory count has drained)
// before the chunk counts itself, so the last arrival reads complete keys.
#pragma once

#include <algorithm>

#include "argmax_ops.h"
#include "gfx950.h"
#include "tree_ops.h"

namespace spectree {

// float4 loads in flight per thread and pass of the argmax scan
constexpr int kPrepUnroll = 8;
// about this many scanning workgroups in all: rows are cut into chunks (a
// whole number of passes each) only as far as that takes, since every chunk
// costs atomics on its row's key and counter
constexpr long long kPrepTargetWgs = 1024;
// a request with at most this many chunks counts them on one word
constexpr int kPrepOneLevel = 64;

struct PrepArgs {
  const int32_t* parents;
  const int32_t* draft_tokens;
  const float* logits;
  int64_t V;
  int64_t row_stride;
  int64_t chunk_len;     // logits per chunk, a whole number of scan passes
  int chunks;            // chunks per row
  int one_level;         // count chunks straight into the request's counter
  int n_mask_wg;         // workgroups that build the masks
  int n_scan_wg;         // workgroups that scan a chunk each
  int held;              // chunks [0, held) are scanned by the attention's workgroups (chunk g by workgroup g)
  int mask_counts;       // each request's mask wave counts itself in as one more arrival
  int vec;               // rows 16-byte aligned: float4 loads
  uint64_t* anc_mask;
  int32_t* depth;
  int32_t* target_argmax;
  int32_t* accept_len;
  int32_t* path_nodes;
  int32_t* out_tokens;
  uint64_t* keys;        // [rows], zero between calls
  uint32_t* row_cnt;     // [rows], zero between calls
  uint32_t* req_cnt;     // [B], zero between calls
};

// Bytes of workspace the prep role needs (keys, row and request counters),
// rounded up to 256.
inline size_t prep_workspace_bytes(int B, int N) {
  const size_t raw = (size_t)B * N * (sizeof(uint64_t) + sizeof(uint32_t)) + (size_t)B * sizeof(uint32_t);
  return (raw + 255) & ~(size_t)255;
}

// Fill in the work split of pa for workgroups of nt threads; returns the
// number of prep workgroups.  host_wgs > 0: the prep role rides in the
// attention's launch, whose first host_wgs workgroups are the attention's.
// Then, when every chunk (host_unroll float4 per thread, what the attention's
// LDS stage holds) fits one attention workgroup each and a request's chunks
// fit one counter, the attention's workgroups scan them in their prologue (in
// the shadow of their first tiles) and count them in at once, and the mask
// waves in the tail arrive last and run the walks while the attention still
// works.  Otherwise scanning workgroups take the chunks, about
// kPrepTargetWgs of them (in the attention's tail they start as its
// workgroups leave their CUs).
inline long long plan_prep(PrepArgs* pa, int B, int N, int nt, long long host_wgs, int host_unroll = 0) {
  const long long rows = (long long)B * N;
  pa->n_mask_wg = (B + nt / kWave - 1) / (nt / kWave);
  pa->held = 0;
  pa->mask_counts = 0;
  const long long hpass = (long long)nt * host_unroll * 4;   // a chunk in the attention's prologue
  const long long h_chunks = host_unroll > 0 ? (pa->V + hpass - 1) / hpass : 0;
  if (host_wgs > 0 && host_unroll > 0 && pa->vec && pa->V % 4 == 0 && N * h_chunks <= kPrepOneLevel &&
      rows * h_chunks <= host_wgs) {
    pa->chunk_len = hpass;
    pa->chunks = (int)h_chunks;
    pa->one_level = 1;
    pa->held = (int)(rows * h_chunks);
    pa->mask_counts = 1;
    pa->n_scan_wg = 0;
    return pa->n_mask_wg;
  }
  long long target = kPrepTargetWgs;
  const long long pass = (long long)nt * kPrepUnroll * 4;
  const long long max_chunks = (pa->V + pass - 1) / pass;
  long long want = (target + rows - 1) / rows;
  if (want > max_chunks) want = max_chunks;
  if (want < 1) want = 1;
  const long long per = (pa->V + want - 1) / want;
  pa->chunk_len = ((per + pass - 1) / pass) * pass;
  pa->chunks = (int)((pa->V + pa->chunk_len - 1) / pa->chunk_len);
  pa->one_level = (long long)N * pa->chunks <= kPrepOneLevel;
  pa->n_scan_wg = (int)(rows * pa->chunks);
  return pa->n_mask_wg + pa->n_scan_wg;
}

// Arrivals that complete request b's counter (one-level counting).
__host__ __device__ inline uint32_t prep_arrivals(const PrepArgs& pa, int N) {
  return (uint32_t)(N * pa.chunks + pa.mask_counts);
}

// Point the keys and counters at the start of a workspace.
inline void place_prep_workspace(PrepArgs* pa, void* ws, int B, int N) {
  const size_t rows = (size_t)B * N;
  pa->keys = static_cast<uint64_t*>(ws);
  pa->row_cnt = reinterpret_cast<uint32_t*>(pa->keys + rows);
  pa->req_cnt = pa->row_cnt + rows;
}

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

// Fold a workgroup's best into its row's key (thread 0).  The atomic is
// complete once the thread's vector memory count drains (prep_finish waits
// for that before counting).
__device__ __forceinline__ void prep_fold(const PrepArgs& pa, int g, ArgBest best) {
  __hip_atomic_fetch_max(pa.keys + g / pa.chunks, arg_key(best), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Request b's walk, by one whole wave (lane = node), once every key of the
// request is final: swap the keys back to zero (reading them), recompute the
// masks in registers, walk, and clear the request's counter.  p, d: the
// lane's node's parent and draft token.
__device__ __forceinline__ void prep_walk(const PrepArgs& pa, int b, int N, int lane, int p, int d,
                                          uint32_t* err_word) {
  const bool live = lane < N;
  const size_t o = (size_t)b * N + lane;
  const uint64_t key =
      live ? __hip_atomic_exchange(pa.keys + o, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) : 0ull;
  const int t = (int)(0xFFFFFFFFu - (uint32_t)key);
  if (live) pa.target_argmax[o] = t;
  bool req_bad;
  const uint64_t anc = ancestor_set(p, lane, live, nullptr, &req_bad);   // the mask wave flags errors
  accept_walk_wave(b, lane, live, N, (int)pa.V, p, anc, d, t, pa.accept_len, pa.path_nodes, pa.out_tokens,
                   err_word);
  if (lane == 0) __hip_atomic_store(pa.req_cnt + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Count chunk g in after its fold (thread 0); returns whether it completed its
// request.
__device__ __forceinline__ bool prep_count(const PrepArgs& pa, int g, int N) {
  constexpr int SCOPE = __HIP_MEMORY_SCOPE_SYSTEM;
  const int r = g / pa.chunks;
  const int b = r / N;
  wait_vmcnt<0>();                                     // the fold's max has been performed
  if (!pa.one_level && pa.chunks > 1) {
    const uint32_t seen = __hip_atomic_fetch_add(pa.row_cnt + r, 1u, __ATOMIC_RELAXED, SCOPE);
    if (seen != (uint32_t)(pa.chunks - 1)) return false;
    __hip_atomic_store(pa.row_cnt + r, 0u, __ATOMIC_RELAXED, SCOPE);
  }
  const uint32_t total = pa.one_level ? prep_arrivals(pa, N) : (uint32_t)N;
  return __hip_atomic_fetch_add(pa.req_cnt + b, 1u, __ATOMIC_RELAXED, SCOPE) == total - 1;
}

// After chunk g's fold (every thread of the workgroup calls it): count the
// chunk in; the workgroup that completes a request runs its walk.  Wave 0
// fetches the request's parents and draft tokens first, so they arrive while
// the counts are in flight.
template <int NT>
__device__ __forceinline__ void prep_finish(const PrepArgs& pa, int g, int B, int N, uint32_t* err_word) {
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int b = g / pa.chunks / N;
  const size_t o = (size_t)b * N + lane;
  int p = 0, d = 0;
  if (tid < kWave && lane < N) {
    p = pa.parents[o];
    d = pa.draft_tokens[o];
  }
  __shared__ uint32_t s_last;
  if (tid == 0) s_last = prep_count(pa, g, N) ? 1u : 0u;
  __syncthreads();
  if (s_last && tid < kWave) prep_walk(pa, b, N, lane, p, d, err_word);
}

// Scan chunk g (= c of row r: logits [c * chunk_len, min(V, (c + 1) *
// chunk_len))) in passes of UNROLL float4 loads per thread, fold it and count
// it in (every thread of the workgroup calls it).
template <int NT, int UNROLL>
__device__ __forceinline__ void prep_chunk(const PrepArgs& pa, int g, int B, int N, uint32_t* err_word) {
  const int tid = threadIdx.x;
  const int r = g / pa.chunks, c = g - r * pa.chunks;
  const float* row = pa.logits + (int64_t)r * pa.row_stride;
  const int64_t V = pa.V;
  const int64_t lo = (int64_t)c * pa.chunk_len;
  const int64_t end = lo + pa.chunk_len;
  ArgBest best{-INFINITY, 0x7fffffff};
  if (pa.vec) {
    const int64_t V4 = V >> 2;
    best = scan_vec4<NT, UNROLL>(row, lo / 4, end / 4 < V4 ? end / 4 : V4, tid, best);
    if (c == pa.chunks - 1) best = scan_scalar<NT>(row, V4 << 2, V, tid, best);
  } else {
    best = scan_scalar<NT>(row, lo, end < V ? end : V, tid, best);
  }
  best = wg_best<NT>(best, tid);
  if (tid == 0) prep_fold(pa, g, best);
  prep_finish<NT>(pa, g, B, N, err_word);
}

// Prep workgroup blk of NT threads (every thread of the workgroup calls it):
// a mask builder, or the scanner of chunk blk - n_mask_wg.
template <int NT, int UNROLL>
__device__ __forceinline__ void prep_block(const PrepArgs& pa, int blk, int B, int N, uint32_t* err_word) {
  const int tid = threadIdx.x;
  const int lane = tid % kWave;

  if (blk < pa.n_mask_wg) {
    const int b = blk * (NT / kWave) + tid / kWave;
    if (b >= B) return;                                // the whole wave leaves; no barrier follows
    const bool live = lane < N;
    const size_t o = (size_t)b * N + lane;
    const int p = live ? pa.parents[o] : 0;
    bool req_bad;
    const uint64_t set = ancestor_set(p, lane, live, err_word, &req_bad);
    if (live) {
      pa.anc_mask[o] = set;
      if (pa.depth) pa.depth[o] = req_bad ? -1 : (__popcll(set) - 1);
    }
    if (pa.mask_counts) {
      // the request's last arrival: usually this wave, after every chunk
      const int d = live ? pa.draft_tokens[o] : 0;
      uint32_t seen = 0;
      if (lane == 0)
        seen = __hip_atomic_fetch_add(pa.req_cnt + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      seen = __shfl(seen, 0, kWave);
      if (seen == prep_arrivals(pa, N) - 1) prep_walk(pa, b, N, lane, p, d, err_word);
    }
    return;
  }
  prep_chunk<NT, UNROLL>(pa, blk - pa.n_mask_wg, B, N, err_word);
}

}  // namespace spectree
