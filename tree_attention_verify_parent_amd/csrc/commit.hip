// Commit step after verification (gfx950).
//
// Each verification ends with the accepted draft tokens and, for every
// proposed token, whether the target accepted or rejected it: the record the
// serving engine streams on (Aurora, section 2, the inference server and the
// mapping of accepted tokens and rejected proposals to rewards).  Here the
// cache keeps the prefix, the root (node 0, row P) and the accepted nodes in
// path order, the node at depth k moving to row P + k, and every node gets an
// outcome label.
//
// One workgroup per (request, kv head).  The accepted path satisfies
// path[k] >= k, so a destination row can be the source of an earlier depth:
// every source row is staged in LDS before any destination is written.  The
// copy is a few rows per request; the launch is latency-bound.
//
// Paged caches (the layout of the paged attention: token t of request b in
// page table[b][t / page_size], slot t % page_size, each token a [Hkv][D]
// block): the same moves through the block table.  This kernel writes, so a
// request whose tree tokens touch a page id outside the pool is flagged and
// left unchanged (the attention reads page 0 in its place instead).
#include "common.h"

namespace spectree {

constexpr int kCommitThreads = 256;

// Paged cache description (null table: contiguous caches).
struct CommitPages {
  const int32_t* table;
  int max_pages, ps_log2, num_pages;
};

template <bool PAGED>
__global__ __launch_bounds__(kCommitThreads) void commit_accepted_kernel(
    unsigned char* __restrict__ kc, unsigned char* __restrict__ vc, int row_bytes,
    const int32_t* __restrict__ prefix_lens, const int32_t* __restrict__ accept_len,
    const int32_t* __restrict__ path_nodes, int N, int Hkv, int S_max,
    int32_t* __restrict__ new_prefix, int8_t* __restrict__ labels, uint32_t* __restrict__ err_word,
    const CommitPages pg) {
  extern __shared__ uint4 stage[];                 // [2][L][row_bytes / 16]: K rows, then V rows
  __shared__ int s_path[SPEC_MAX_NODES];
  __shared__ int s_page[SPEC_MAX_NODES];           // paged: ids of the pages of tokens P .. P+N-1
  __shared__ int s_bad, s_bad_page;
  const int b = blockIdx.x / Hkv;
  const int kvh = blockIdx.x % Hkv;
  const int tid = threadIdx.x;
  const int P = prefix_lens[b];
  const int L = accept_len[b];
  const bool bad_prefix = P < 0 || P > S_max - N;
  const bool bad_len = L < 0 || L > N - 1;
  if (tid == 0) {
    s_bad = 0;
    s_bad_page = 0;
  }
  __syncthreads();
  if (!bad_len && tid <= L) {
    const int node = path_nodes[(size_t)b * N + tid];
    s_path[tid] = node;
    // the root first, then strictly increasing node indices inside the tree
    const int prev = (tid == 0) ? -1 : path_nodes[(size_t)b * N + tid - 1];
    if ((tid == 0 && node != 0) || (tid > 0 && !(prev < node && node < N))) atomicOr(&s_bad, 1);
  }
  const int pg0 = PAGED && !bad_prefix ? (P >> pg.ps_log2) : 0;
  if constexpr (PAGED) {
    const int np = bad_prefix ? 0 : ((P + N - 1) >> pg.ps_log2) - pg0 + 1;   // at most N pages
    if (tid < np) {
      const int id = pg.table[(size_t)b * pg.max_pages + pg0 + tid];
      s_page[tid] = id;
      if (id < 0 || id >= pg.num_pages) atomicOr(&s_bad_page, 1);
    }
  }
  __syncthreads();
  if (bad_prefix || bad_len || s_bad || s_bad_page) {
    if (kvh == 0 && tid == 0)
      flag_error(err_word, (bad_prefix ? SPEC_DERR_PREFIX : 0u) | ((bad_len || s_bad) ? SPEC_DERR_PATH : 0u) |
                               (s_bad_page ? SPEC_DERR_PAGE : 0u));
    return;
  }
  if (kvh == 0) {
    if (tid == 0) new_prefix[b] = P + 1 + L;
    if (labels)
      for (int i = tid; i < N; i += kCommitThreads) {
        // node i is accepted iff it is on the path; the path is increasing,
        // so at most one k has s_path[k] == i
        int8_t lab = (i == 0) ? int8_t(2) : int8_t(0);
        for (int k = 1; k <= L; ++k) lab = (s_path[k] == i) ? int8_t(1) : lab;
        labels[(size_t)b * N + i] = lab;
      }
  }
  // rows already in place (a fully accepted chain) need no copy
  bool moves = false;
  for (int k = 1; k <= L; ++k) moves = moves || (s_path[k] != k);
  if (!moves) return;
  const int U = row_bytes / 16;                    // 16-byte units per row
  // the 16-byte unit index of token t's row (this request, this kv head)
  auto row_unit = [&](int t) -> size_t {
    if constexpr (PAGED) {
      const size_t page = (size_t)s_page[(t >> pg.ps_log2) - pg0];
      const size_t slot = (size_t)(t & ((1 << pg.ps_log2) - 1));
      return (((page << pg.ps_log2) | slot) * Hkv + kvh) * U;
    } else {
      return ((size_t)(b * Hkv + kvh) * S_max + t) * U;
    }
  };
  const uint4* ksrc = reinterpret_cast<const uint4*>(kc);
  const uint4* vsrc = reinterpret_cast<const uint4*>(vc);
  const int total = L * U;
  for (int idx = tid; idx < total; idx += kCommitThreads) {
    const int k = idx / U + 1, un = idx % U;
    const size_t src = row_unit(P + s_path[k]) + un;
    stage[idx] = ksrc[src];
    stage[total + idx] = vsrc[src];
  }
  __syncthreads();
  uint4* kdst = reinterpret_cast<uint4*>(kc);
  uint4* vdst = reinterpret_cast<uint4*>(vc);
  for (int idx = tid; idx < total; idx += kCommitThreads) {
    const int k = idx / U + 1, un = idx % U;
    const size_t dst = row_unit(P + k) + un;
    kdst[dst] = stage[idx];
    vdst[dst] = stage[total + idx];
  }
}

}  // namespace spectree

using namespace spectree;

static spec_status commit_launch(void* k_cache, void* v_cache, spec_dtype kv_dtype, const int32_t* prefix_lens,
                                 const int32_t* accept_len, const int32_t* path_nodes, int B, int N, int Hkv, int D,
                                 int S_max, int32_t* new_prefix_lens, int8_t* node_labels, uint32_t* err_word,
                                 const CommitPages& pg, hipStream_t stream) {
  if (!k_cache || !v_cache || !prefix_lens || !accept_len || !path_nodes || !new_prefix_lens)
    return SPEC_ERR_NULL;
  if (B < 1 || N < 1 || N > SPEC_MAX_NODES || Hkv < 1 || (D != 64 && D != 128) || S_max < N) return SPEC_ERR_SHAPE;
  int eb;
  switch (kv_dtype) {
    case SPEC_F32: eb = 4; break;
    case SPEC_BF16: eb = 2; break;
    case SPEC_FP8_E4M3: eb = 1; break;
    default: return SPEC_ERR_DTYPE;
  }
  if ((reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) & 15u) return SPEC_ERR_ALIGN;
  if ((long long)B * Hkv >= (1ll << 31)) return SPEC_ERR_SHAPE;
  const int row_bytes = D * eb;
  const size_t lds = (size_t)2 * (N - 1) * row_bytes;          // at most N - 1 accepted rows
  hip_clear_error();
  if (pg.table)
    hipLaunchKernelGGL(commit_accepted_kernel<true>, dim3((unsigned)(B * Hkv)), dim3(kCommitThreads), lds, stream,
                       static_cast<unsigned char*>(k_cache), static_cast<unsigned char*>(v_cache), row_bytes,
                       prefix_lens, accept_len, path_nodes, N, Hkv, S_max, new_prefix_lens, node_labels, err_word,
                       pg);
  else
    hipLaunchKernelGGL(commit_accepted_kernel<false>, dim3((unsigned)(B * Hkv)), dim3(kCommitThreads), lds, stream,
                       static_cast<unsigned char*>(k_cache), static_cast<unsigned char*>(v_cache), row_bytes,
                       prefix_lens, accept_len, path_nodes, N, Hkv, S_max, new_prefix_lens, node_labels, err_word,
                       pg);
  return launch_status();
}

extern "C" spec_status spec_commit_accepted(void* k_cache, void* v_cache, spec_dtype kv_dtype,
                                            const int32_t* prefix_lens, const int32_t* accept_len,
                                            const int32_t* path_nodes, int B, int N, int Hkv, int D,
                                            int S_max, int32_t* new_prefix_lens, int8_t* node_labels,
                                            uint32_t* err_word, hipStream_t stream) {
  return commit_launch(k_cache, v_cache, kv_dtype, prefix_lens, accept_len, path_nodes, B, N, Hkv, D, S_max,
                       new_prefix_lens, node_labels, err_word, CommitPages{nullptr, 0, 0, 0}, stream);
}

extern "C" spec_status spec_commit_accepted_paged(void* k_pages, void* v_pages, spec_dtype kv_dtype,
                                                  const int32_t* block_table, int max_pages, int page_size,
                                                  int num_pages, const int32_t* prefix_lens,
                                                  const int32_t* accept_len, const int32_t* path_nodes, int B,
                                                  int N, int Hkv, int D, int32_t* new_prefix_lens,
                                                  int8_t* node_labels, uint32_t* err_word, hipStream_t stream) {
  if (!block_table) return SPEC_ERR_NULL;
  if (page_size < 1 || (page_size & (page_size - 1)) || page_size > 4096) return SPEC_ERR_SHAPE;
  if (max_pages < 1 || max_pages > 2048 || num_pages < 1) return SPEC_ERR_SHAPE;   // the paged attention's bounds
  if ((long long)num_pages * page_size * Hkv * D >= (1ll << 40)) return SPEC_ERR_SHAPE;
  int ps_log2 = 0;
  while ((1 << ps_log2) < page_size) ++ps_log2;
  return commit_launch(k_pages, v_pages, kv_dtype, prefix_lens, accept_len, path_nodes, B, N, Hkv, D,
                       max_pages * page_size, new_prefix_lens, node_labels, err_word,
                       CommitPages{block_table, max_pages, ps_log2, num_pages}, stream);
}
