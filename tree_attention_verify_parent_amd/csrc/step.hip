// The whole verify step -- ancestor masks, tree attention, per-node
// vocabulary argmax, accept walk -- in one launch: the attention kernel's grid
// (the split kernel's for bf16 and fp8 caches, contiguous or paged; the fp32
// kernel's) gains the prep workgroups of step_ops.h, and its waves build
// their rows' masks themselves.
#include <mutex>

#include "host_api.h"
#include "step_ops.h"

namespace spectree {

static bool aligned_to(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace spectree

using namespace spectree;

extern "C" size_t spec_verify_step_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int S_max) {
  if (B < 1 || N < 1 || N > SPEC_MAX_NODES) return 0;
  // the attention's part is never empty for sizes it accepts
  const size_t attn = spec_tree_attn_workspace_bytes(B, N, Hq, Hkv, D, S_max);
  return attn ? prep_workspace_bytes(B, N) + attn : 0;
}

namespace spectree {

// The step's own pointers and sizes.
static spec_status step_check(const int32_t* parents, const int32_t* draft_tokens, const float* logits, int64_t V,
                              int64_t logits_row_stride, int B, int N, const uint64_t* anc_mask,
                              const int32_t* target_argmax, const int32_t* accept_len, const int32_t* path_nodes,
                              const int32_t* out_tokens) {
  if (!parents || !draft_tokens || !logits || !anc_mask || !target_argmax || !accept_len || !path_nodes ||
      !out_tokens)
    return SPEC_ERR_NULL;
  if (B < 1 || N < 1 || N > SPEC_MAX_NODES || V < 1 || V > 0x7fffffffLL || logits_row_stride < V)
    return SPEC_ERR_SHAPE;
  return SPEC_OK;
}

// The workspace check (full_ws_bytes: the step's size for these sizes, the
// same for every dtype; the fp32 attention leaves its part unused) and the
// prep arguments; on SPEC_OK *attn_ws / *attn_ws_bytes are the attention's
// part of the workspace.
static spec_status step_place(const int32_t* parents, const int32_t* draft_tokens, const float* logits, int64_t V,
                              int64_t logits_row_stride, int B, int N, size_t full_ws_bytes, uint64_t* anc_mask,
                              int32_t* depth, int32_t* target_argmax, int32_t* accept_len, int32_t* path_nodes,
                              int32_t* out_tokens, void* workspace, size_t workspace_bytes, PrepArgs* pa,
                              void** attn_ws, size_t* attn_ws_bytes) {
  // (0 for sizes the attention rejects: its own check reports them)
  if (!workspace || workspace_bytes < full_ws_bytes) return SPEC_ERR_WORKSPACE;
  if (!aligned_to(workspace, 16)) return SPEC_ERR_ALIGN;
  const size_t prep_bytes = prep_workspace_bytes(B, N);
  *attn_ws = static_cast<char*>(workspace) + prep_bytes;
  *attn_ws_bytes = workspace_bytes - prep_bytes;
  *pa = PrepArgs{};
  pa->parents = parents;
  pa->draft_tokens = draft_tokens;
  pa->logits = logits;
  pa->V = V;
  pa->row_stride = logits_row_stride;
  pa->vec = aligned_to(logits, 16) && (logits_row_stride % 4 == 0);
  pa->anc_mask = anc_mask;
  pa->depth = depth;
  pa->target_argmax = target_argmax;
  pa->accept_len = accept_len;
  pa->path_nodes = path_nodes;
  pa->out_tokens = out_tokens;
  place_prep_workspace(pa, workspace, B, N);
  return SPEC_OK;
}

}  // namespace spectree

extern "C" spec_status spec_verify_step(
    const int32_t* parents, const int32_t* draft_tokens, const int32_t* prefix_lens, const void* q,
    spec_dtype q_dtype, const void* k_cache, const void* v_cache, spec_dtype kv_dtype, const float* k_scale,
    const float* v_scale, const float* logits, int64_t V, int64_t logits_row_stride, int B, int N, int Hq,
    int Hkv, int D, int S_max, float sm_scale, uint64_t* anc_mask, int32_t* depth, void* out, float* lse,
    int32_t* target_argmax, int32_t* accept_len, int32_t* path_nodes, int32_t* out_tokens, void* workspace,
    size_t workspace_bytes, uint32_t* err_word, hipStream_t stream) {
  spec_status st = step_check(parents, draft_tokens, logits, V, logits_row_stride, B, N, anc_mask, target_argmax,
                              accept_len, path_nodes, out_tokens);
  if (st != SPEC_OK) return st;
  PrepArgs pa;
  void* attn_ws;
  size_t attn_ws_bytes;
  st = step_place(parents, draft_tokens, logits, V, logits_row_stride, B, N,
                  spec_verify_step_workspace_bytes(B, N, Hq, Hkv, D, S_max), anc_mask, depth, target_argmax,
                  accept_len, path_nodes, out_tokens, workspace, workspace_bytes, &pa, &attn_ws, &attn_ws_bytes);
  if (st != SPEC_OK) return st;
  // everything the attention would refuse is refused before the first launch
  st = tree_attn_check(q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, prefix_lens, anc_mask, B, N, Hq,
                       Hkv, D, S_max, sm_scale, out, attn_ws, attn_ws_bytes);
  if (st != SPEC_OK) return st;
  if (q_dtype == SPEC_F32)
    return tree_attn_f32_with_prep(q, k_cache, v_cache, prefix_lens, B, N, Hq, Hkv, D, S_max, sm_scale, out, lse,
                                   err_word, pa, stream);
  return tree_attn_verify_with_prep(q, k_cache, v_cache, kv_dtype, k_scale, v_scale, prefix_lens, B, N, Hq, Hkv, D,
                                    S_max, sm_scale, out, lse, attn_ws, attn_ws_bytes, err_word, pa, stream);
}

extern "C" spec_status spec_verify_step_paged(
    const int32_t* parents, const int32_t* draft_tokens, const int32_t* prefix_lens, const void* q,
    spec_dtype q_dtype, const void* k_pages, const void* v_pages, spec_dtype kv_dtype, const float* k_scale,
    const float* v_scale, const int32_t* block_table, int max_pages, int page_size, int num_pages,
    const float* logits, int64_t V, int64_t logits_row_stride, int B, int N, int Hq, int Hkv, int D,
    float sm_scale, uint64_t* anc_mask, int32_t* depth, void* out, float* lse, int32_t* target_argmax,
    int32_t* accept_len, int32_t* path_nodes, int32_t* out_tokens, void* workspace, size_t workspace_bytes,
    uint32_t* err_word, hipStream_t stream) {
  spec_status st = step_check(parents, draft_tokens, logits, V, logits_row_stride, B, N, anc_mask, target_argmax,
                              accept_len, path_nodes, out_tokens);
  if (st != SPEC_OK) return st;
  // the page geometry before the workspace: max_pages * page_size is the
  // attention's S_max only for accepted sizes
  st = tree_attn_paged_check(q, q_dtype, k_pages, v_pages, kv_dtype, k_scale, v_scale, prefix_lens, anc_mask,
                             block_table, max_pages, page_size, num_pages, B, N, Hq, Hkv, D, sm_scale, out);
  if (st != SPEC_OK) return st;
  PrepArgs pa;
  void* attn_ws;
  size_t attn_ws_bytes;
  st = step_place(parents, draft_tokens, logits, V, logits_row_stride, B, N,
                  spec_verify_step_workspace_bytes(B, N, Hq, Hkv, D, max_pages * page_size), anc_mask, depth,
                  target_argmax, accept_len, path_nodes, out_tokens, workspace, workspace_bytes, &pa, &attn_ws,
                  &attn_ws_bytes);
  if (st != SPEC_OK) return st;
  // one launch: every remaining check of the paged attention comes before it
  return tree_attn_verify_paged_run(q, q_dtype, k_pages, v_pages, kv_dtype, k_scale, v_scale, prefix_lens, anc_mask,
                                    block_table, max_pages, page_size, num_pages, B, N, Hq, Hkv, D, sm_scale, out,
                                    lse, attn_ws, attn_ws_bytes, err_word, &pa, stream);
}

// ---- spec_verify_step_static: the step's workspace in a file-scope device
// array instead of the caller's memory, for callers that cannot allocate.
// Each GPU the library runs on holds its own copy until the process ends.
// Host code never uses the array's name as an address: the device address
// comes from hipGetSymbolAddress, once per device.
namespace spectree {

static __device__ __align__(256) unsigned char scratch[SPEC_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];             // per device, set up on its first call

// Zero fill of the whole array with vector stores: a kernel, not a memset,
// and enqueued at set-up only.
__global__ void clear_scratch_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The current device's scratch.  First call on a device: its address, then
// a clear on `stream` (the counters and argmax keys must start at zero;
// every step leaves them at zero again).  Under stream capture the clear is
// not recorded, and the array's zero initialisation at load stands in.
static spec_status static_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPEC_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SPEC_ERR_HIP;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return SPEC_ERR_HIP;
    if (cap == hipStreamCaptureStatusNone) {
      hip_clear_error();
      hipLaunchKernelGGL(clear_scratch_kernel, dim3(1024), dim3(256), 0, stream, static_cast<uint4*>(p),
                         (size_t)SPEC_STATIC_SCRATCH_BYTES / 16);
      if (launch_status() != SPEC_OK) return SPEC_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SPEC_OK;
}

}  // namespace spectree

extern "C" spec_status spec_verify_step_static(
    const int32_t* parents, const int32_t* draft_tokens, const int32_t* prefix_lens, const void* q,
    spec_dtype q_dtype, const void* k_cache, const void* v_cache, spec_dtype kv_dtype, const float* k_scale,
    const float* v_scale, const float* logits, int64_t V, int64_t logits_row_stride, int B, int N, int Hq,
    int Hkv, int D, int S_max, float sm_scale, uint64_t* anc_mask, int32_t* depth, void* out, float* lse,
    int32_t* target_argmax, int32_t* accept_len, int32_t* path_nodes, int32_t* out_tokens, uint32_t* err_word,
    hipStream_t stream) {
  // every argument check before the set-up, so a refused call enqueues nothing
  spec_status st = step_check(parents, draft_tokens, logits, V, logits_row_stride, B, N, anc_mask, target_argmax,
                              accept_len, path_nodes, out_tokens);
  if (st != SPEC_OK) return st;
  st = tree_attn_check_args(q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, prefix_lens, anc_mask, B, N,
                            Hq, Hkv, D, S_max, sm_scale, out);
  if (st != SPEC_OK) return st;
  if (spec_verify_step_workspace_bytes(B, N, Hq, Hkv, D, S_max) > (size_t)SPEC_STATIC_SCRATCH_BYTES)
    return SPEC_ERR_SCRATCH;
  void* ws = nullptr;
  st = static_scratch(stream, &ws);
  if (st != SPEC_OK) return st;
  return spec_verify_step(parents, draft_tokens, prefix_lens, q, q_dtype, k_cache, v_cache, kv_dtype, k_scale,
                          v_scale, logits, V, logits_row_stride, B, N, Hq, Hkv, D, S_max, sm_scale, anc_mask, depth,
                          out, lse, target_argmax, accept_len, path_nodes, out_tokens, ws,
                          (size_t)SPEC_STATIC_SCRATCH_BYTES, err_word, stream);
}
