// Host-side functions that one source file of the library exposes to another
// (not part of the C ABI).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "spectree.h"

#include <hip/hip_runtime_api.h>

namespace spectree {

struct PrepArgs;

// SPEC_OK when spec_tree_attn_verify would accept these arguments, else the
// status it would return without launching anything.
spec_status tree_attn_check(const void* q, spec_dtype q_dtype, const void* k_cache, const void* v_cache,
                            spec_dtype kv_dtype, const float* k_scale, const float* v_scale,
                            const int32_t* prefix_lens, const uint64_t* anc_mask, int B, int N, int Hq,
                            int Hkv, int D, int S_max, float sm_scale, const void* out, const void* workspace,
                            size_t workspace_bytes);

// tree_attn_check without the workspace: every other reason it can refuse.
spec_status tree_attn_check_args(const void* q, spec_dtype q_dtype, const void* k_cache, const void* v_cache,
                                 spec_dtype kv_dtype, const float* k_scale, const float* v_scale,
                                 const int32_t* prefix_lens, const uint64_t* anc_mask, int B, int N, int Hq,
                                 int Hkv, int D, int S_max, float sm_scale, const void* out);

// spec_tree_attn_verify for bf16 or decoded-fp8 caches (arguments already
// accepted by tree_attn_check), with the verify step's prep role (masks,
// argmax, accept walk) added to the same launch.
spec_status tree_attn_verify_with_prep(const void* q, const void* k_cache, const void* v_cache, spec_dtype kv_dtype,
                                       const float* k_scale, const float* v_scale, const int32_t* prefix_lens,
                                       int B, int N, int Hq, int Hkv, int D, int S_max, float sm_scale, void* out,
                                       float* lse, void* workspace, size_t workspace_bytes, uint32_t* err_word,
                                       const PrepArgs& prep, hipStream_t stream);

// spec_tree_attn_verify for fp32 (arguments already accepted by
// tree_attn_check), with the verify step's prep role in the same launch.
spec_status tree_attn_f32_with_prep(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* prefix_lens, int B, int N, int Hq, int Hkv, int D, int S_max,
                                    float sm_scale, void* out, float* lse, uint32_t* err_word, const PrepArgs& prep,
                                    hipStream_t stream);

// SPEC_OK when spec_tree_attn_verify_paged would accept these arguments
// (workspace aside), else the status it would return without launching.
spec_status tree_attn_paged_check(const void* q, spec_dtype q_dtype, const void* k_pages, const void* v_pages,
                                  spec_dtype kv_dtype, const float* k_scale, const float* v_scale,
                                  const int32_t* prefix_lens, const uint64_t* anc_mask, const int32_t* block_table,
                                  int max_pages, int page_size, int num_pages, int B, int N, int Hq, int Hkv, int D,
                                  float sm_scale, const void* out);

// spec_tree_attn_verify_paged; with prep non-null the verify step's prep
// role joins the same launch.
spec_status tree_attn_verify_paged_run(const void* q, spec_dtype q_dtype, const void* k_pages, const void* v_pages,
                                       spec_dtype kv_dtype, const float* k_scale, const float* v_scale,
                                       const int32_t* prefix_lens, const uint64_t* anc_mask,
                                       const int32_t* block_table, int max_pages, int page_size, int num_pages, int B,
                                       int N, int Hq, int Hkv, int D, float sm_scale, void* out, float* lse,
                                       void* workspace, size_t workspace_bytes, uint32_t* err_word,
                                       const PrepArgs* prep, hipStream_t stream);

}  // namespace spectree
