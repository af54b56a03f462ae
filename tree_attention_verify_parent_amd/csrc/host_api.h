// Host-side functions that one source file of the library exposes to another
// (not part of the C ABI).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "spectree.h"

namespace spectree {

// SPEC_OK when spec_tree_attn_verify would accept these arguments, else the
// status it would return without launching anything.
spec_status tree_attn_check(const void* q, spec_dtype q_dtype, const void* k_cache, const void* v_cache,
                            spec_dtype kv_dtype, const float* k_scale, const float* v_scale,
                            const int32_t* prefix_lens, const uint64_t* anc_mask, int B, int N, int Hq,
                            int Hkv, int D, int S_max, float sm_scale, const void* out, const void* workspace,
                            size_t workspace_bytes);

}  // namespace spectree
