// Host-side entry of the backward pass for more than 128 packed rows
// (tree_attn_bwd_wide.hip), for spec_tree_attn_backward (not part of the C ABI).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "spectree.h"

#include <hip/hip_runtime_api.h>

namespace spectree {

// Row statistics, then the dq pass, then the dK / dV pass (arguments already
// checked; bf16).  The workspace holds bwd_wide_workspace_bytes(B, N, Hq)
// bytes: D and lse * log2(e) of every (request, node, head) row.
size_t bwd_wide_workspace_bytes(int B, int N, int Hq);
spec_status bwd_wide_launch(const void* q, const void* k, const void* v, const int32_t* prefix_lens,
                            const uint64_t* anc_mask, const void* out, const float* lse, const void* dout, int B,
                            int N, int Hq, int Hkv, int D, int S_max, float sm_scale, void* dq, void* dk, void* dv,
                            void* workspace, uint32_t* err_word, hipStream_t stream);

}  // namespace spectree
