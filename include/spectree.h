/*
 * spectree -- speculative-decoding tree verify step for AMD CDNA4 (gfx950).
 *
 * A draft model proposes a tree of tokens; the target model checks the whole
 * tree in one parallel pass and keeps the longest prefix it agrees with
 * (Aurora, chernovdev.ru / everytik.com mirrors, section 2 "serve-to-train
 * flywheel": the inference server verifies the draft's proposal in parallel;
 * Runtime Draft Model Training, moreh.io, "Overview").  One verify step is:
 *
 *   spec_tree_mask_build   parent array -> 64-bit ancestor-or-self masks
 *   spec_tree_attn_verify  tree-masked split-KV attention over the KV cache
 *   spec_vocab_argmax      per-node argmax of the target logits
 *   spec_accept_walk       longest matched root-to-node path -> accepted tokens
 *   spec_commit_accepted   (after the step) keep the accepted path's K/V, label outcomes
 *   spec_commit_accepted_paged  the same over a paged cache
 *   spec_tree_attn_backward (training) gradients of the tree-masked attention
 *   spec_tree_attn_verify_f8 the attention in fp8 arithmetic over an e4m3 cache
 *   spec_tree_attn_verify_f4 ... over an e2m1 (FP4) cache
 *   spec_verify_step       mask, attention, argmax and accept walk in one launch
 *   spec_verify_step_paged the same over a paged cache
 *
 * Conventions shared by every entry point
 *   - Every array argument is DEVICE memory owned by the caller.  The library
 *     never allocates, frees or synchronises; each call validates its host-side
 *     arguments, enqueues kernels on `stream` and returns.
 *   - Inputs are read only; outputs are fully overwritten.  Inputs and outputs
 *     must not alias.
 *   - A non-SPEC_OK return means nothing was enqueued (except SPEC_ERR_HIP,
 *     which reports a failed launch).
 *   - Errors that only the data can show are found on the device and OR'ed
 *     into *err_word (nullable; the caller zeroes it before the call and reads
 *     it after synchronising).  A request whose data is flagged gets
 *     unspecified outputs; other requests are unaffected.
 *   - Calls are thread safe; the library holds no state.
 *
 * Tree layout (a reading: the pages describe the mask only as following "the
 * causal structure of the speculative tree", Aurora section 2, closing
 * paragraph): request b has N nodes, parents[b][0] == -1 is the root (the
 * last committed token) and 0 <= parents[b][i] < i.  A node attends to the
 * request's whole KV prefix plus its ancestors and itself.
 */
#ifndef SPECTREE_H
#define SPECTREE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Both enums are int-sized.  In C++ they get int as their fixed underlying
 * type, so any int a C caller passes (say an unknown dtype) is a value of
 * the type, which the library then rejects with a status. */
#ifdef __cplusplus
#define SPEC_ENUM_INT : int
#else
#define SPEC_ENUM_INT
#endif

typedef enum SPEC_ENUM_INT {
  SPEC_OK = 0,
  SPEC_ERR_NULL = 1,      /* a required pointer is NULL                         */
  SPEC_ERR_SHAPE = 2,     /* a size is out of range or inconsistent             */
  SPEC_ERR_DTYPE = 3,     /* unsupported dtype or dtype pair                    */
  SPEC_ERR_WORKSPACE = 4, /* workspace missing or smaller than required         */
  SPEC_ERR_HIP = 5,       /* a kernel launch failed                             */
  SPEC_ERR_ALIGN = 6,     /* a pointer is not 16-byte aligned where required    */
  SPEC_ERR_SCRATCH = 7    /* the sizes need more than the static scratch holds  */
} spec_status;

typedef enum SPEC_ENUM_INT {
  SPEC_F32 = 0,
  SPEC_BF16 = 1,
  SPEC_FP8_E4M3 = 2,      /* OCP FP8 E4M3 ("e4m3fn"): bias 7, no inf, max 448 */
  SPEC_FP4_E2M1 = 3       /* OCP FP4 E2M1: two codes per byte, element 2j in the
                             low nibble of byte j; values 0, .5, 1, 1.5, 2, 3, 4, 6 */
} spec_dtype;

/* Device-detected data errors, OR'ed into *err_word. */
#define SPEC_DERR_ROOT   1u  /* parents[b][0] != -1                          */
#define SPEC_DERR_PARENT 2u  /* parents[b][i] not in [0, i) for some i >= 1   */
#define SPEC_DERR_PREFIX 4u  /* prefix_lens[b] < 0 or prefix_lens[b]+N > S_max */
#define SPEC_DERR_TOKEN  8u  /* a draft token or target argmax not in [0, V)  */
#define SPEC_DERR_PATH  16u  /* accept_len not in [0, N-1], or the accepted
                                path is not root-first, increasing, in [0, N) */
#define SPEC_DERR_PAGE  32u  /* a block-table entry a request uses is not in
                                [0, num_pages)                                 */

#define SPEC_MAX_NODES 64

/*
 * spec_tree_mask_build -- ancestor-or-self bitmasks of each draft tree.
 *
 * The custom attention mask that follows the speculative tree's causal
 * structure (Aurora section 2, closing paragraph on tree attention), packed
 * as one 64-bit word per node.
 *
 *   parents   int32[B][N]   parent index of each node (see tree layout above)
 *   B         >= 1          requests
 *   N         1..64         nodes per request
 *   anc_mask  uint64[B][N]  out: bit j of anc_mask[b][i] set iff node j is node
 *                           i or one of its ancestors
 *   depth     int32[B][N]   out, nullable: edges from the root to node i
 *   err_word  uint32*       nullable: SPEC_DERR_ROOT / SPEC_DERR_PARENT
 *   stream    HIP stream to enqueue on
 */
spec_status spec_tree_mask_build(const int32_t* parents, int B, int N,
                                 uint64_t* anc_mask, int32_t* depth,
                                 uint32_t* err_word, hipStream_t stream);

/*
 * spec_tree_attn_workspace_bytes -- scratch needed by spec_tree_attn_verify
 * for these sizes (any cache dtype).  Pure function of its arguments; returns
 * 0 for sizes spec_tree_attn_verify would reject.  The fp32 path uses none of
 * it.
 */
size_t spec_tree_attn_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int S_max);

/*
 * spec_tree_attn_verify -- tree-masked attention of every draft node.
 *
 * The target model checks all proposed tokens in one parallel pass (Runtime
 * Draft Model Training, "Overview"), each node's query seeing the request's
 * KV-cache prefix plus only its own ancestors and itself (Aurora section 2,
 * tree attention).  For request b, node i, query head h, kv head
 * kvh = h / (Hq/Hkv), with P = prefix_lens[b]:
 *     keys c in [0, P)                        : the prefix, always visible
 *     keys c = P + j, j in [0, N)             : tree node j, visible iff bit j
 *                                               of anc_mask[b][i] is set
 *     s_c = sm_scale * <q[b][i][h], K[b][kvh][c]>
 *     out[b][i][h] = sum_c softmax(s)_c * V[b][kvh][c]
 *     lse[b][i][h] = log sum_c exp(s_c)
 * Cache rows >= P + N are never read.
 *
 *   B          1..1024 requests, with B*S_max and Hkv*S_max below 2^31
 *   q          [B][N][Hq][D] of q_dtype (SPEC_F32 or SPEC_BF16), 16-B aligned
 *   k_cache,
 *   v_cache    [B][Hkv][S_max][D] of kv_dtype, 16-B aligned; tree node j of
 *              request b is row prefix_lens[b] + j
 *   k_scale,
 *   v_scale    float[Hkv]: per-KV-head dequantisation scales; required iff
 *              kv_dtype == SPEC_FP8_E4M3 (K = code * k_scale[kvh]), else ignored
 *   prefix_lens int32[B]
 *   anc_mask   uint64[B][N] from spec_tree_mask_build
 *   D          64 or 128
 *   sm_scale   softmax scale, finite and > 0 (typically 1/sqrt(D))
 *   out        [B][N][Hq][D] of q_dtype, 16-B aligned
 *   lse        float[B][N][Hq], nullable
 *   workspace  >= spec_tree_attn_workspace_bytes(...) bytes, 16-B aligned;
 *              may be NULL when that size is 0.  It must be zero-filled
 *              before its first use; every call leaves it ready for the next
 *              one (its split counters back at zero), so it can be reused
 *              without clearing.  Calls that overlap in time (other streams)
 *              must not share one workspace.
 *   err_word   nullable: SPEC_DERR_PREFIX
 * Supported (q_dtype, kv_dtype): (F32, F32), (BF16, BF16), (BF16, FP8_E4M3).
 * Results are deterministic: the split-K merge runs in a fixed order.
 * Work is cut into about one unit per resident workgroup: fixed splits of
 * S_max when every request fills its cache (prefix_lens[b] == S_max - N),
 * otherwise equal shares of the actual tokens; the kernel picks from the data.
 * A request spread over several workgroups is merged, in the same launch, by
 * the last of them to finish.
 */
spec_status spec_tree_attn_verify(const void* q, spec_dtype q_dtype,
                                  const void* k_cache, const void* v_cache, spec_dtype kv_dtype,
                                  const float* k_scale, const float* v_scale,
                                  const int32_t* prefix_lens, const uint64_t* anc_mask,
                                  int B, int N, int Hq, int Hkv, int D, int S_max,
                                  float sm_scale, void* out, float* lse,
                                  void* workspace, size_t workspace_bytes,
                                  uint32_t* err_word, hipStream_t stream);

/*
 * spec_tree_attn_verify_paged -- spec_tree_attn_verify over a paged cache.
 *
 * The verify pass runs inside a serving engine (SGLang or vLLM: Aurora,
 * section 2, the inference server) whose K/V caches are paged.  A reading of
 * that layout: a pool of pages of page_size tokens, token-major (each token a
 * [Hkv][D] block); request b's logical token t is in page
 * block_table[b][t / page_size], slot t % page_size.  Everything else --
 * tree layout (node j at logical token prefix_lens[b] + j), mask, outputs,
 * dtypes, workspace (query spec_tree_attn_workspace_bytes with
 * S_max = max_pages * page_size) and errors -- is as in spec_tree_attn_verify.
 *
 *   k_pages,
 *   v_pages      [num_pages][page_size][Hkv][D] of kv_dtype (SPEC_BF16 or
 *                SPEC_FP8_E4M3; q_dtype SPEC_BF16), 16-B aligned
 *   block_table  int32[B][max_pages], 1 <= max_pages <= 2048
 *   page_size    a power of two, 1..4096
 *   err_word     nullable: SPEC_DERR_PREFIX; SPEC_DERR_PAGE for an entry a
 *                request uses outside [0, num_pages) (it reads page 0 instead)
 */
spec_status spec_tree_attn_verify_paged(const void* q, spec_dtype q_dtype,
                                        const void* k_pages, const void* v_pages, spec_dtype kv_dtype,
                                        const float* k_scale, const float* v_scale,
                                        const int32_t* prefix_lens, const uint64_t* anc_mask,
                                        const int32_t* block_table, int max_pages, int page_size,
                                        int num_pages, int B, int N, int Hq, int Hkv, int D,
                                        float sm_scale, void* out, float* lse,
                                        void* workspace, size_t workspace_bytes,
                                        uint32_t* err_word, hipStream_t stream);

/*
 * spec_vocab_argmax -- per-row argmax of float32 logits.
 *
 * Under greedy verification the target's token at a node is the argmax of
 * its logits (the target "verifies" the draft: Aurora section 2).  Ties go
 * to the lowest index; -0.0 and +0.0 compare equal.  Logits must be finite.
 *
 *   logits     float[rows][row_stride], row r's V logits at logits + r*row_stride
 *   rows       >= 1;  V >= 1;  row_stride >= V
 *   out_idx    int32[rows]
 */
spec_status spec_vocab_argmax(const float* logits, int64_t rows, int64_t V, int64_t row_stride,
                              int32_t* out_idx, hipStream_t stream);

/*
 * spec_accept_walk -- accepted path, tokens and acceptance length per request.
 *
 * Acceptance length is the number of draft tokens the target accepts in one
 * verification step (Runtime Draft Model Training, "Evaluation").  Node
 * i >= 1 matches when draft_tokens[b][i] == target_argmax[b][parents[b][i]];
 * a node is accepted when every node on its root path (root excluded)
 * matches; the accepted path ends at the deepest accepted node, ties going to
 * the lowest node index.
 *
 *   parents        int32[B][N]
 *   anc_mask       uint64[B][N] from spec_tree_mask_build
 *   draft_tokens   int32[B][N]  (node 0's token is never compared)
 *   target_argmax  int32[B][N]  (spec_vocab_argmax of the [B*N][V] logits)
 *   V              vocabulary size (token range check)
 *   accept_len     int32[B]     out: L = accepted draft tokens, 0 <= L <= depth
 *   path_nodes     int32[B][N]  out: node at depth k of the path, k = 0..L; -1 after
 *   out_tokens     int32[B][N]  out: target_argmax along the path, k = 0..L (the
 *                               L accepted tokens, then the bonus token); -1 after
 *   err_word       nullable: SPEC_DERR_ROOT / _PARENT / _TOKEN
 */
spec_status spec_accept_walk(const int32_t* parents, const uint64_t* anc_mask,
                             const int32_t* draft_tokens, const int32_t* target_argmax,
                             int B, int N, int V,
                             int32_t* accept_len, int32_t* path_nodes, int32_t* out_tokens,
                             uint32_t* err_word, hipStream_t stream);

/*
 * spec_commit_accepted -- keep the accepted path in the cache, label outcomes.
 *
 * The step after verification: the accepted and rejected outcomes of every
 * proposed token are the record the serving engine streams on (Aurora,
 * section 2, the inference server, and the mapping of accepted tokens and
 * rejected proposals to positive and negative feedback).  A reading of it
 * for the cache: it keeps the prefix, the root (node 0, row P) and the
 * accepted draft nodes in path order, so the node at depth k of the accepted
 * path moves to row P + k (k = 1..L); rows past P + L are left as they were
 * and are free for the next tree.  The bonus token has no K/V yet.
 *
 *   k_cache,
 *   v_cache         [B][Hkv][S_max][D] of kv_dtype (any of the three), 16-B
 *                   aligned; updated in place
 *   prefix_lens     int32[B]   P of each request before this step
 *   accept_len      int32[B]   L from spec_accept_walk
 *   path_nodes      int32[B][N] from spec_accept_walk (entries 0..L read)
 *   D               64 or 128
 *   new_prefix_lens int32[B]   out: P + 1 + L (prefix, root, accepted tokens)
 *   node_labels     int8[B][N] out, nullable: 2 root, 1 accepted draft node,
 *                   0 rejected draft node
 *   err_word        nullable: SPEC_DERR_PREFIX / SPEC_DERR_PATH; a flagged
 *                   request's cache rows and outputs are left unchanged
 */
spec_status spec_commit_accepted(void* k_cache, void* v_cache, spec_dtype kv_dtype,
                                 const int32_t* prefix_lens, const int32_t* accept_len,
                                 const int32_t* path_nodes, int B, int N, int Hkv, int D, int S_max,
                                 int32_t* new_prefix_lens, int8_t* node_labels,
                                 uint32_t* err_word, hipStream_t stream);

/*
 * spec_commit_accepted_paged -- spec_commit_accepted over a paged cache.
 *
 * The same step for the serving engine whose caches are paged (Aurora,
 * section 2), in the page layout of spec_tree_attn_verify_paged: request b's
 * logical row t is slot t % page_size of page block_table[b][t / page_size].
 * The moves, outputs and errors are those of spec_commit_accepted on the
 * logical rows (S_max = max_pages * page_size); pages are never allocated,
 * freed or reordered.
 *
 *   k_pages,
 *   v_pages      [num_pages][page_size][Hkv][D] of kv_dtype (any of the
 *                three), 16-B aligned; updated in place
 *   block_table  int32[B][max_pages], 1 <= max_pages <= 2048
 *   page_size    a power of two, 1..4096
 *   err_word     nullable: as spec_commit_accepted, plus SPEC_DERR_PAGE when
 *                a page holding one of the request's tree rows (P .. P+N-1)
 *                is outside [0, num_pages); that request is left unchanged
 */
spec_status spec_commit_accepted_paged(void* k_pages, void* v_pages, spec_dtype kv_dtype,
                                       const int32_t* block_table, int max_pages, int page_size, int num_pages,
                                       const int32_t* prefix_lens, const int32_t* accept_len,
                                       const int32_t* path_nodes, int B, int N, int Hkv, int D,
                                       int32_t* new_prefix_lens, int8_t* node_labels,
                                       uint32_t* err_word, hipStream_t stream);

/*
 * spec_tree_attn_verify_f8 -- the same attention in fp8 arithmetic, for e4m3
 * caches.
 *
 * The pages count numeric precision (FP8 / FP4) among what decides real
 * serving speed (Aurora, section 1, on acceptance rate versus speed-up).
 * This variant computes spec_tree_attn_verify's result for an e4m3 cache
 * with both products on the fp8 matrix cores:
 *     K, V        the cache's e4m3 codes as they are (no decode)
 *     q           each (node, head) row quantized to e4m3 with its own scale
 *                 amax(|row|) / 448 (round to nearest even)
 *     p           exp(s - running row max) quantized as e4m3(p * 2^8)
 *     sums        fp32; the softmax denominator sums the unquantized p
 * OUTSIDE THE PARITY CONTRACT of spec_tree_attn_verify: the e4m3 roundings
 * of q and p (3 mantissa bits) put the result about 3% (relative L2) from
 * the exact attention, above the contract's 1e-2 relative-L2 guard (it
 * stays within 5e-2).  Each element is within 2^-3 of the largest |V| its
 * row sees; with at least 64 prefix tokens per request also within the
 * fp8-cache bound 6e-2 + 1e-2 |exact|, which prefixes of a few tokens can
 * exceed.  Use spec_tree_attn_verify where the contract must hold.
 *
 *   Arguments as spec_tree_attn_verify with q_dtype = SPEC_BF16 and
 *   kv_dtype = SPEC_FP8_E4M3 (k_scale, v_scale required), D = 128 only; the
 *   same workspace size (spec_tree_attn_workspace_bytes) and rules.
 */
spec_status spec_tree_attn_verify_f8(const void* q, const void* k_cache, const void* v_cache,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* prefix_lens, const uint64_t* anc_mask,
                                     int B, int N, int Hq, int Hkv, int D, int S_max,
                                     float sm_scale, void* out, float* lse,
                                     void* workspace, size_t workspace_bytes,
                                     uint32_t* err_word, hipStream_t stream);

/*
 * spec_tree_attn_verify_f8_scores -- spec_tree_attn_verify over bf16 caches
 * with the scores on the fp8 matrix cores (16x16x128 e4m3 MFMA).
 * OUTSIDE THE PARITY CONTRACT: q is rounded per row to e4m3 (as in
 * spec_tree_attn_verify_f8) and each K tile, once per workgroup in LDS, to
 * e4m3 codes K / kq; the probabilities and V stay bf16, so only the scores
 * are rounded (both operands to 3 mantissa bits: a few percent relative L2
 * against the exact attention on the test data).
 *
 *   q, out        [B][N][Hq][D] bf16, 16-B aligned
 *   k_cache,
 *   v_cache       [B][Hkv][S_max][D] bf16, 16-B aligned
 *   k_scale       nullable float[Hkv]: kq for kv head h is the power of two
 *                 of k_scale[h] (its exponent; positive normal floats);
 *                 NULL means kq = 1.  Precondition: |K| < 448 kq, else the
 *                 codes are NaN.
 *   D             128
 * Other arguments, workspace and results as spec_tree_attn_verify.
 */
spec_status spec_tree_attn_verify_f8_scores(const void* q, const void* k_cache, const void* v_cache,
                                            const float* k_scale, const int32_t* prefix_lens,
                                            const uint64_t* anc_mask, int B, int N, int Hq, int Hkv, int D,
                                            int S_max, float sm_scale, void* out, float* lse,
                                            void* workspace, size_t workspace_bytes,
                                            uint32_t* err_word, hipStream_t stream);

/*
 * spec_tree_attn_verify_f4 -- the same attention over an e2m1 (FP4) cache,
 * in the fp8 arithmetic of spec_tree_attn_verify_f8.
 *
 * FP4 is the other precision the pages name (Aurora, section 1).  The
 * cache holds OCP E2M1 codes, two a byte (element 2j in the low nibble of
 * byte j), with one fp32 scale per KV head for K and one for V (the same
 * scheme as the e4m3 cache): K = code * k_scale[kvh].  The codes are the A
 * operands of e2m1 x e4m3 matrix-core products; q and p are quantized to
 * e4m3 exactly as in spec_tree_attn_verify_f8, and like it this variant
 * lies outside the parity contract (about 3% relative L2 from the exact
 * attention of the same cache).  The cache moves half the bytes of an e4m3
 * one.
 *
 *   k_cache,
 *   v_cache    [B][Hkv][S_max][D/2] bytes, 16-B aligned
 *   Other arguments as spec_tree_attn_verify_f8 (D = 128 only; the same
 *   workspace size and rules).
 */
spec_status spec_tree_attn_verify_f4(const void* q, const void* k_cache, const void* v_cache,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* prefix_lens, const uint64_t* anc_mask,
                                     int B, int N, int Hq, int Hkv, int D, int S_max,
                                     float sm_scale, void* out, float* lse,
                                     void* workspace, size_t workspace_bytes,
                                     uint32_t* err_word, hipStream_t stream);

/*
 * spec_tree_attn_backward_workspace_bytes -- scratch needed by
 * spec_tree_attn_backward for these sizes.  Pure function of its arguments;
 * 0 when the sizes need none or would be rejected.
 */
size_t spec_tree_attn_backward_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int S_max);

/*
 * spec_tree_attn_backward -- gradients of spec_tree_attn_verify's attention.
 *
 * The draft model is trained on all accepted and rejected branches of a
 * verification in one batched forward and backward pass under the same tree
 * mask (Aurora, section 2, closing paragraph).  With the notation of
 * spec_tree_attn_verify (keys c < L = P + N of request b, kv head kvh, the
 * mask, sm_scale) and the upstream gradient dO of every output row, this
 * returns the gradients of  sum_{b,i,h} <dO[b][i][h], out[b][i][h]>:
 *     p_c   = exp(s_c - lse[b][i][h]) on visible keys, 0 elsewhere
 *     ds_c  = sm_scale * p_c * (<dO[b][i][h], V[c]> - <dO[b][i][h], out[b][i][h]>)
 *     dq[b][i][h]  = sum_c ds_c K[c]
 *     dk[b][kvh][c] = sum over (i, h in kvh's group) of ds_c q[b][i][h]
 *     dv[b][kvh][c] = sum over (i, h in kvh's group) of p_c dO[b][i][h]
 *
 *   q, out, d_out [B][N][Hq][D] of dtype, 16-B aligned; out and lse are the
 *                 forward pass's results for the same inputs
 *   k_cache,
 *   v_cache       [B][Hkv][S_max][D] of dtype, 16-B aligned
 *   dtype         SPEC_F32 (all fp32) or SPEC_BF16 (all bf16)
 *   lse           float[B][N][Hq], required
 *   D             64 or 128
 *   dq            out: [B][N][Hq][D] of dtype
 *   dk, dv        out: [B][Hkv][S_max][D] of dtype; rows c < P_b + N are
 *                 written, later rows are left as they are
 *   workspace     >= spec_tree_attn_backward_workspace_bytes(...) bytes,
 *                 16-B aligned, zero-filled before its first use; every call
 *                 leaves its counters at zero again (the forward pass's
 *                 rules).  With more than 128 packed rows (Hq/Hkv * N) in
 *                 bf16 it holds instead two floats per (request, node, head)
 *                 row, written by the call before they are read: no
 *                 clearing needed.
 *   err_word      nullable: SPEC_DERR_PREFIX
 * Accumulation is fp32; bf16 results are rounded to nearest even.  More
 * than 128 packed rows in bf16 run as three launches: per-row statistics,
 * a dq pass (128 rows per workgroup, over all keys) and a dK / dV pass (a
 * run of 128-key tiles per workgroup, over all rows), with no partial sums
 * in memory.  Every sum is taken in a fixed order, so results are
 * deterministic.
 */
spec_status spec_tree_attn_backward(const void* q, const void* k_cache, const void* v_cache, spec_dtype dtype,
                                    const int32_t* prefix_lens, const uint64_t* anc_mask, const void* out,
                                    const float* lse, const void* d_out, int B, int N, int Hq, int Hkv,
                                    int D, int S_max, float sm_scale, void* dq, void* dk, void* dv,
                                    void* workspace, size_t workspace_bytes, uint32_t* err_word,
                                    hipStream_t stream);

/*
 * spec_verify_step_workspace_bytes -- scratch needed by spec_verify_step for
 * these sizes: a 64-bit argmax key and a counter per node and a counter per
 * request, rounded up to 256 bytes, followed by
 * spec_tree_attn_workspace_bytes(...).  0 for sizes that spec_verify_step
 * would reject.
 */
size_t spec_verify_step_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int S_max);

/*
 * spec_verify_step -- one whole verify step: spec_tree_mask_build,
 * spec_tree_attn_verify, spec_vocab_argmax and spec_accept_walk in one launch.
 *
 * The target verifies the draft's whole tree in one parallel pass and keeps
 * the longest path it agrees with (Aurora, section 2; Runtime Draft Model
 * Training, "Overview" and "Evaluation").  The walk needs the argmax and the
 * tree but not the attention's output, so the attention's launch also holds
 * workgroups that build the masks, take the argmax (each logits row cut into
 * chunks, folded with 64-bit atomic maxima) and run each request's walk as
 * soon as its last chunk is done, while the attention builds its rows' masks
 * itself.  Every output equals that of the four separate calls on the same
 * inputs.
 *
 *   parents, draft_tokens, prefix_lens, q, q_dtype, k_cache, v_cache,
 *   kv_dtype, k_scale, v_scale, B, N, Hq, Hkv, D, S_max, sm_scale, out, lse
 *                 as in spec_tree_mask_build / spec_tree_attn_verify /
 *                 spec_accept_walk
 *   logits        float[B*N][logits_row_stride]: node (b, i)'s V logits at
 *                 row b*N + i; finite; V in 1..2^31-1, row stride >= V
 *   anc_mask      uint64[B][N] out (as spec_tree_mask_build)
 *   depth         int32[B][N] out, nullable
 *   target_argmax int32[B][N] out (as spec_vocab_argmax)
 *   accept_len, path_nodes, out_tokens  out (as spec_accept_walk)
 *   workspace     >= spec_verify_step_workspace_bytes(...) bytes, 16-B
 *                 aligned, zero-filled before its first use; every call
 *                 leaves it ready for the next one (its argmax keys and
 *                 counters back at zero, as the attention's split counters),
 *                 so it is reused without clearing.
 *                 Calls that overlap in time must not share one workspace.
 *   err_word      nullable: SPEC_DERR_ROOT / _PARENT / _TOKEN / _PREFIX
 * Every argument check of spec_tree_attn_verify is made before the first
 * launch, so a non-SPEC_OK status other than SPEC_ERR_HIP means nothing was
 * enqueued.
 */
spec_status spec_verify_step(const int32_t* parents, const int32_t* draft_tokens, const int32_t* prefix_lens,
                             const void* q, spec_dtype q_dtype, const void* k_cache, const void* v_cache,
                             spec_dtype kv_dtype, const float* k_scale, const float* v_scale,
                             const float* logits, int64_t V, int64_t logits_row_stride,
                             int B, int N, int Hq, int Hkv, int D, int S_max, float sm_scale,
                             uint64_t* anc_mask, int32_t* depth, void* out, float* lse,
                             int32_t* target_argmax, int32_t* accept_len, int32_t* path_nodes,
                             int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                             uint32_t* err_word, hipStream_t stream);

/*
 * spec_verify_step_paged -- spec_verify_step over a paged cache, in one
 * launch.
 *
 * The same step (Aurora, section 2; Runtime Draft Model Training, "Overview")
 * with the K/V caches in the page layout of spec_tree_attn_verify_paged, for
 * the serving engine that keeps its caches paged.  Every output equals that
 * of spec_tree_mask_build, spec_tree_attn_verify_paged, spec_vocab_argmax and
 * spec_accept_walk on the same inputs.
 *
 *   k_pages, v_pages, kv_dtype, block_table, max_pages, page_size, num_pages
 *                 as in spec_tree_attn_verify_paged (bf16 q; bf16 or e4m3
 *                 pages)
 *   workspace     >= spec_verify_step_workspace_bytes(B, N, Hq, Hkv, D,
 *                 max_pages * page_size) bytes; the rules of spec_verify_step
 *   err_word      nullable: as spec_verify_step, plus SPEC_DERR_PAGE
 *   everything else as in spec_verify_step.
 * Every argument check is made before the launch, so a non-SPEC_OK status
 * other than SPEC_ERR_HIP means nothing was enqueued.
 */
spec_status spec_verify_step_paged(const int32_t* parents, const int32_t* draft_tokens, const int32_t* prefix_lens,
                                   const void* q, spec_dtype q_dtype, const void* k_pages, const void* v_pages,
                                   spec_dtype kv_dtype, const float* k_scale, const float* v_scale,
                                   const int32_t* block_table, int max_pages, int page_size, int num_pages,
                                   const float* logits, int64_t V, int64_t logits_row_stride,
                                   int B, int N, int Hq, int Hkv, int D, float sm_scale,
                                   uint64_t* anc_mask, int32_t* depth, void* out, float* lse,
                                   int32_t* target_argmax, int32_t* accept_len, int32_t* path_nodes,
                                   int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                                   uint32_t* err_word, hipStream_t stream);

/*
 * spec_verify_step_static -- spec_verify_step with the library's own scratch
 * instead of a workspace argument.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * allocates nothing (no hipMalloc, no hipFree, no allocating library call):
 * the step's workspace is a file-scope device array of
 * SPEC_STATIC_SCRATCH_BYTES (72 MiB, enough for 16 requests of 60-node trees
 * over 32768-token prefixes with 64 query heads over 4 KV heads), of which
 * every GPU the library runs on holds its own copy until the process ends.
 *
 *   Arguments as spec_verify_step, without workspace / workspace_bytes.
 *   Returns SPEC_ERR_SCRATCH, before anything is enqueued, when
 *   spec_verify_step_workspace_bytes(B, N, Hq, Hkv, D, S_max) exceeds
 *   SPEC_STATIC_SCRATCH_BYTES; every other check as spec_verify_step's, also
 *   before anything is enqueued.
 * The first call on a device looks up the array's address and, unless
 * `stream` is capturing, enqueues a zero fill of it on `stream` (a first
 * call under capture relies on the array's zero initialisation at load).
 * Every step leaves the array's counters and argmax keys at zero again.
 * All calls on one GPU share that GPU's array: calls that overlap in time on
 * one GPU (other streams, other threads) race and must not be issued.
 */
#define SPEC_STATIC_SCRATCH_BYTES (72u << 20)
spec_status spec_verify_step_static(const int32_t* parents, const int32_t* draft_tokens, const int32_t* prefix_lens,
                                    const void* q, spec_dtype q_dtype, const void* k_cache, const void* v_cache,
                                    spec_dtype kv_dtype, const float* k_scale, const float* v_scale,
                                    const float* logits, int64_t V, int64_t logits_row_stride,
                                    int B, int N, int Hq, int Hkv, int D, int S_max, float sm_scale,
                                    uint64_t* anc_mask, int32_t* depth, void* out, float* lse,
                                    int32_t* target_argmax, int32_t* accept_len, int32_t* path_nodes,
                                    int32_t* out_tokens, uint32_t* err_word, hipStream_t stream);

/* Human-readable name of a status code (static storage).  Takes any int:
 * codes outside spec_status give "unknown spec_status". */
const char* spec_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPECTREE_H */
