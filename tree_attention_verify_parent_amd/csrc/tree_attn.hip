// Tree-masked split-KV attention for the verify step (gfx950).
//
// Every draft node's query attends to its request's KV-cache prefix plus its
// own ancestors and itself (the custom tree mask of Aurora, section 2, closing
// paragraph; all proposed tokens are verified in one parallel pass, Runtime
// Draft Model Training, "Overview").  The pass is bound by streaming K/V from
// HBM (the same page notes that verification is memory- rather than
// compute-bound), so each K/V byte is read once per (request, kv head): the
// g = Hq/Hkv query heads of a kv head and the N tree nodes are packed into the
// M dimension of small dense MFMA tiles (row = node * g + head).
//
// bf16 / e4m3 KV kernel:
//   workgroup = one (request b, kv head, M-tile, KV split), WM x WT waves;
//   K/V tiles of 64 tokens go HBM -> LDS by direct 16-byte DMA
//   (global_load_lds) into an NSTAGE-deep ring of row-major tiles with
//   XOR-swizzled 16-byte units -- no staging registers, no VALU work;
//   S^T = K . Q^T and O^T = V^T . P^T on v_mfma_f32_16x16x32_bf16, with V^T
//   operands produced by the LDS transpose reads; a lane holds one query row
//   of S and of O, so the online-softmax statistics of a row live in the four
//   lanes {l, l^16, l^32, l^48};
//   the 64-bit ancestor mask of each row is applied in registers, only on
//   tiles that reach the tree rows.
// A request whose tokens fit one split writes its output directly; otherwise
// each split writes (O, m, l) partials and the last split to finish combines
// them in split order (deterministic), in the same launch.
#include <cmath>
#include <type_traits>

#include "gfx950.h"
#include "host_api.h"
#include "step_ops.h"

namespace spectree {

constexpr int kTile = 64;                 // tokens per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// token held by MFMA A-row m of token group G within a 32-token chunk.  With
// this order lane group q = lane/16 ends up holding the 8 consecutive tokens
// 8q..8q+7 of the chunk in its 8 S^T accumulators (4 from each group), which
// is exactly the K-slot run its B operand needs in the PV product.
__device__ __forceinline__ int chunk_token(int G, int m) { return 8 * (m >> 2) + 4 * G + (m & 3); }

// XOR swizzle of the 16-byte units of an LDS row, by units per row (UPR).
// The K operand read of a 16-lane group touches rows {0-3, 8-11, 16-19,
// 24-27} (+4G) at one unit; the V transpose read touches the same row set at
// two adjacent units.  The swizzle gives those rows distinct bank groups, so
// each read runs at the minimum number of LDS passes.
template <int UPR>
__device__ __forceinline__ int swz(int row) {
  if constexpr (UPR >= 16) return (row & 3) | (((row >> 3) & 3) << 2);
  else if constexpr (UPR == 8) return ((row >> 1) & 1) | (((row >> 3) & 3) << 1);
  else return (row >> 1) & 3;
}

template <int I>
using Int = std::integral_constant<int, I>;

// Internal K/V format id: e4m3 caches read by fp8 arithmetic.  The codes go
// to v_mfma_f32_16x16x128_f8f6f4 as they are (no decode), and the kernel
// quantizes Q (per row) and the probabilities P to e4m3 itself.
constexpr int kKvF8Mma = 16 + SPEC_FP8_E4M3;

// LDS swizzle of that path (128-byte rows, 8 units): its K operand reads 16
// consecutive rows at one unit, and its V transpose reads rows 4g..4g+3 and
// 16+4g..19+4g (+32h) at one unit; this XOR map of row bits (found by an
// exhaustive search over linear maps) gives both distinct banks.
__device__ __forceinline__ int swz_f8(int row) { return ((row >> 1) & 3) | ((((row >> 3) ^ (row >> 4)) & 1) << 2); }

// ... and e2m1 (fp4) caches, read by the same fp8 arithmetic: the codes are
// the A operands of fp4 x fp8 MFMAs (q and p stay e4m3).
constexpr int kKvF4Mma = 16 + SPEC_FP4_E2M1;

// bf16 caches with the scores on the fp8 matrix cores: the workgroup turns
// each K tile into e4m3 codes in LDS once (K divided by a per-head power of
// two), Q is quantized per row as in the fp8 path, and S^T = K . Q^T runs on
// the 16x16x128 e4m3 MFMA; the probabilities and V stay bf16.
constexpr int kKvBf16F8S = 32 + SPEC_BF16;

// LDS swizzle of the fp4 path (64-byte rows, 4 units): its K reads take 16
// consecutive rows at one unit, its V transpose reads the 16 tokens
// {16a + 4g' + r} of one contraction run; both land on distinct banks.
__device__ __forceinline__ int swz_f4(int row) { return ((row >> 2) ^ (row >> 4)) & 3; }

// Contraction slot k of an e2m1 A operand, for lane group g and nibble n (of
// the low four dwords, element 2j in the low nibble of byte j): the hardware
// order, measured.  (An e4m3 operand has k = 32g + byte.)
__device__ __forceinline__ int f4_slot(int g, int n) {
  return 64 * (g & 1) + 16 * (g >> 1) + (n & 15) + 32 * (n >> 4);
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// 16x16x128 e4m3 x e4m3 MFMA, fp32 accumulate (the zero scale operands select
// the unscaled instruction)
__device__ __forceinline__ f32x4_t mfma_f8(i32x8_t a, i32x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 16x16x128 e2m1 (A) x e4m3 (B) MFMA, fp32 accumulate
__device__ __forceinline__ f32x4_t mfma_f4f8(i32x8_t a, i32x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, 0, 0, 0);
}

// four floats -> four e4m3 codes (round to nearest even) in one dword, first in the low byte
__device__ __forceinline__ int pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// Visibility of the 64 tokens t0 .. t0+63 of a tile to one query row: bit k
// is set iff token t0+k is in the row's prefix, or is a tree node on the
// row's ancestor-or-self path, and lies before the split end t_end.
__device__ __forceinline__ uint64_t tile_visibility(uint64_t anc, int t0, int P, int t_end) {
  const int pre = P - t0;                         // prefix tokens in the tile (may be <= 0)
  const uint64_t prefix = pre <= 0 ? 0ull : ((1ull << pre) - 1ull);   // pre < 64 here
  const uint64_t tree = pre >= 0 ? (anc << pre) : (anc >> (-pre));    // -pre < N <= 64
  const int lim = t_end - t0;                     // 1 .. 64
  const uint64_t inside = lim >= 64 ? ~0ull : ((1ull << lim) - 1ull);
  return (prefix | tree) & inside;
}

// One workgroup = one (request b, kv head, M-tile, KV split).
//   Wave (wm, wt) owns RB 16-row blocks of the M-tile and the 32-token chunks
//   wt*CPT .. wt*CPT+CPT-1 of every 64-token tile (CPT = 2/WT).
// Waves per SIMD the kernel is built for: the planner puts as many
// workgroups on a CU as a bf16 ring leaves room for in the 160 KB LDS (at
// most 2; the same count for every cache format, so one workspace size serves
// all), and the compiler may spend 512 / that many waves registers per wave.
// Two row blocks per wave need about 200+ registers, so at most 2 waves per
// SIMD there.
template <int D, int RB, int WM, int WT, int NSTAGE>
struct SplitOccupancy {
  static constexpr int ring_bf16 = NSTAGE * 2 * kTile * D * 2 + 4 * 1024 + 16;
  static constexpr int fit = (160 * 1024) / ring_bf16;
  static constexpr int wg_per_cu = fit < 1 ? 1 : (fit > 2 ? 2 : fit);
  static constexpr int w = (wg_per_cu * WM * WT + 3) / 4;
  static constexpr int cap = (RB >= 2) ? 2 : 4;
  static constexpr int value = w < 1 ? 1 : (w > cap ? cap : w);
};

// A piece of work never starts or ends closer than this many tokens to either
// end of its (request, kv head) sequence: a unit boundary that would leave a
// shorter remainder moves to that end.
constexpr int kMinPiece = 128;
// K and V operand fragments a wave keeps in flight: the tile loop reads them
// in batches, the next batch's reads issued before the current batch's
// products (ds_read latency is otherwise exposed on every fragment).
constexpr int kFragBatch = 4;
// How far (base 2) a row's running max may rise above the reference max the
// row's p = 2^(s - m) are taken against before the reference moves.
constexpr float kMaxLag = 8.0f;
// Requests per launch: every workgroup keeps a table of their lengths in LDS.
constexpr int kMaxBatch = 1024;
// Paged caches: a workgroup stages the page ids of its current piece in LDS.
constexpr int kMaxPages = 2048;

// One (request, kv head) token sequence of the concatenated work stream:
// request b, kv head kvh, L = P_b + N tokens, starting at stream offset start.
struct Seg {
  int b, kvh, L;
  long long start;
};

template <int D, int KVF, int RB, int WM, int WT, int NSTAGE, bool PAGED, bool STEP>
__global__ __launch_bounds__(WM * WT * kWave)
__attribute__((amdgpu_waves_per_eu(SplitOccupancy<D, RB, WM, WT, NSTAGE>::value)))
void tree_attn_split_kernel(
    const __bf16* __restrict__ q, const unsigned char* __restrict__ kc,
    const unsigned char* __restrict__ vc, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ prefix_lens,
    const uint64_t* __restrict__ anc_mask, int B, int N, int Hq, int Hkv, int S_max,
    float sm_scale, int split_len, int n_splits, int n_units, int n_mt, __bf16* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_o, float2* __restrict__ part_ml,
    uint32_t* __restrict__ counters, uint32_t* __restrict__ err_word,
    const int32_t* __restrict__ block_table, int max_pages, int ps_log2, int num_pages, int attn_grid,
    const PrepArgs pa) {
  static_assert(WT == 1 || WT == 2, "waves split a 64-token tile in one or two 32-token halves");
  static_assert(NSTAGE >= 2 && NSTAGE <= 8, "ring depth");
  constexpr int NW = WM * WT;
  constexpr bool F4 = (KVF == kKvF4Mma);             // fp8 arithmetic on an e2m1 cache
  constexpr bool F8 = (KVF == kKvF8Mma) || F4;       // fp8 arithmetic (e4m3 or e2m1 cache)
  constexpr bool S8 = (KVF == kKvBf16F8S);          // bf16 cache, scores on the fp8 matrix cores
  constexpr bool BF = (KVF == SPEC_BF16) || S8;      // bf16 rows in the ring
  constexpr bool QF8 = F8 || S8;                     // Q quantized per row to e4m3
  constexpr int EB = BF ? 2 : 1;                     // bytes per cached element (fp4: half)
  static_assert(!S8 || D == 128, "fp8 scores over a bf16 cache: D = 128");
  static_assert(!F8 || (WT == 1 && D == 128), "the fp8 path covers whole tiles per wave, D = 128");
  constexpr int CPT = 2 / WT;                        // 32-token chunks per wave per tile
  constexpr int RBYTES = F4 ? D / 2 : D * EB;        // bytes per K/V row
  constexpr int UPR = RBYTES / 16;                   // 16-byte units per row
  // tokens per ring tile: 64, or 128 for fp8 arithmetic (its PV product
  // contracts 128 tokens per MFMA); pieces still start on 64-token bounds
  constexpr int TILE = F8 ? 2 * kTile : kTile;
  constexpr int TB = TILE * RBYTES;                  // bytes per tensor per stage
  constexpr int NLOAD = TB / 1024;                   // 1-KB wave DMA instructions per tensor
  constexpr int KPW = NLOAD / NW;                    // per wave per tensor per stage
  constexpr int PT = 2 * KPW;                        // DMA instructions per wave per tile
  constexpr int RPI = 1024 / RBYTES;                 // rows per DMA instruction
  constexpr int MT = WM * RB * 16;                   // packed rows per workgroup
  constexpr int KC = D / 32;
  constexpr int DB = D / 16;
  static_assert(NLOAD % NW == 0, "DMA instructions must split evenly over the waves");
  static_assert((NSTAGE - 1) * PT < 64, "tiles in flight must fit the vmcnt counter");
  // The whole verify step in one launch (STEP; bf16 / decoded-fp8 caches,
  // contiguous or paged): workgroups past the attention's grid take the prep
  // role (masks, argmax, accept walk), and the attention builds its rows'
  // ancestor masks from pa.parents itself.  They come last, so they fill the
  // CUs that the attention's workgroups leave as they finish.
  constexpr bool FUSABLE = STEP;
  static_assert(!STEP || (!F8 && !S8), "the one-launch step covers bf16 / decoded-fp8 caches");
  if constexpr (FUSABLE) {
    if ((int)blockIdx.x >= attn_grid) {
      prep_block<NW * kWave, kPrepUnroll>(pa, (int)blockIdx.x - attn_grid, B, N, err_word);
      return;
    }
  }


  // the ring: stage s holds K at smem + 2s*TB and V at smem + (2s+1)*TB
  __shared__ __align__(1024) unsigned char smem[NSTAGE * 2 * TB];
  __shared__ int s_cum[kMaxBatch + 1];
  __shared__ uint32_t s_last;
  __shared__ int s_pages[PAGED ? kMaxPages : 1];
  __shared__ __align__(16) unsigned char s_k8[S8 ? kTile * 128 : 16];   // e4m3 codes of the K tile
  auto kst = [&](int st) -> unsigned char* { return smem + (2 * st) * TB; };
  auto vst = [&](int st) -> unsigned char* { return smem + (2 * st + 1) * TB; };

  // Every kernel argument at once: left to first use, each would be a scalar
  // load with its own wait, and several of them stand before the first DMA.
  asm volatile("" ::"s"(q), "s"(kc), "s"(vc), "s"(prefix_lens), "s"(anc_mask), "s"(B), "s"(N), "s"(Hq),
               "s"(Hkv), "s"(S_max), "s"(split_len), "s"(n_splits), "s"(n_units), "s"(n_mt));

  // ---- work unit, XCD-aware: workgroups are dispatched round-robin over the
  // 8 XCDs, so the M-tiles of one unit get ids congruent mod 8 and share that
  // XCD's L2.
  const int id = blockIdx.x;
  const int per = 8 * n_mt;
  const int mt = (id % per) / 8;
  const int u = (id / per) * 8 + (id % 8);
  const int n_fixed = B * Hkv * n_splits;
  const int lane0 = threadIdx.x & 63;
  const int wave0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // One-launch verify step with the argmax in the prologue (when pa.held >
  // 0): workgroup id scans logits chunk id.  The chunk goes out first, as
  // LDS DMA into the ring's last stage (empty until the loop refills it), and
  // is reduced while the first tiles are still in flight; its max is folded
  // into the row's key, and counted in once the workgroup's first loads have
  // drained.  The count's result is read only when the workgroup leaves:
  // usually the request's mask wave, in the tail, arrives after every chunk
  // and runs the walk; if a chunk's count came last, its workgroup runs it on
  // the way out.
  constexpr int PU = (2 * TB) / (NW * kWave * 16) < kPrepUnroll ? (2 * TB) / (NW * kWave * 16) : kPrepUnroll;
  static_assert(!FUSABLE || PU >= 1, "a logits chunk fits the ring's last stage");
  const int held_g = (FUSABLE && pa.parents != nullptr && id < pa.held) ? id : -1;
  uint32_t prep_seen = 0;                            // thread 0: the count's result
  bool prep_counted = false;
  __shared__ float s_pv[NW];
  __shared__ int s_pi[NW];
  __shared__ uint32_t s_walk;                        // prep_leave's own flag (s_last may still be being read)
  // the chunk's PU 1-KB DMA instructions per wave (addresses past the row's
  // end read its last float4, which the reduction ignores)
  auto prep_issue = [&]() {
    if constexpr (FUSABLE) {
      const int r = held_g / pa.chunks, c = held_g - r * pa.chunks;
      const float* row = pa.logits + (int64_t)r * pa.row_stride;
      const int64_t V4 = pa.V >> 2;
#pragma unroll
      for (int j = 0; j < PU; ++j) {
        const int64_t e4 = (int64_t)c * (NW * kWave * PU) + (int64_t)(wave0 * PU + j) * kWave + lane0;
        dma16(row + 4 * (e4 < V4 ? e4 : V4 - 1), LDS_ADDR(smem) + (2 * (NSTAGE - 1)) * TB + (wave0 * PU + j) * 1024);
      }
    }
  };
  // after the wave issued n_tiles more tiles: wait for the chunk, reduce it,
  // fold (thread 0); every wave calls it
  auto prep_reduce = [&](int n_tiles) {
    if constexpr (FUSABLE) {
      switch (n_tiles) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<PT>(); break;
        case 2: if constexpr (NSTAGE > 2) wait_vmcnt<2 * PT>(); break;
        case 3: if constexpr (NSTAGE > 3) wait_vmcnt<3 * PT>(); break;
        case 4: if constexpr (NSTAGE > 4) wait_vmcnt<4 * PT>(); break;
        case 5: if constexpr (NSTAGE > 5) wait_vmcnt<5 * PT>(); break;
        default: if constexpr (NSTAGE > 6) wait_vmcnt<6 * PT>(); break;
      }
      const int r = held_g / pa.chunks, c = held_g - r * pa.chunks;
      const int64_t V4 = pa.V >> 2;
      ArgBest best{-INFINITY, 0x7fffffff};
#pragma unroll
      for (int j = 0; j < PU; ++j) {
        const int64_t e4 = (int64_t)c * (NW * kWave * PU) + (int64_t)(wave0 * PU + j) * kWave + lane0;
        const f32x4_t x = *reinterpret_cast<const f32x4_t*>(smem + (2 * (NSTAGE - 1)) * TB +
                                                           (wave0 * PU + j) * 1024 + 16 * lane0);
        if (e4 < V4) {
          const int i0 = (int)(e4 << 2);
          if (x.x > best.v) { best.v = x.x; best.i = i0; }
          if (x.y > best.v) { best.v = x.y; best.i = i0 + 1; }
          if (x.z > best.v) { best.v = x.z; best.i = i0 + 2; }
          if (x.w > best.v) { best.v = x.w; best.i = i0 + 3; }
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) best = arg_better(best, ArgBest{__shfl_xor(best.v, o, kWave), __shfl_xor(best.i, o, kWave)});
      if (lane0 == 0) {
        s_pv[wave0] = best.v;
        s_pi[wave0] = best.i;
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0): the wave's best is in LDS
      wg_barrier();
      if (threadIdx.x == 0) {
        ArgBest b{s_pv[0], s_pi[0]};
#pragma unroll
        for (int w = 1; w < NW; ++w) b = arg_better(b, ArgBest{s_pv[w], s_pi[w]});
        prep_fold(pa, held_g, b);
      }
    }
  };
  // count the chunk in (thread 0) once the fold has been performed (the wait
  // costs nothing where the caller's loads have just drained)
  auto prep_count_in = [&]() {
    if constexpr (FUSABLE) {
      if (threadIdx.x == 0) {
        wait_vmcnt<0>();
        prep_seen = __hip_atomic_fetch_add(pa.req_cnt + held_g / pa.chunks / N, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_SYSTEM);
      }
      prep_counted = true;
    }
  };
  auto prep_leave = [&]() {
    if constexpr (FUSABLE) {
      if (!prep_counted) prep_count_in();
      if (threadIdx.x == 0) s_walk = (prep_seen == prep_arrivals(pa, N) - 1) ? 1u : 0u;
      __syncthreads();
      if (s_walk && threadIdx.x < kWave) {
        const int b = held_g / pa.chunks / N, ln = (int)threadIdx.x;
        const bool live = ln < N;
        const int p = live ? pa.parents[(size_t)b * N + ln] : 0;
        const int d = live ? pa.draft_tokens[(size_t)b * N + ln] : 0;
        prep_walk(pa, b, N, ln, p, d, err_word);
      }
    }
  };
  // (a paged fixed unit issues it after its page ids, whose loads would
  // otherwise wait for the chunk as well)
  if (held_g >= 0 && (!PAGED || u >= n_fixed)) prep_issue();
  if (u >= max(n_fixed, n_units)) {
    if (held_g >= 0) {
      prep_reduce(0);
      prep_leave();
    }
    return;
  }
  const int g = Hq / Hkv;
  const int M = g * N;

  // ---- DMA of one tile (tokens t0 .. t0+TILE-1 of the sequence at
  // kbase / vbase; rows at or past t_end repeat row t_end - 1) into stage st:
  // wave w issues instructions w, w+NW, ...; lane l of instruction j fills LDS
  // bytes j*1024 + 16l, i.e. row j*RPI + l/UPR at swizzled unit l%UPR.
  // Paged caches: kbase / vbase point at the kv head's row in the pool's first
  // token, and token c of the sequence sits in page s_pages[c/page - pg0]
  // (the page ids of the current piece, staged by stage_pages), with rows of
  // Hkv * RBYTES bytes per token.
  auto dma_tile = [&](const unsigned char* kbase, const unsigned char* vbase, int t0, int t_end, int st,
                      int wave, int lane, int pg0) {
    if constexpr (!PAGED) {
      if (t0 + TILE <= t_end) {
        // a whole tile: the wave-uniform tile base in SGPRs, the lane's 32-bit
        // offset in a VGPR (no per-lane 64-bit address arithmetic)
        const unsigned char* kt = kbase + (size_t)t0 * RBYTES;
        const unsigned char* vt = vbase + (size_t)t0 * RBYTES;
#pragma unroll
        for (int qd = 0; qd < KPW; ++qd) {
          const int j = wave + qd * NW;
          const int row = j * RPI + lane / UPR;
          int sw;
          if constexpr (F4) sw = swz_f4(row);
          else if constexpr (F8) sw = swz_f8(row);
          else sw = swz<UPR>(row);
          const uint32_t lo = (uint32_t)(row * RBYTES + ((lane % UPR) ^ sw) * 16);
          dma16s(kt, lo, LDS_ADDR(smem) + (2 * st) * TB + j * 1024);
          dma16s(vt, lo, LDS_ADDR(smem) + (2 * st + 1) * TB + j * 1024);
        }
        return;
      }
    }
#pragma unroll
    for (int qd = 0; qd < KPW; ++qd) {
      const int j = wave + qd * NW;
      const int row = j * RPI + lane / UPR;
      int sw;
      if constexpr (F4) sw = swz_f4(row);
      else if constexpr (F8) sw = swz_f8(row);
      else sw = swz<UPR>(row);
      const int unit16 = (lane % UPR) ^ sw;
      const int c = min(t0 + row, t_end - 1);
      size_t goff;
      if constexpr (PAGED) {
        const size_t page = (size_t)s_pages[(c >> ps_log2) - pg0];
        goff = ((page << ps_log2) | (size_t)(c & ((1 << ps_log2) - 1))) * ((size_t)Hkv * RBYTES) + unit16 * 16;
      } else {
        goff = (size_t)c * RBYTES + unit16 * 16;
      }
      dma16(kbase + goff, LDS_ADDR(smem) + (2 * st) * TB + j * 1024);
      dma16(vbase + goff, LDS_ADDR(smem) + (2 * st + 1) * TB + j * 1024);
    }
  };

  // Paged caches: the page ids of tokens [t0, t1) of request b into s_pages
  // (an id outside the pool is flagged and replaced by page 0, so no access
  // leaves the pool), then a barrier.  Every wave of the workgroup calls it.
  auto stage_pages = [&](int b, int t0, int t1) {
    if constexpr (PAGED) {
      const int pg0 = t0 >> ps_log2;
      const int np = ((t1 - 1) >> ps_log2) - pg0 + 1;
      for (int i = threadIdx.x; i < np; i += NW * kWave) {
        int id = block_table[(size_t)b * max_pages + pg0 + i];
        if (id < 0 || id >= num_pages) {
          flag_error(err_word, SPEC_DERR_PAGE);
          id = 0;
        }
        s_pages[i] = id;
      }
      __syncthreads();
    }
  };
  // the kv head's K / V row base of sequence (b, kvh)
  auto seq_base = [&](const unsigned char* pool, int b, int kvh) -> const unsigned char* {
    if constexpr (PAGED) return pool + (size_t)kvh * RBYTES;
    else return pool + ((size_t)(b * Hkv + kvh) * S_max) * RBYTES;
  };

  // ---- Q rows of a wave as MFMA B operands (K-slots 32c + 8lg .. +7) and
  // the rows' ancestor masks, for sequence (b, kvh)
  bf16x8_t qreg[RB][KC];
  uint64_t anc[RB];
  // in one-launch mode: the lane's node's parent (lane = node), for the
  // ancestor masks built after the loads complete
  const bool own_masks = FUSABLE && pa.parents != nullptr;
  int par_lane = 0;
  auto load_q = [&](int b, int kvh, int row0, int l16, int lg) {
    if (own_masks) {
      const int nd = l16 + 16 * lg;
      par_lane = nd < N ? pa.parents[(size_t)b * N + nd] : 0;
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = row0 + rb * 16 + l16;
      if (row < M) {
        const int i = row / g, hl = row % g;
        const __bf16* qp = q + ((size_t)(b * N + i) * Hq + kvh * g + hl) * D;
        // bf16: the B operand's K-slots 32c + 8lg .. +7; fp8: the 32 columns
        // 32lg .. 32lg+31 the lane quantizes for its 16x16x128 B operand
#pragma unroll
        for (int c = 0; c < KC; ++c)
          qreg[rb][c] = *reinterpret_cast<const bf16x8_t*>(qp + (QF8 ? 32 * lg + 8 * c : 32 * c + 8 * lg));
        anc[rb] = own_masks ? 0ull : anc_mask[(size_t)b * N + i];
      } else {
#pragma unroll
        for (int c = 0; c < KC; ++c) qreg[rb][c] = bf16x8_t{};
        anc[rb] = 0ull;
      }
    }
  };

  // ---- Two schedules.  Fixed: unit u < n_fixed is split u % n_splits of
  // sequence u / n_splits: its ceil(S_max / 64) tiles dealt out in order,
  // split_len / 64 to a split and one more to each of the last splits that
  // the remainder needs (so the sequence's final, partial tile goes with a
  // longer split and no split holds two tiles more than another).  When
  // every request fills its
  // cache (P_b = S_max - N) that divides the work evenly and needs nothing but
  // the sizes, so the unit's first tiles and Q rows are fetched at once, before
  // the prefix lengths are known.  Balanced (below): for ragged lengths the
  // units instead take equal shares of the actual tokens.  Every workgroup
  // reads all prefix lengths and so makes the same choice.
  //
  // Wave 0 fetches the prefix lengths into LDS (raw, in s_cum) with dword
  // DMAs before anything else, so they land ahead of the tiles.
  if (wave0 == 0)
    for (int c0 = 0; c0 < B; c0 += kWave) dma4(prefix_lens + min(c0 + lane0, B - 1), LDS_ADDR(s_cum) + 4 * c0);
  int f_seg = -1, f_begin = 0, f_end = 0;
  int pro_tiles = 0;                                 // tiles issued below
  if (u < n_fixed) {
    f_seg = u / n_splits;
    const int sp = u % n_splits, q_t = split_len / kTile;
    const int long0 = n_splits - ((S_max + kTile - 1) / kTile - n_splits * q_t);   // first longer split
    f_begin = (sp * q_t + max(0, sp - long0)) * kTile;
    f_end = min(S_max, f_begin + (q_t + (sp >= long0 ? 1 : 0)) * kTile);
    stage_pages(f_seg / Hkv, f_begin, f_end);
    if constexpr (PAGED)
      if (held_g >= 0) prep_issue();
    const unsigned char* kb = seq_base(kc, f_seg / Hkv, f_seg % Hkv);
    const unsigned char* vb = seq_base(vc, f_seg / Hkv, f_seg % Hkv);
    const int nt = (f_end - f_begin + TILE - 1) / TILE;
#pragma unroll
    for (int i = 0; i < NSTAGE - 1; ++i)
      if (i < nt) dma_tile(kb, vb, f_begin + i * TILE, f_end, i, wave0, lane0, f_begin >> ps_log2);
    pro_tiles = min(nt, NSTAGE - 1);
  }
  if (held_g >= 0) prep_reduce(pro_tiles);
  if (u < n_fixed) load_q(f_seg / Hkv, f_seg % Hkv, mt * MT + (wave0 % WM) * RB * 16, lane0 & 15, lane0 >> 4);
  // whether every raw prefix length in s_cum is S_max - N (after a barrier
  // that follows wave 0's wait for its DMAs)
  auto uniform = [&]() -> bool {
    bool bad = false;
    for (int c0 = 0; c0 < B; c0 += kWave) {
      const int bb = c0 + lane0;
      bad = bad || (bb < B && s_cum[bb] != S_max - N);
    }
    return __ballot(bad) == 0;
  };

  // ---- The work stream: the (request, kv head) sequences back to back, in
  // request-major order; unit v of n_act owns stream tokens [bnd(v),
  // bnd(v+1)), about an equal share, so ragged prefix lengths do not leave
  // some workgroups with twice the work of others.  Every workgroup derives
  // the same boundaries from a table of exclusive prefix sums of the
  // per-request token counts (0 for a request whose prefix length is
  // invalid: it is flagged once and skipped).  Wave 0 builds the table in
  // place from the raw prefix lengths in s_cum.
  auto build_table = [&]() {
    int carry = 0;
    for (int c0 = 0; c0 < B; c0 += kWave) {
      const int bb = c0 + lane0;
      int lb = 0;
      if (bb < B) {
        const int pb = s_cum[bb];
        if (pb >= 0 && pb <= S_max - N) lb = pb + N;
        else if (u == 0 && mt == 0) flag_error(err_word, SPEC_DERR_PREFIX);
      }
      int incl = lb;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const int t = __shfl_up(incl, d);
        if (lane0 >= d) incl += t;
      }
      if (bb < B) s_cum[bb] = carry + incl - lb;
      carry += __shfl(incl, kWave - 1);
    }
    if (lane0 == 0) s_cum[B] = carry;
    __builtin_amdgcn_s_waitcnt(0xC07F);              // lgkmcnt(0): the table is in LDS before the next barrier
  };
  // Unit v's nominal start, about v*T/n: any deterministic rule that is
  // monotone in v serves (every workgroup evaluates the same one, and the
  // result is snapped to a tile anyway), so it is computed in fp32, not with
  // slow 64-bit integer or fp64 division.
  auto share = [](int v, long long T, int n) -> long long {
    return (long long)((float)v * ((float)T * __builtin_amdgcn_rcpf((float)n)));
  };
  long long T = 0;
  int n_act = 1;
  auto set_schedule = [&]() {
    T = (long long)Hkv * __builtin_amdgcn_readfirstlane(s_cum[B]);
    n_act = (int)max(1ll, min((long long)n_units, T / kMinPiece));   // units of >= kMinPiece tokens
  };

  // The sequence holding stream offset x (0 <= x < T): the last request b with
  // Hkv * s_cum[b] <= x (searched 64 table entries at a time, first over
  // every 64th entry), then the kv head within it.
  auto find = [&](long long x) -> Seg {
    int blk = 0;
    const int nblk = B / kWave + 1;                  // blocks of the B + 1 entries
    if (nblk > 1) {
      const bool le = lane0 < nblk && (long long)Hkv * s_cum[min(lane0 * kWave, B)] <= x;
      blk = __popcll(__ballot(le)) - 1;
    }
    const int e = min(blk * kWave + lane0, B);
    const bool le2 = blk * kWave + lane0 <= B && (long long)Hkv * s_cum[e] <= x;
    const int bsel = blk * kWave + __popcll(__ballot(le2)) - 1;
    const int cb = __builtin_amdgcn_readfirstlane(s_cum[bsel]);
    const int lb = __builtin_amdgcn_readfirstlane(s_cum[bsel + 1]) - cb;
    const long long base = (long long)Hkv * cb;
    const int kvh = (int)(x - base) / lb;             // x - base < Hkv * S_max < 2^31
    return Seg{bsel, kvh, lb, base + (long long)kvh * lb};
  };
  // Unit v starts at stream offset v*T/n_act, moved to the nearest whole
  // tile of its sequence, or to the sequence's start or end if that leaves
  // less than kMinPiece tokens on one side.
  auto snap = [&](long long x) -> long long {
    if (x <= 0) return 0;
    if (x >= T) return T;
    const Seg sg = find(x);
    const int lx = (((int)(x - sg.start) + kTile / 2) / kTile) * kTile;
    if (lx < kMinPiece) return sg.start;
    if (sg.L - lx < kMinPiece) return sg.start + sg.L;
    return sg.start + lx;
  };
  auto bnd = [&](int v) -> long long { return v <= 0 ? 0 : (v >= n_act ? T : snap(share(v, T, n_act))); };
  // the unit whose range holds stream offset y (0 <= y < T)
  auto unit_of = [&](long long y) -> int {
    int v = (int)min((long long)n_act - 1, (long long)((float)y * ((float)n_act * __builtin_amdgcn_rcpf((float)T))));
    while (v > 0 && bnd(v) > y) --v;
    while (v + 1 < n_act && bnd(v + 1) <= y) ++v;
    return v;
  };
  // partial-result row r of slot sl: every unit has two slots, for its first
  // and its last piece (the only ones that can cover part of a sequence)
  auto part_row = [&](int sl, int r) -> size_t { return ((size_t)sl * n_mt + mt) * MT + r; };

  long long u_start = 0, u_end = 0;
  // leave the fixed schedule: the table, then this unit's balanced range
  auto to_balanced = [&]() -> bool {
    if (wave0 == 0) build_table();
    __syncthreads();
    set_schedule();
    if (u >= n_act) return false;
    u_start = bnd(u);
    u_end = bnd(u + 1);
    return true;
  };

  bool fixed = f_seg >= 0;                           // running a fixed split, not yet checked
  if (!fixed) {
    // no fixed split for this unit: it only has work under the balanced schedule
    wait_vmcnt<0>();
    __syncthreads();
    if (uniform() || !to_balanced()) {
      if (held_g >= 0) prep_leave();
      return;
    }
  }
  for (long long x = fixed ? 0 : u_start; x < (fixed ? 1 : u_end);) {
    int b, kvh, L, t_begin, t_end;
    long long seg_start;
    if (fixed) {
      b = f_seg / Hkv;
      kvh = f_seg % Hkv;
      L = S_max;
      seg_start = 0;
      t_begin = f_begin;
      t_end = f_end;
      x = 1;
    } else {
      const Seg sg = find(x);
      b = sg.b;
      kvh = sg.kvh;
      L = sg.L;
      seg_start = sg.start;
      t_begin = (int)(x - seg_start);
      t_end = (int)min((long long)L, u_end - seg_start);
      x = seg_start + L;
    }
    const int P = L - N;
    const int ntiles = (t_end - t_begin + TILE - 1) / TILE;
    const bool direct = (t_begin == 0 && t_end == L);   // the whole sequence is in this piece

    __syncthreads();                                 // the previous piece is done with the LDS

    // Thread indices from an opaque copy of threadIdx.x: without it the
    // compiler hoists every per-lane LDS and global address of the tile loop
    // out of the piece loop and keeps them live across it.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM;
    const int wt = wave / WM;
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    const int row0 = mt * MT + wm * RB * 16;

    float scale_log2 = sm_scale * kLog2e;
    float out_scale = 1.0f;
    if constexpr (S8) {
      // K's codes are K / 2^e, e the exponent of k_scale[kvh] (1 without scales)
      if (k_scale) scale_log2 *= __uint_as_float(__float_as_uint(k_scale[kvh]) & 0x7F800000u);
    } else if constexpr (KVF != SPEC_BF16) {
      scale_log2 *= k_scale[kvh];
      out_scale = v_scale[kvh];
    }
    // fp8 arithmetic: P goes to the MFMA as e4m3(p * 2^8), which keeps weights
    // down to 2^-17 of the row maximum representable (p * 2^8 <= 256 < 448).
    // The 2^8 rides in the running max (kept 8 below the true one), so the
    // row sums, the partials' merge and the log-sum-exp stay consistent.

    const unsigned char* kbase = seq_base(kc, b, kvh);
    const unsigned char* vbase = seq_base(vc, b, kvh);
    const int pg0 = t_begin >> ps_log2;

    auto issue = [&](int st, int i) { dma_tile(kbase, vbase, t_begin + i * TILE, t_end, st, wave, lane, pg0); };

    // tiles 0 .. NSTAGE-2 go in flight first; everything up to the wait below
    // runs in their shadow
    if (!fixed) {                                    // a fixed split's first tiles are in flight already
      stage_pages(b, t_begin, t_end);
#pragma unroll
      for (int i = 0; i < NSTAGE - 1; ++i)
        if (i < ntiles) issue(i, i);
      load_q(b, kvh, row0, l16, lg);
    }

    // merge bookkeeping for a piece that covers only part of its sequence:
    // this piece's partial-result slot, and the slots of all its sequence's
    // pieces.  Fixed: piece sp of sequence f_seg has slot f_seg*n_splits + sp.
    // Balanced: the units u_first .. u_first+npieces-1 hold the pieces, each
    // unit has two slots (for its first and its last piece, the only ones that
    // can cover part of a sequence), and the first unit's piece is its last
    // one if it started in an earlier sequence.
    int u_first = u, npieces = n_splits, my_slot = u;
    bool first_odd = false;
    if (fixed) {
      u_first = f_seg * n_splits;
    } else if (!direct) {
      u_first = (u_start <= seg_start) ? u : unit_of(seg_start);
      const int u_last = (u_end >= seg_start + L) ? u : unit_of(seg_start + L - 1);
      npieces = u_last - u_first + 1;
      first_odd = bnd(u_first) < seg_start;
      my_slot = (u_start >= seg_start) ? 2 * u : 2 * u + 1;
    }
    // Complete the Q / mask loads here, once: the compiler cannot count the
    // DMA instructions, so any wait it places for these loads drains the ring;
    // inside the tile loop that would happen on every tile.  Here it only waits
    // for the tiles issued above, which the loop needs first anyway.
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      asm volatile("" ::"v"(anc[rb]));
#pragma unroll
      for (int c = 0; c < KC; ++c) asm volatile("" ::"v"(qreg[rb][c]));
    }
    if (own_masks) {
      // the request's ancestor-or-self sets by pointer doubling across the
      // wave (lane = node), then each row takes its node's set; a request
      // with a bad parent gets self-only sets, as the mask build writes them
      asm volatile("" ::"v"(par_lane));
      bool req_bad;
      const uint64_t set = ancestor_set(par_lane, lane, lane < N, nullptr, &req_bad);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int row = row0 + rb * 16 + l16;
        const uint64_t a = shfl_u64(set, row < M ? row / g : 0);
        anc[rb] = row < M ? a : 0ull;
      }
    }
    // fp8 arithmetic: each (node, head) row of Q as e4m3 codes with its own
    // scale amax / 448 (rows of zeros get scale 1); the four lanes of a row
    // hold a quarter each.  srow is the row's score scale in base 2.
    i32x8_t qf8[QF8 ? RB : 1];
    float srow[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      srow[rb] = scale_log2;
      if constexpr (QF8) {
        float amax = 0.0f;
#pragma unroll
        for (int c = 0; c < KC; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)qreg[rb][c][e]));
        amax = row4_max(amax);
        const float inv = amax > 0.0f ? 448.0f / amax : 1.0f;
        srow[rb] = scale_log2 * (amax > 0.0f ? amax * (1.0f / 448.0f) : 1.0f);
#pragma unroll
        for (int c = 0; c < KC; ++c)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            // q * (448 / amax) can exceed 448 by an ulp in fp32: clamp (the
            // value it rounds to anyway)
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = fminf(fmaxf((float)qreg[rb][c][4 * h + e] * inv, -448.0f), 448.0f);
            qf8[rb][2 * c + h] = pack_e4m3x4(v[0], v[1], v[2], v[3]);
          }
      }
    }

    wait_vmcnt<0>();   // usually already met by the wait above; a wave with no Q rows has none
    if (fixed) {
      // wave 0's prefix lengths have landed (the wait above); once they are
      // visible, check that the fixed schedule is the balanced one
      __syncthreads();
      if (!uniform()) {
        fixed = false;
        if (!to_balanced()) break;
        x = u_start;
        continue;
      }
    }
    // A prologue chunk counts in now: its fold has been performed (the wait
    // above), and the count's round trip is not waited for before the loop
    // (its first counted wait comes after NSTAGE - 1 tiles of compute).
    if (held_g >= 0 && !prep_counted) prep_count_in();

    f32x4_t oacc[RB][DB];
    float m_run[RB], l_run[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      m_run[rb] = -INFINITY;
      l_run[rb] = 0.0f;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[rb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }


    // A operand of S^T = K . Q^T: lane (m = l16, lg) holds K[row][32c + 8lg .. +7]
    auto read_k = [&](const unsigned char* st, int row, int c) -> bf16x8_t {
      if constexpr (BF) {
        return *reinterpret_cast<const bf16x8_t*>(st + row * RBYTES + (((4 * c + lg) ^ swz<UPR>(row)) << 4));
      } else {
        const uint2 w = *reinterpret_cast<const uint2*>(
            st + row * RBYTES + (((2 * c + (lg >> 1)) ^ swz<UPR>(row)) << 4) + ((lg & 1) << 3));
        return fp8x8_to_bf16(w.x, w.y);
      }
    };
    // A operand of O^T = V^T . P^T: lane (l16, lg) holds V[32ch + 8lg + k][16db + l16],
    // k = 0..7.  Transpose reads: a 16-lane group's 8-byte chunks form a vector
    // E and lane j receives E[j + 16k]; so lanes 4k'..4k'+3 (bf16) or 2k, 2k+1
    // (fp8) point at the 16 columns of token k.
    auto read_v = [&](const unsigned char* st, int ch, int db) -> bf16x8_t {
      if constexpr (BF) {
        i16x4_t t[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int row = 32 * ch + 8 * lg + 4 * r + (l16 >> 2);
          const int u = 2 * db + ((l16 >> 1) & 1);
          const int off = row * RBYTES + ((u ^ swz<UPR>(row)) << 4) + ((l16 & 1) << 3);
          t[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(st + off));
        }
        // whole-vector bit casts: assembling the operand element by element
        // from bit-cast shorts is lowered wrongly (half-words get duplicated)
        const i16x8_t both = __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8_t, both);
      } else {
        const int row = 32 * ch + 8 * lg + (l16 >> 1);
        const int off = row * RBYTES + ((db ^ swz<UPR>(row)) << 4) + ((l16 & 1) << 3);
        const i32x2_t t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(st + off));
        return fp8x8_to_bf16((uint32_t)t[0], (uint32_t)t[1]);
      }
    };

    // fp8 arithmetic operands (128-token tiles).  K: lane (m = l16, lg)
    // holds K[row][32lg .. 32lg+31], the A operand of S^T = K . Q^T over all
    // of D = 128.  V^T: lane (l16, lg) holds V[16b + 4lg + r][16db + l16] at
    // K-slot 4b + r (b = 0..7, r = 0..3): exactly the tokens its S^T
    // accumulators hold, so P goes from accumulators to operand in place.
    auto read_k8 = [&](const unsigned char* st, int row) -> i32x8_t {
      const u32x4_t a = *reinterpret_cast<const u32x4_t*>(st + row * RBYTES + (((2 * lg) ^ swz_f8(row)) << 4));
      const u32x4_t c = *reinterpret_cast<const u32x4_t*>(st + row * RBYTES + (((2 * lg + 1) ^ swz_f8(row)) << 4));
      return i32x8_t{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)c[0], (int)c[1], (int)c[2], (int)c[3]};
    };
    auto read_v8 = [&](const unsigned char* st, int db) -> i32x8_t {
      i32x2_t t[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int kk = l16 >> 1;                     // lanes 2k, 2k+1 point at token k
        const int row = 16 * (2 * h + (kk >> 2)) + 4 * lg + (kk & 3);
        const int off = row * RBYTES + ((db ^ swz_f8(row)) << 4) + ((l16 & 1) << 3);
        t[h] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(st + off));
      }
      return i32x8_t{t[0][0], t[0][1], t[1][0], t[1][1], t[2][0], t[2][1], t[3][0], t[3][1]};
    };

    // fp4: K row m at lane group lg holds d = f4_slot(lg, n), two 8-byte runs
    // of the 64-byte row; V^T nibble n of lane (d, lg) is the token whose P
    // sits at the B operand's slot f4_slot(lg, n) (byte s of group g': token
    // 16(s/4) + 4g' + s%4), fetched by the 4-bit transpose reads, one token
    // per supplier lane.
    auto read_k4 = [&](const unsigned char* st, int row) -> i32x8_t {
      const int b0 = 32 * (lg & 1) + 8 * (lg >> 1);
      uint2 w[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int bb = b0 + 16 * h;
        w[h] = *reinterpret_cast<const uint2*>(st + row * RBYTES + (((bb >> 4) ^ swz_f4(row)) << 4) + (bb & 8));
      }
      return i32x8_t{(int)w[0].x, (int)w[0].y, (int)w[1].x, (int)w[1].y, 0, 0, 0, 0};
    };
    auto read_v4 = [&](const unsigned char* st, int db) -> i32x8_t {
      i32x2_t t[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = f4_slot(lg, 16 * h + l16);       // this supplier lane's slot
        const int gs = k >> 5, s8 = k & 31;
        const int row = 16 * (s8 >> 2) + 4 * gs + (s8 & 3);
        const int off = row * RBYTES + (((db >> 1) ^ swz_f4(row)) << 4) + ((db & 1) << 3);
        t[h] = __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_i32x2_t*)(st + off));
      }
      return i32x8_t{t[0][0], t[0][1], t[1][0], t[1][1], 0, 0, 0, 0};
    };

    // Tiles come in two kinds, told apart once per tile (the test is
    // wave-uniform): plain tiles, whose tokens are all prefix and all inside
    // the piece, and masked ones.  MASKED is a compile-time flag, so plain
    // tiles carry no per-score select at all.
    auto compute_f8 = [&](int st, int i, auto masked_tag) {
      constexpr bool MASKED = decltype(masked_tag)::value != 0;
      const unsigned char* ks = kst(st);
      const unsigned char* vs = vst(st);
      const int t0 = t_begin + i * TILE;
      // ---- S^T = K . Q^T: eight 16-token blocks, lane holds tokens 16b + 4lg + r
      f32x4_t sacc[RB][8];
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        if (kb == 4) asm volatile("" ::: "memory");   // K reads in two batches of four (registers)
        if constexpr (F4) {
          const i32x8_t a = read_k4(ks, 16 * kb + l16);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) sacc[rb][kb] = mfma_f4f8(a, qf8[rb], f32x4_t{0.f, 0.f, 0.f, 0.f});
        } else {
          const i32x8_t a = read_k8(ks, 16 * kb + l16);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) sacc[rb][kb] = mfma_f8(a, qf8[rb], f32x4_t{0.f, 0.f, 0.f, 0.f});
        }
      }
      // a 64-token half of the tile: all prefix inside the piece, past the
      // piece's end, or masked in registers
      auto half_vis = [&](uint64_t a, int th) -> uint64_t {
        if (th + kTile <= min(P, t_end)) return ~0ull;
        if (th >= t_end) return 0ull;
        return tile_visibility(a, th, P, t_end);
      };
      i32x8_t pb8[RB];
      float alpha[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        uint64_t vis[2] = {~0ull, ~0ull};
        if constexpr (MASKED) {
          vis[0] = half_vis(anc[rb], t0);
          vis[1] = half_vis(anc[rb], t0 + kTile);
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float s = sacc[rb][kb][r];
            if constexpr (MASKED) s = ((vis[kb >> 2] >> (16 * (kb & 3) + 4 * lg + r)) & 1ull) ? s : -INFINITY;
            sacc[rb][kb][r] = s;
            mx = fmaxf(mx, s);
          }
        mx = row4_max(mx) * srow[rb] - 8.0f;
        const float m_new = fmaxf(m_run[rb], mx);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        alpha[rb] = fast_exp2(m_run[rb] - m_use);
        m_run[rb] = m_new;
        float lsum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
          float p[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            p[r] = fast_exp2(__builtin_fmaf(sacc[rb][kb][r], srow[rb], -m_use));
            lsum += p[r];
          }
          pb8[rb][kb] = pack_e4m3x4(p[0], p[1], p[2], p[3]);
        }
        l_run[rb] = l_run[rb] * alpha[rb] + lsum;
      }
      bool moved = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) moved |= (alpha[rb] != 1.0f);
      if (__any(moved)) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[rb][db] *= alpha[rb];
      }
      // ---- O^T += V^T . P^T, 128 tokens per MFMA.  (The V reads stay below
      // the softmax: hoisted above it they hold 64 more registers.)
      asm volatile("" ::: "memory");
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        if constexpr (F4) {
          const i32x8_t a = read_v4(vs, db);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) oacc[rb][db] = mfma_f4f8(a, pb8[rb], oacc[rb][db]);
        } else {
          const i32x8_t a = read_v8(vs, db);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) oacc[rb][db] = mfma_f8(a, pb8[rb], oacc[rb][db]);
        }
      }
    };

    // fp8 scores over a bf16 cache: the workgroup's waves turn the K tile of
    // stage st into e4m3 codes in s_k8, 16 elements (one 16-byte unit of a
    // 128-byte code row, unit u of row r at (u ^ swz<8>(r))) at a time, then
    // meet at a barrier.  The codes are K / kq, kq the power of two of the
    // head's k_scale (values past 448 kq become NaN: a precondition).
    auto convert_k = [&](int stg) {
      if constexpr (S8) {
        constexpr int CPL = (kTile * 8) / (NW * kWave);   // 16-element units per lane
        static_assert(CPL * NW * kWave == kTile * 8, "code units split evenly over the lanes");
        const float kq = k_scale ? __uint_as_float(__float_as_uint(k_scale[kvh]) & 0x7F800000u) : 1.0f;
        const unsigned char* ks = kst(stg);
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
          const int ci = lane + kWave * (wave + NW * k);
          const int row = ci >> 3, c8 = ci & 7;
          typedef short s16x2_t __attribute__((ext_vector_type(2)));
          u32x4_t wd;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const bf16x8_t x =
                *reinterpret_cast<const bf16x8_t*>(ks + row * RBYTES + (((2 * c8 + h) ^ swz<UPR>(row)) << 4));
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              s16x2_t r{0, 0};
              r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, bf16x2_t{x[4 * j], x[4 * j + 1]}, kq, false);
              r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, bf16x2_t{x[4 * j + 2], x[4 * j + 3]}, kq, true);
              wd[2 * h + j] = __builtin_bit_cast(uint32_t, r);
            }
          }
          *reinterpret_cast<u32x4_t*>(s_k8 + row * 128 + ((c8 ^ swz<8>(row)) << 4)) = wd;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0): the codes are in LDS
        wg_barrier();
      }
    };

    auto compute = [&](int st, int i, auto masked_tag) {
      constexpr bool MASKED = decltype(masked_tag)::value != 0;
      const unsigned char* ks = kst(st);
      const unsigned char* vs = vst(st);
      const int t0 = t_begin + i * kTile;
      // ---- S^T = K . Q^T for this wave's chunks of the tile
      f32x4_t sacc[RB][CPT][2];
      if constexpr (S8) {
        // one 16x16x128 e4m3 MFMA per 16 tokens and row block: lane (m =
        // l16, lg) holds the codes K8[row][32lg .. 32lg+31] (contraction slot
        // 32lg + byte), rows in the chunk_token order of the bf16 path, so the
        // accumulators come out in its layout
        // the CPT * 2 code fragments (cp, G): all reads first, then the products
        u32x4_t a0[CPT * 2], a1[CPT * 2];
#pragma unroll
        for (int f = 0; f < CPT * 2; ++f) {
          const int row = 32 * (wt * CPT + f / 2) + chunk_token(f % 2, l16);
          a0[f] = *reinterpret_cast<const u32x4_t*>(s_k8 + row * 128 + (((2 * lg) ^ swz<8>(row)) << 4));
          a1[f] = *reinterpret_cast<const u32x4_t*>(s_k8 + row * 128 + (((2 * lg + 1) ^ swz<8>(row)) << 4));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int f = 0; f < CPT * 2; ++f) {
          const i32x8_t a{(int)a0[f][0], (int)a0[f][1], (int)a0[f][2], (int)a0[f][3],
                          (int)a1[f][0], (int)a1[f][1], (int)a1[f][2], (int)a1[f][3]};
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) sacc[rb][f / 2][f % 2] = mfma_f8(a, qf8[rb], f32x4_t{0.f, 0.f, 0.f, 0.f});
        }
      } else {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int cp = 0; cp < CPT; ++cp)
#pragma unroll
            for (int G = 0; G < 2; ++G) sacc[rb][cp][G] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // K fragments (cp, c, G), kFragBatch in flight
        constexpr int NF = CPT * KC * 2;
        bf16x8_t ka[NF];
        batched_products<NF, (NF < kFragBatch ? NF : kFragBatch)>(
            [&](int f) {
              const int cp = f / (KC * 2), c = (f / 2) % KC, G = f % 2;
              ka[f] = read_k(ks, 32 * (wt * CPT + cp) + chunk_token(G, l16), c);
            },
            [&](int f) {
              const int cp = f / (KC * 2), c = (f / 2) % KC, G = f % 2;
#pragma unroll
              for (int rb = 0; rb < RB; ++rb)
                sacc[rb][cp][G] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[f], qreg[rb][c], sacc[rb][cp][G], 0, 0, 0);
            });
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- mask, online softmax (base 2), P in bf16
      bf16x8_t pb[RB][CPT];
      float alpha[RB];
      // each lane's max over its raw scores (the scale is positive, so it
      // keeps the order and commutes with the max exactly), masked tokens to
      // -inf
      float mxl[RB];
      bool over = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        // this lane's 8 tokens of chunk cp sit at bits 32*ch + 8*lg .. +7
        uint32_t vis8[CPT];
        if constexpr (MASKED) {
          const uint64_t vis = tile_visibility(anc[rb], t0, P, t_end);
#pragma unroll
          for (int cp = 0; cp < CPT; ++cp) vis8[cp] = (uint32_t)(vis >> (32 * (wt * CPT + cp) + 8 * lg)) & 0xFFu;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int cp = 0; cp < CPT; ++cp)
#pragma unroll
          for (int G = 0; G < 2; ++G)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float s = sacc[rb][cp][G][r];
              if constexpr (MASKED) s = ((vis8[cp] >> (4 * G + r)) & 1u) ? s : -INFINITY;
              sacc[rb][cp][G][r] = s;
              mx = fmaxf(mx, s);
            }
        mxl[rb] = mx;
        over = over || (mx * srow[rb] > m_run[rb] + kMaxLag);
      }
      // The reference max of a row moves only when the tile's max passes it
      // by more than kMaxLag (base 2): p then stays at most 2^8, which bf16
      // and the fp32 sums hold exactly as well as p <= 1, and O, l and m stay
      // consistent, so the result is the same softmax; O is rescaled on about
      // the first tile only.  No lane's own max passing its row's reference
      // means no row's max does (the row max is the largest lane max), so the
      // cross-lane reduction runs only when some lane's does.
      const bool any_over = __any(over);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        alpha[rb] = 1.0f;
        if (any_over) {
          const float m_new = fmaxf(m_run[rb], row4_max(mxl[rb]) * srow[rb]);
          const bool bump = m_new > m_run[rb] + kMaxLag;
          const float m_keep = bump ? m_new : m_run[rb];
          alpha[rb] = bump ? fast_exp2(m_run[rb] - ((m_keep == -INFINITY) ? 0.0f : m_keep)) : 1.0f;
          m_run[rb] = m_keep;
        }
        const float m_use = (m_run[rb] == -INFINITY) ? 0.0f : m_run[rb];
        // p = 2^(s*scale - m) with one fma; the row sum (for the output's
        // normalisation and the exact log-sum-exp) is over the fp32 p
        float lsum = 0.0f;
#pragma unroll
        for (int cp = 0; cp < CPT; ++cp)
#pragma unroll
          for (int G = 0; G < 2; ++G)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float p = fast_exp2(__builtin_fmaf(sacc[rb][cp][G][r], srow[rb], -m_use));
              lsum += p;
              pb[rb][cp][4 * G + r] = (__bf16)p;
            }
        l_run[rb] = l_run[rb] * alpha[rb] + lsum;
      }
      // rescale O only when some row's reference max moved (alpha != 1)
      bool moved = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) moved |= (alpha[rb] != 1.0f);
      if (__any(moved)) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[rb][db] *= alpha[rb];
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- O^T += V^T . P^T, V fragments (cp, db) batched as K's
      {
        constexpr int NF = CPT * DB;
        bf16x8_t va[NF];
        batched_products<NF, (NF < kFragBatch ? NF : kFragBatch)>(
            [&](int f) { va[f] = read_v(vs, wt * CPT + f / DB, f % DB); },
            [&](int f) {
#pragma unroll
              for (int rb = 0; rb < RB; ++rb)
                oacc[rb][f % DB] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[f], pb[rb][f / DB], oacc[rb][f % DB], 0, 0, 0);
            });
      }
    };

    // ring: wait for tile i (the tiles after it stay in flight), make it visible
    // to all waves, refill the stage tile i-1 used, compute tile i
    int st = 0;
    // the ring stage is a compile-time constant in the unrolled plain loop
    // (LDS addresses then take it as an immediate offset)
    auto tile_step_c = [&](int i, auto masked_tag, auto stage_tag) {
      constexpr int sc = decltype(stage_tag)::value;
      const int ahead = min(NSTAGE - 2, ntiles - 1 - i);
      if (i >= NSTAGE - 1) switch (ahead) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<1 * PT>(); break;
        case 2: if constexpr (NSTAGE > 3) wait_vmcnt<2 * PT>(); break;
        case 3: if constexpr (NSTAGE > 4) wait_vmcnt<3 * PT>(); break;
        case 4: if constexpr (NSTAGE > 5) wait_vmcnt<4 * PT>(); break;
        case 5: if constexpr (NSTAGE > 6) wait_vmcnt<5 * PT>(); break;
        default: if constexpr (NSTAGE > 7) wait_vmcnt<6 * PT>(); break;
      }
      wg_barrier();
      if (i + NSTAGE - 1 < ntiles) issue(sc == 0 ? NSTAGE - 1 : sc - 1, i + NSTAGE - 1);
      convert_k(sc);
      if constexpr (F8) compute_f8(sc, i, masked_tag);
      else compute(sc, i, masked_tag);
    };
    auto tile_step = [&](int i, auto masked_tag) {
      const int ahead = min(NSTAGE - 2, ntiles - 1 - i);
      // tiles 0 .. NSTAGE-2 went out before the loads' wait above and have
      // landed; the counted waits start with the first tile the loop issued
      if (i >= NSTAGE - 1) switch (ahead) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<1 * PT>(); break;
        case 2: if constexpr (NSTAGE > 3) wait_vmcnt<2 * PT>(); break;
        case 3: if constexpr (NSTAGE > 4) wait_vmcnt<3 * PT>(); break;
        case 4: if constexpr (NSTAGE > 5) wait_vmcnt<4 * PT>(); break;
        case 5: if constexpr (NSTAGE > 6) wait_vmcnt<5 * PT>(); break;
        default: if constexpr (NSTAGE > 7) wait_vmcnt<6 * PT>(); break;
      }
      wg_barrier();
      if (i + NSTAGE - 1 < ntiles) issue(st == 0 ? NSTAGE - 1 : st - 1, i + NSTAGE - 1);
      convert_k(st);
      if constexpr (F8) compute_f8(st, i, masked_tag);
      else compute(st, i, masked_tag);
      st = (st + 1 == NSTAGE) ? 0 : st + 1;
    };
    // Plain tiles (every token prefix and inside the piece) come first, the
    // masked ones (tree rows, the piece's ragged end) after them: two loops,
    // so the plain loop holds none of the masked path's registers.
    const int n_plain = __builtin_amdgcn_readfirstlane(max(0, min(ntiles, (min(P, t_end) - t_begin) / TILE)));
    const int n_unr = n_plain - n_plain % NSTAGE;
    for (int i = 0; i < n_unr; i += NSTAGE) {
      tile_step_c(i, Int<0>{}, Int<0>{});
      tile_step_c(i + 1, Int<0>{}, Int<1>{});
      if constexpr (NSTAGE > 2) tile_step_c(i + 2, Int<0>{}, Int<2 % NSTAGE>{});
      if constexpr (NSTAGE > 3) tile_step_c(i + 3, Int<0>{}, Int<3 % NSTAGE>{});
    }
    static_assert(NSTAGE <= 4, "the plain loop unrolls up to 4 stages");
    for (int i = n_unr; i < n_plain; ++i) tile_step(i, Int<0>{});
    for (int i = n_plain; i < ntiles; ++i) tile_step(i, Int<1>{});
    // ---- waves that split the tile's tokens combine their states in LDS
    if constexpr (WT == 2) {
      // scratch in the ring: O blocks (1 KB per row block and column block)
      // first, then (m, l) pairs (512 B per row block)
      constexpr int OBYTES = WM * RB * DB * 1024;
      static_assert(OBYTES + WM * RB * 512 <= NSTAGE * 2 * TB, "combine scratch");
      __syncthreads();                                    // all DMA and LDS stage reads are done
      auto scratch = [&](int off) -> unsigned char* { return smem + off; };
      auto oslot = [&](int blk, int db) -> f32x4_t* {
        return reinterpret_cast<f32x4_t*>(scratch((blk * DB + db) * 1024)) + lane;
      };
      auto mlslot = [&](int blk) -> float2* {
        return reinterpret_cast<float2*>(scratch(OBYTES + blk * 512)) + lane;
      };
      if (wt == 1) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
          for (int db = 0; db < DB; ++db) *oslot(wm * RB + rb, db) = oacc[rb][db];
          *mlslot(wm * RB + rb) = make_float2(m_run[rb], l_run[rb]);
        }
      }
      __syncthreads();
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (wt == 1) break;                              // combined state lives in the wt == 0 waves
        const float2 o = *mlslot(wm * RB + rb);
        const float m_new = fmaxf(m_run[rb], o.x);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        const float a0 = fast_exp2(m_run[rb] - m_use), a1 = fast_exp2(o.x - m_use);
        m_run[rb] = m_new;
        l_run[rb] = l_run[rb] * a0 + o.y * a1;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[rb][db] = oacc[rb][db] * a0 + *oslot(wm * RB + rb, db) * a1;
      }
    }


    // ---- epilogue: lane holds O^T[16db + 4lg + r][row l16]
    if (direct) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (wt != 0) break;                          // the token-split partner waves hold no result
        const float l = row4_sum(l_run[rb]);
        const int row = row0 + rb * 16 + l16;
        if (row >= M) continue;
        const int i = row / g, hl = row % g;
        const float inv = out_scale / l;
        __bf16* op = out + ((size_t)(b * N + i) * Hq + kvh * g + hl) * D + 4 * lg;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          bf16x4_t v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = (__bf16)(oacc[rb][db][r] * inv);
          *reinterpret_cast<bf16x4_t*>(op + 16 * db) = v;
        }
        if (lse && lg == 0) lse[(size_t)(b * N + i) * Hq + kvh * g + hl] = (m_run[rb] + log2f(l)) * kLn2;
      }
    } else if (wt == 0) {
      // Partials go out in the lanes' own order (16 B per lane, 1 KB per wave
      // store, fully coalesced): chunk ((wm*RB + rb)*DB + db)*64 + lane of the
      // slot's O block, and (m, l) of row (wm*RB + rb)*16 + l16.  They are
      // read by another workgroup of this launch, maybe on another XCD, so
      // the stores are device scope.
      const __amdgpu_buffer_rsrc_t ro = dev_rsrc(part_o + part_row(my_slot, 0) * D, MT * D * 4);
      const __amdgpu_buffer_rsrc_t rm = dev_rsrc(part_ml + part_row(my_slot, 0), MT * 8);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float l = row4_sum(l_run[rb]);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          store_dev4(ro, (((wm * RB + rb) * DB + db) * kWave + lane) * 16, oacc[rb][db] * out_scale);
        if (lg == 0) store_dev2(rm, ((wm * RB + rb) * 16 + l16) * 8, m_run[rb], l);
      }
    }
    if (direct) continue;

    // ---- merge, fused: the last workgroup to finish a piece of this
    // (request, kv head, M-tile) combines every piece's partial in unit order,
    // so the result does not depend on which workgroup that is.  The per-
    // sequence counter lives in the workspace; it starts at zero and the
    // merging workgroup resets it, leaving the workspace ready for the next
    // call.
    wait_vmcnt<0>();                                 // this lane's partial stores have completed
    __syncthreads();                                 // ... for every lane
    uint32_t* cnt = counters + (size_t)(b * Hkv + kvh) * n_mt + mt;
    if (tid == 0) {
      const uint32_t seen = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      s_last = (seen == (uint32_t)(npieces - 1)) ? 1u : 0u;
    }
    __syncthreads();
    if (!s_last) continue;
    // Every load of the merge is independent and each costs a trip to the
    // device coherence point, so they are issued together: a thread owns IPT
    // 16-byte chunks of the lane-ordered partial block and loads, per round,
    // BATCH chunks x SG pieces plus each piece's (m, l) for the chunk's row;
    // rounds over further pieces rescale the running sums (online softmax
    // over the pieces).
    constexpr int NT = NW * kWave;
    constexpr int NCHUNK = MT * D / 4;                 // 16-byte chunks per block
    static_assert(NCHUNK % NT == 0, "merge chunks split evenly over the threads");
    constexpr int IPT = NCHUNK / NT;                   // chunks per thread
    constexpr int BATCH = IPT < 8 ? IPT : 8;
    constexpr int SG = 16 / BATCH;                     // pieces per load round
    static_assert(IPT % BATCH == 0, "merge batches");
#pragma unroll
    for (int k0 = 0; k0 < IPT; k0 += BATCH) {
      float m[BATCH], den[BATCH];
      f32x4_t acc[BATCH];
#pragma unroll
      for (int k = 0; k < BATCH; ++k) {
        m[k] = -INFINITY;
        den[k] = 0.f;
        acc[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
      for (int s0 = 0; s0 < npieces; s0 += SG) {
        float2 ml[SG][BATCH];
        f32x4_t o[SG][BATCH];
#pragma unroll
        for (int j = 0; j < SG; ++j) {
          const int sp = s0 + j;
          const int sl = fixed ? u_first + sp : 2 * (u_first + sp) + ((sp == 0 && first_odd) ? 1 : 0);
          const __amdgpu_buffer_rsrc_t ro = dev_rsrc(part_o + part_row(sl, 0) * D, MT * D * 4);
          const __amdgpu_buffer_rsrc_t rm = dev_rsrc(part_ml + part_row(sl, 0), MT * 8);
#pragma unroll
          for (int k = 0; k < BATCH; ++k) {
            const int c = tid + (k0 + k) * NT;
            const int rloc = (c / (DB * kWave)) * 16 + (c & 15);
            ml[j][k] = make_float2(-INFINITY, 0.f);
            o[j][k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (sp < npieces) {
              ml[j][k] = load_dev2(rm, rloc * 8);
              o[j][k] = load_dev4(ro, c * 16);
            }
          }
        }
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
          float mc = m[k];
#pragma unroll
          for (int j = 0; j < SG; ++j) mc = fmaxf(mc, ml[j][k].x);
          const float m_use = (mc == -INFINITY) ? 0.f : mc;
          const float a = fast_exp2(m[k] - m_use);
          den[k] *= a;
          acc[k] *= a;
#pragma unroll
          for (int j = 0; j < SG; ++j) {
            const float w = fast_exp2(ml[j][k].x - m_use);
            den[k] += w * ml[j][k].y;
            acc[k] += w * o[j][k];
          }
          m[k] = mc;
        }
      }
#pragma unroll
      for (int k = 0; k < BATCH; ++k) {
        const int c = tid + (k0 + k) * NT;
        const int ln = c & 63;
        const int db = (c / kWave) % DB;
        const int row = mt * MT + (c / (DB * kWave)) * 16 + (ln & 15);
        if (row >= M) continue;
        const int i = row / g, hl = row % g;
        const size_t orow = (size_t)(b * N + i) * Hq + kvh * g + hl;
        const float inv = 1.0f / den[k];
        bf16x4_t v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[k][e] * inv);
        *reinterpret_cast<bf16x4_t*>(out + orow * D + 16 * db + 4 * (ln >> 4)) = v;
        if (lse && db == 0 && ln < 16) lse[orow] = (m[k] + log2f(den[k])) * kLn2;
      }
    }
    if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  wait_vmcnt<0>();   // a unit whose range came out empty still has its guessed tiles in flight
  if (held_g >= 0) prep_leave();
}

// fp32 Q/K/V: one workgroup of kF32Waves waves per (request, node, head),
// exact fp32 arithmetic on the VALU.  Wave w takes the 64-key chunks w,
// w + kF32Waves, ... with its own online softmax; per chunk: lane = key for
// the scores (its K row's loads all in flight together), then lane = output
// column for the PV sum, with the chunk's 64 V rows loaded at once and each
// key's p read from its lane.  The waves' states are merged in LDS at the end.
// The whole verify step in one launch (STEP): blocks past the attention's
// grid take the prep role (masks, argmax, accept walk), and each attention
// wave builds its node's ancestor set from pa.parents itself.
constexpr int kF32Waves = 4;

template <int D, bool STEP>
__global__ __launch_bounds__(kF32Waves * kWave) void tree_attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kc, const float* __restrict__ vc,
    const int32_t* __restrict__ prefix_lens, const uint64_t* __restrict__ anc_mask, int N,
    int Hq, int Hkv, int S_max, float sm_scale, float* __restrict__ out, float* __restrict__ lse,
    uint32_t* __restrict__ err_word, int B, int attn_grid, const PrepArgs pa) {
  constexpr int NT = kF32Waves * kWave;
  if constexpr (STEP) {
    if ((int)blockIdx.x >= attn_grid) {
      prep_block<NT, kPrepUnroll>(pa, (int)blockIdx.x - attn_grid, B, N, err_word);
      return;
    }
  }
  constexpr int DPL = D / kWave;                 // output columns per lane
  const int h = blockIdx.x % Hq;
  const int i = (blockIdx.x / Hq) % N;
  const int b = blockIdx.x / (Hq * N);
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int kvh = h / (Hq / Hkv);
  const int P = prefix_lens[b];
  if (P < 0 || P > S_max - N) {
    if (threadIdx.x == 0 && i == 0 && h == 0) flag_error(err_word, SPEC_DERR_PREFIX);
    return;
  }
  const int L = P + N;
  uint64_t anc;
  if constexpr (STEP) {
    // the request's ancestor-or-self sets by pointer doubling across the wave
    // (lane = node; a request with a bad parent gets self-only sets, as the
    // mask build writes them), then this node's
    const int par = lane < N ? pa.parents[(size_t)b * N + lane] : 0;
    bool req_bad;
    anc = shfl_u64(ancestor_set(par, lane, lane < N, nullptr, &req_bad), i);
  } else {
    anc = anc_mask[(size_t)b * N + i];
  }
  const float* qp = q + ((size_t)(b * N + i) * Hq + h) * D;
  float qv[D];
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    const float4 x = *reinterpret_cast<const float4*>(qp + d);
    qv[d] = x.x; qv[d + 1] = x.y; qv[d + 2] = x.z; qv[d + 3] = x.w;
  }
  const float* kb = kc + ((size_t)(b * Hkv + kvh) * S_max) * D;
  const float* vb = vc + ((size_t)(b * Hkv + kvh) * S_max) * D;
  const float scale_log2 = sm_scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.f;
  float o[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) o[k] = 0.f;

  for (int c0 = wave * kWave; c0 < L; c0 += kF32Waves * kWave) {
    const int cmax = min(kWave, L - c0);
    // this chunk's V rows, one column set per lane, all loads in flight
    float vv[kWave][DPL];
#pragma unroll
    for (int j = 0; j < kWave; ++j)
#pragma unroll
      for (int k = 0; k < DPL; ++k)
        vv[j][k] = (j < cmax) ? vb[(size_t)(c0 + j) * D + lane + k * kWave] : 0.f;
    const int c = c0 + lane;
    const bool ok = (c < L) && (c < P || ((anc >> (c - P)) & 1ull));
    float s = -INFINITY;
    if (ok) {
      const float* kr = kb + (size_t)c * D;
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; d += 4) {
        const float4 x = *reinterpret_cast<const float4*>(kr + d);
        acc = fmaf(qv[d], x.x, acc);
        acc = fmaf(qv[d + 1], x.y, acc);
        acc = fmaf(qv[d + 2], x.z, acc);
        acc = fmaf(qv[d + 3], x.w, acc);
      }
      s = acc * scale_log2;
    }
    const float m_new = fmaxf(m_run, wave_max(s));
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    const float p = exp2f(s - m_use);
    l_run = l_run * alpha + wave_sum(p);
    m_run = m_new;
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      float acc = o[k] * alpha;
#pragma unroll
      for (int j = 0; j < kWave; ++j)
        acc = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), j)), vv[j][k], acc);
      o[k] = acc;
    }
  }
  // merge the waves' states (a wave with no chunk holds m = -inf, l = 0, o = 0)
  __shared__ float s_m[kF32Waves], s_l[kF32Waves];
  __shared__ float s_o[kF32Waves][D];
  if (lane == 0) {
    s_m[wave] = m_run;
    s_l[wave] = l_run;
  }
#pragma unroll
  for (int k = 0; k < DPL; ++k) s_o[wave][lane + k * kWave] = o[k];
  __syncthreads();
  if (wave != 0) return;
  float m_tot = s_m[0];
#pragma unroll
  for (int w = 1; w < kF32Waves; ++w) m_tot = fmaxf(m_tot, s_m[w]);   // finite: the node sees itself
  float l_tot = 0.f, acc[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
#pragma unroll
  for (int w = 0; w < kF32Waves; ++w) {
    const float a = exp2f(s_m[w] - m_tot);
    l_tot = fmaf(s_l[w], a, l_tot);
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = fmaf(s_o[w][lane + k * kWave], a, acc[k]);
  }
  float* op = out + ((size_t)(b * N + i) * Hq + h) * D;
  const float inv = 1.0f / l_tot;
#pragma unroll
  for (int k = 0; k < DPL; ++k) op[lane + k * kWave] = acc[k] * inv;
  if (lse && lane == 0) lse[(size_t)(b * N + i) * Hq + h] = (m_tot + log2f(l_tot)) * kLn2;
}

// ------------------------------------------------------------------ planning

struct AttnPlan {
  int rb, wm, wt, nstage, mt_rows, n_mt, M_pad;
  int split_len, n_splits, n_units;
  size_t ws_bytes;
};

// Bytes of LDS a workgroup holds besides its K/V ring: the request-length
// table and the merge flag.
constexpr int kTableBytes = 4 * (1024 + 1) + 4;

// Rows per workgroup follow the packed M = g*N.  Small M (<= 32) lets the
// waves also split each tile's tokens (a 3-stage K/V ring, one workgroup per
// CU); larger M splits rows over the waves (a 2-stage ring, two workgroups per
// CU, so two waves share each SIMD).  Above 128 rows with D = 128, when 256-row
// tiles pad M no further than 128-row ones, one 8-wave workgroup a CU takes
// 256 rows (with D = 64 an e4m3 tile is too small to give all 8 waves a DMA
// instruction, so D = 64 keeps 128-row tiles): each
// K/V tile then reaches LDS once for 256 rows instead of twice for 128 (60-node
// trees of 16 heads at 32768 tokens: 971 -> 920 us).  Work then comes in about one unit per
// resident workgroup slot (256 CUs), each unit for all M-tiles, under one of
// two schedules the kernel picks from the data: fixed splits of S_max
// (whole 64-token tiles, at least 4, dealt out evenly) when every request
// fills its cache, or equal shares of the actual tokens otherwise.  The plan does not depend on
// the cached dtype, so one workspace size serves every format: partial
// results for the larger of the two slot counts (a fixed split each, or two
// per balanced unit) and one counter per (request, kv head, M-tile).
static bool make_plan(int B, int N, int Hq, int Hkv, int D, int S_max, AttnPlan* p) {
  if (B < 1 || B > 1024 || N < 1 || N > SPEC_MAX_NODES || Hkv < 1 || Hq < Hkv || Hq % Hkv) return false;
  if (D != 64 && D != 128) return false;
  if (S_max < N) return false;
  if ((long long)B * S_max >= (1ll << 31) || (long long)Hkv * S_max >= (1ll << 31)) return false;
  // query rows index in int (B * N * Hq of them; the packed M = g * N is at most that)
  if ((long long)B * N * Hq >= (1ll << 31)) return false;
  const int M = (Hq / Hkv) * N;
  if (M <= 32) { p->rb = 1; p->wm = 2; p->wt = 2; p->nstage = 3; }
  else if (M <= 64) { p->rb = 2; p->wm = 2; p->wt = 1; p->nstage = 2; }
  else if (D != 128 || ((M + 127) / 128) % 2 == 1) { p->rb = 2; p->wm = 4; p->wt = 1; p->nstage = 2; }
  else { p->rb = 2; p->wm = 8; p->wt = 1; p->nstage = 2; }
  const int lds_bf16 = p->nstage * 2 * kTile * D * 2 + kTableBytes;
  // an 8-wave workgroup takes both of a CU's wave slots per SIMD at this
  // register budget: one a CU
  const long long per_cu = p->wm * p->wt >= 8 ? 1 : std::max(1, std::min(2, (160 * 1024) / lds_bf16));
  long long target_wgs = 256 * per_cu;
  p->mt_rows = p->rb * p->wm * 16;
  p->n_mt = (M + p->mt_rows - 1) / p->mt_rows;
  p->M_pad = p->n_mt * p->mt_rows;
  p->n_units = (int)std::max<long long>(1, target_wgs / p->n_mt);
  const long long seqs = (long long)B * Hkv;
  const int want = (int)std::max<long long>(1, (p->n_units + seqs - 1) / seqs);
  // fixed splits of whole 64-token tiles, at least 4 each: split_len / 64
  // tiles to a split, one more to each of the last (tiles mod n_splits)
  const int tiles = (S_max + kTile - 1) / kTile;
  p->n_splits = std::min(want, std::max(1, tiles / 4));
  p->split_len = (tiles / p->n_splits) * kTile;
  if (seqs * p->n_splits * p->n_mt >= (1ll << 31)) return false;
  const size_t slots = (size_t)std::max<long long>(seqs * p->n_splits, 2ll * p->n_units);
  const size_t rows = slots * p->M_pad;
  const size_t counters = (size_t)seqs * p->n_mt;
  p->ws_bytes = rows * (size_t)D * sizeof(float) + rows * sizeof(float2) + counters * sizeof(uint32_t);
  return true;
}

// Paged cache description (null table: contiguous caches).
struct PagedArgs {
  const int32_t* table;
  int max_pages, ps_log2, num_pages;
};

template <int D, int KVF, int RB, int WM, int WT, int NS, bool PAGED, bool STEP>
static void launch_split(const AttnPlan& pl, const void* q, const void* k, const void* v,
                         const float* ks, const float* vs, const int32_t* pre, const uint64_t* anc,
                         int B, int N, int Hq, int Hkv, int S_max, float sm_scale, void* out,
                         float* lse, float* po, float2* pml, uint32_t* cnt, uint32_t* err,
                         const PagedArgs& pg, const PrepArgs* prep, hipStream_t st) {
  const int units = std::max(B * Hkv * pl.n_splits, pl.n_units);
  const int units_pad = ((units + 7) / 8) * 8;
  const long long attn_grid = (long long)units_pad * pl.n_mt;
  // one-launch verify step: the prep workgroups follow the attention's
  PrepArgs pa{};
  long long grid = attn_grid;
  if constexpr (STEP) {
    pa = *prep;
    constexpr int TBB = (KVF == kKvF8Mma || KVF == kKvF4Mma ? 2 * kTile : kTile) *
                        (KVF == kKvF4Mma ? D / 2 : D * (KVF == SPEC_BF16 || KVF == kKvBf16F8S ? 2 : 1));
    constexpr int PU = std::min(kPrepUnroll, (2 * TBB) / (WM * WT * kWave * 16));
    grid += plan_prep(&pa, B, N, WM * WT * kWave, attn_grid, PU);
  }
  hipLaunchKernelGGL((tree_attn_split_kernel<D, KVF, RB, WM, WT, NS, PAGED, STEP>), dim3((unsigned)grid),
                     dim3(WM * WT * kWave), 0, st, static_cast<const __bf16*>(q),
                     static_cast<const unsigned char*>(k), static_cast<const unsigned char*>(v), ks, vs, pre,
                     anc, B, N, Hq, Hkv, S_max, sm_scale, pl.split_len, pl.n_splits, pl.n_units, pl.n_mt,
                     static_cast<__bf16*>(out), lse, po, pml, cnt, err, pg.table, pg.max_pages, pg.ps_log2,
                     pg.num_pages, (int)attn_grid, pa);
}

// Whether an instantiation is buildable: the ring (plus the length table and,
// for paged caches, the page ids) fits the LDS, the tiles in flight fit the
// vmcnt counter, the DMA splits evenly over the waves and the token-split
// combine has scratch room.
template <int D, int KVF, int RB, int WM, int WT, int NS, bool PAGED>
constexpr bool split_fits() {
  constexpr bool FA = (KVF == kKvF8Mma || KVF == kKvF4Mma);
  constexpr bool S8 = (KVF == kKvBf16F8S);
  constexpr int TB = (FA ? 2 * kTile : kTile) * (KVF == kKvF4Mma ? D / 2 : D * ((KVF == SPEC_BF16 || S8) ? 2 : 1));
  constexpr int NW = WM * WT;
  constexpr int NLOAD = TB / 1024;
  if (NS * 2 * TB + kTableBytes + (PAGED ? 4 * kMaxPages : 0) + (S8 ? kTile * 128 : 0) > 160 * 1024) return false;
  if (S8 && (D != 128 || PAGED || (kTile * 8) % (WM * WT * kWave) != 0)) return false;
  if (NLOAD % NW != 0) return false;
  if ((NS - 1) * 2 * (NLOAD / NW) >= 64) return false;   // a full ring start fits the vmcnt counter
  if ((KVF == kKvF8Mma || KVF == kKvF4Mma) && (WT != 1 || D != 128 || PAGED)) return false;
  if (WT == 2 && WM * RB * (D / 16) * 1024 + WM * RB * 512 > NS * 2 * TB) return false;
  return true;
}

// (RB, WM, WT, NSTAGE) instantiations the planner may pick.
#define SPEC_SPLIT_PLANS(X) X(1, 2, 2, 3) X(2, 2, 1, 2) X(2, 4, 1, 2) X(2, 8, 1, 2)
// The fp8-arithmetic path: every wave covers whole tiles (WT = 1); for M <= 32
// the plan keeps the 32-row tile of the bf16 plan, so the workspace is the same.
#define SPEC_F8_PLANS(X) X(1, 2, 1, 3) X(2, 2, 1, 2) X(2, 4, 1, 2) X(2, 8, 1, 2)

template <int D, int KVF, bool PAGED>
static bool dispatch_shape(const AttnPlan& pl, const void* q, const void* k, const void* v,
                           const float* ks, const float* vs, const int32_t* pre,
                           const uint64_t* anc, int B, int N, int Hq, int Hkv, int S_max,
                           float sm_scale, void* out, float* lse, float* po, float2* pml,
                           uint32_t* cnt, uint32_t* err, const PagedArgs& pg, const PrepArgs* prep,
                           hipStream_t st) {
#define SPEC_TRY(RB_, WM_, WT_, NS_)                                                                  \
  if constexpr (split_fits<D, KVF, RB_, WM_, WT_, NS_, PAGED>()) {                                    \
    if (pl.rb == RB_ && pl.wm == WM_ && pl.wt == WT_ && pl.nstage == NS_) {                           \
      if (!prep) {                                                                                    \
        launch_split<D, KVF, RB_, WM_, WT_, NS_, PAGED, false>(pl, q, k, v, ks, vs, pre, anc, B, N, Hq, Hkv, \
                                                               S_max, sm_scale, out, lse, po, pml, cnt, err, \
                                                               pg, prep, st);                          \
        return true;                                                                                  \
      }                                                                                               \
      if constexpr (KVF != kKvF8Mma && KVF != kKvF4Mma && KVF != kKvBf16F8S) {                         \
        launch_split<D, KVF, RB_, WM_, WT_, NS_, PAGED, true>(pl, q, k, v, ks, vs, pre, anc, B, N, Hq, Hkv, \
                                                              S_max, sm_scale, out, lse, po, pml, cnt, err, pg, \
                                                              prep, st);                              \
        return true;                                                                                  \
      }                                                                                               \
      return false;                                                                                   \
    }                                                                                                 \
  }
  if constexpr (KVF == kKvF8Mma || KVF == kKvF4Mma) {
    SPEC_F8_PLANS(SPEC_TRY)
  } else {
    SPEC_SPLIT_PLANS(SPEC_TRY)
  }
#undef SPEC_TRY
  return false;
}

}  // namespace spectree

using namespace spectree;

extern "C" size_t spec_tree_attn_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int S_max) {
  AttnPlan pl;
  if (!make_plan(B, N, Hq, Hkv, D, S_max, &pl)) return 0;
  return pl.ws_bytes;
}

static inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The split kernel for either cache layout (pg.table set: paged); kvf is
// SPEC_BF16, SPEC_FP8_E4M3 (decoded to bf16) or kKvF8Mma (fp8 arithmetic).
static spec_status run_split(const AttnPlan& pl, int kvf, const void* q, const void* k, const void* v,
                             const float* k_scale, const float* v_scale, const int32_t* prefix_lens,
                             const uint64_t* anc_mask, int B, int N, int Hq, int Hkv, int D, int S_max,
                             float sm_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                             uint32_t* err_word, const PagedArgs& pg, hipStream_t stream,
                             const PrepArgs* prep = nullptr) {
  float* po = nullptr;
  float2* pml = nullptr;
  uint32_t* cnt = nullptr;
  if (pl.ws_bytes) {
    if (!workspace) return SPEC_ERR_WORKSPACE;
    if (workspace_bytes < pl.ws_bytes) return SPEC_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SPEC_ERR_ALIGN;
    const size_t rows = (size_t)std::max<long long>((long long)B * Hkv * pl.n_splits, 2ll * pl.n_units) * pl.M_pad;
    po = static_cast<float*>(workspace);
    pml = reinterpret_cast<float2*>(static_cast<char*>(workspace) + rows * D * sizeof(float));
    cnt = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + rows * D * sizeof(float) +
                                      rows * sizeof(float2));
  }

  const bool paged = pg.table != nullptr;
  hip_clear_error();
#define SPEC_DISPATCH(D_, KVF_)                                                                           \
  (paged ? dispatch_shape<D_, KVF_, true>(pl, q, k, v, k_scale, v_scale, prefix_lens, anc_mask, B, N, Hq, Hkv, \
                                          S_max, sm_scale, out, lse, po, pml, cnt, err_word, pg, prep, stream)     \
         : dispatch_shape<D_, KVF_, false>(pl, q, k, v, k_scale, v_scale, prefix_lens, anc_mask, B, N, Hq,    \
                                           Hkv, S_max, sm_scale, out, lse, po, pml, cnt, err_word, pg, prep, stream))
  bool launched;
  if (kvf == SPEC_BF16) launched = (D == 64) ? SPEC_DISPATCH(64, SPEC_BF16) : SPEC_DISPATCH(128, SPEC_BF16);
  else if (kvf == SPEC_FP8_E4M3) launched = (D == 64) ? SPEC_DISPATCH(64, SPEC_FP8_E4M3) : SPEC_DISPATCH(128, SPEC_FP8_E4M3);
  else if (kvf == kKvBf16F8S)
    launched = (D == 128) && dispatch_shape<128, kKvBf16F8S, false>(pl, q, k, v, k_scale, v_scale, prefix_lens,
                                                                     anc_mask, B, N, Hq, Hkv, S_max, sm_scale, out,
                                                                     lse, po, pml, cnt, err_word, pg, prep, stream);
  else if (kvf == kKvF8Mma)
    launched = (D == 128) && dispatch_shape<128, kKvF8Mma, false>(pl, q, k, v, k_scale, v_scale, prefix_lens,
                                                                  anc_mask, B, N, Hq, Hkv, S_max, sm_scale, out,
                                                                  lse, po, pml, cnt, err_word, pg, prep, stream);
  else
    launched = (D == 128) && dispatch_shape<128, kKvF4Mma, false>(pl, q, k, v, k_scale, v_scale, prefix_lens,
                                                                  anc_mask, B, N, Hq, Hkv, S_max, sm_scale, out,
                                                                  lse, po, pml, cnt, err_word, pg, prep, stream);
#undef SPEC_DISPATCH
  if (!launched) return SPEC_ERR_SHAPE;
  if (launch_status() != SPEC_OK) return SPEC_ERR_HIP;

  return SPEC_OK;
}

namespace spectree {

// Every reason spec_tree_attn_verify can refuse a call before it launches
// anything (the fused verify step checks the same before its first launch).
spec_status tree_attn_check_args(const void* q, spec_dtype q_dtype, const void* k_cache, const void* v_cache,
                                 spec_dtype kv_dtype, const float* k_scale, const float* v_scale,
                                 const int32_t* prefix_lens, const uint64_t* anc_mask, int B, int N, int Hq,
                                 int Hkv, int D, int S_max, float sm_scale, const void* out) {
  if (!q || !k_cache || !v_cache || !prefix_lens || !anc_mask || !out) return SPEC_ERR_NULL;
  const bool f32 = (q_dtype == SPEC_F32 && kv_dtype == SPEC_F32);
  const bool bf16 = (q_dtype == SPEC_BF16 && kv_dtype == SPEC_BF16);
  const bool fp8 = (q_dtype == SPEC_BF16 && kv_dtype == SPEC_FP8_E4M3);
  if (!f32 && !bf16 && !fp8) return SPEC_ERR_DTYPE;
  if (fp8 && (!k_scale || !v_scale)) return SPEC_ERR_NULL;
  AttnPlan pl;
  if (!make_plan(B, N, Hq, Hkv, D, S_max, &pl)) return SPEC_ERR_SHAPE;
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale)) return SPEC_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return SPEC_ERR_ALIGN;
  return SPEC_OK;
}

spec_status tree_attn_check(const void* q, spec_dtype q_dtype, const void* k_cache, const void* v_cache,
                            spec_dtype kv_dtype, const float* k_scale, const float* v_scale,
                            const int32_t* prefix_lens, const uint64_t* anc_mask, int B, int N, int Hq,
                            int Hkv, int D, int S_max, float sm_scale, const void* out, const void* workspace,
                            size_t workspace_bytes) {
  const spec_status st = tree_attn_check_args(q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, prefix_lens,
                                              anc_mask, B, N, Hq, Hkv, D, S_max, sm_scale, out);
  if (st != SPEC_OK) return st;
  const bool f32 = (q_dtype == SPEC_F32 && kv_dtype == SPEC_F32);
  AttnPlan pl;
  make_plan(B, N, Hq, Hkv, D, S_max, &pl);
  if (!f32 && pl.ws_bytes) {
    if (!workspace || workspace_bytes < pl.ws_bytes) return SPEC_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SPEC_ERR_ALIGN;
  }
  return SPEC_OK;
}

}  // namespace spectree

// The fp32 kernel, alone or (prep set) with the verify step's prep role in
// the same launch.
static spec_status launch_f32(const void* q, const void* k_cache, const void* v_cache, const int32_t* prefix_lens,
                              const uint64_t* anc_mask, int B, int N, int Hq, int Hkv, int D, int S_max,
                              float sm_scale, void* out, float* lse, uint32_t* err_word, const PrepArgs* prep,
                              hipStream_t stream) {
  const long long attn_grid = (long long)B * N * Hq;
  long long grid = attn_grid;
  PrepArgs pa{};
  if (prep) {
    pa = *prep;
    grid += plan_prep(&pa, B, N, kF32Waves * kWave, 0, 0);
  }
  if (grid >= (1ll << 31)) return SPEC_ERR_SHAPE;
  hip_clear_error();
  const float* qf = static_cast<const float*>(q);
  const float* kf = static_cast<const float*>(k_cache);
  const float* vf = static_cast<const float*>(v_cache);
  float* of = static_cast<float*>(out);
#define SPEC_F32_LAUNCH(D_, STEP_)                                                                   \
  hipLaunchKernelGGL((tree_attn_f32_kernel<D_, STEP_>), dim3((unsigned)grid), dim3(kF32Waves * kWave), 0, \
                     stream, qf, kf, vf, prefix_lens, anc_mask, N, Hq, Hkv, S_max, sm_scale, of, lse, err_word, B, \
                     (int)attn_grid, pa)
  if (D == 64) {
    if (prep) SPEC_F32_LAUNCH(64, true);
    else SPEC_F32_LAUNCH(64, false);
  } else {
    if (prep) SPEC_F32_LAUNCH(128, true);
    else SPEC_F32_LAUNCH(128, false);
  }
#undef SPEC_F32_LAUNCH
  return launch_status();
}

namespace spectree {

spec_status tree_attn_f32_with_prep(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* prefix_lens, int B, int N, int Hq, int Hkv, int D, int S_max,
                                    float sm_scale, void* out, float* lse, uint32_t* err_word, const PrepArgs& prep,
                                    hipStream_t stream) {
  return launch_f32(q, k_cache, v_cache, prefix_lens, prep.anc_mask, B, N, Hq, Hkv, D, S_max, sm_scale, out, lse,
                    err_word, &prep, stream);
}

}  // namespace spectree

extern "C" spec_status spec_tree_attn_verify(const void* q, spec_dtype q_dtype, const void* k_cache,
                                             const void* v_cache, spec_dtype kv_dtype,
                                             const float* k_scale, const float* v_scale,
                                             const int32_t* prefix_lens, const uint64_t* anc_mask,
                                             int B, int N, int Hq, int Hkv, int D, int S_max,
                                             float sm_scale, void* out, float* lse,
                                             void* workspace, size_t workspace_bytes,
                                             uint32_t* err_word, hipStream_t stream) {
  const spec_status st = tree_attn_check(q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, prefix_lens,
                                         anc_mask, B, N, Hq, Hkv, D, S_max, sm_scale, out, workspace,
                                         workspace_bytes);
  if (st != SPEC_OK) return st;
  const bool f32 = (q_dtype == SPEC_F32);
  const bool bf16 = (kv_dtype == SPEC_BF16);
  AttnPlan pl;
  make_plan(B, N, Hq, Hkv, D, S_max, &pl);

  if (f32) return launch_f32(q, k_cache, v_cache, prefix_lens, anc_mask, B, N, Hq, Hkv, D, S_max, sm_scale, out,
                            lse, err_word, nullptr, stream);

  return run_split(pl, bf16 ? SPEC_BF16 : SPEC_FP8_E4M3, q, k_cache, v_cache, k_scale, v_scale, prefix_lens,
                   anc_mask, B, N, Hq, Hkv, D, S_max, sm_scale, out, lse, workspace, workspace_bytes, err_word,
                   PagedArgs{nullptr, 0, 0, 0}, stream);
}

namespace spectree {

spec_status tree_attn_verify_with_prep(const void* q, const void* k_cache, const void* v_cache, spec_dtype kv_dtype,
                                       const float* k_scale, const float* v_scale, const int32_t* prefix_lens,
                                       int B, int N, int Hq, int Hkv, int D, int S_max, float sm_scale, void* out,
                                       float* lse, void* workspace, size_t workspace_bytes, uint32_t* err_word,
                                       const PrepArgs& prep, hipStream_t stream) {
  AttnPlan pl;
  if (!make_plan(B, N, Hq, Hkv, D, S_max, &pl)) return SPEC_ERR_SHAPE;
  if (kv_dtype != SPEC_BF16 && kv_dtype != SPEC_FP8_E4M3) return SPEC_ERR_DTYPE;
  return run_split(pl, kv_dtype, q, k_cache, v_cache, k_scale, v_scale, prefix_lens, prep.anc_mask, B, N, Hq, Hkv,
                   D, S_max, sm_scale, out, lse, workspace, workspace_bytes, err_word, PagedArgs{nullptr, 0, 0, 0},
                   stream, &prep);
}

}  // namespace spectree

extern "C" spec_status spec_tree_attn_verify_f4(const void* q, const void* k_cache, const void* v_cache,
                                                const float* k_scale, const float* v_scale,
                                                const int32_t* prefix_lens, const uint64_t* anc_mask, int B, int N,
                                                int Hq, int Hkv, int D, int S_max, float sm_scale, void* out,
                                                float* lse, void* workspace, size_t workspace_bytes,
                                                uint32_t* err_word, hipStream_t stream) {
  if (!q || !k_cache || !v_cache || !k_scale || !v_scale || !prefix_lens || !anc_mask || !out) return SPEC_ERR_NULL;
  AttnPlan pl;
  if (!make_plan(B, N, Hq, Hkv, D, S_max, &pl) || D != 128) return SPEC_ERR_SHAPE;
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale)) return SPEC_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return SPEC_ERR_ALIGN;
  pl.wt = 1;
  return run_split(pl, kKvF4Mma, q, k_cache, v_cache, k_scale, v_scale, prefix_lens, anc_mask, B, N, Hq, Hkv, D,
                   S_max, sm_scale, out, lse, workspace, workspace_bytes, err_word, PagedArgs{nullptr, 0, 0, 0},
                   stream);
}

extern "C" spec_status spec_tree_attn_verify_f8_scores(const void* q, const void* k_cache, const void* v_cache,
                                                       const float* k_scale, const int32_t* prefix_lens,
                                                       const uint64_t* anc_mask, int B, int N, int Hq, int Hkv, int D,
                                                       int S_max, float sm_scale, void* out, float* lse,
                                                       void* workspace, size_t workspace_bytes, uint32_t* err_word,
                                                       hipStream_t stream) {
  if (!q || !k_cache || !v_cache || !prefix_lens || !anc_mask || !out) return SPEC_ERR_NULL;
  AttnPlan pl;
  if (!make_plan(B, N, Hq, Hkv, D, S_max, &pl) || D != 128) return SPEC_ERR_SHAPE;
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale)) return SPEC_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return SPEC_ERR_ALIGN;
  return run_split(pl, kKvBf16F8S, q, k_cache, v_cache, k_scale, nullptr, prefix_lens, anc_mask, B, N, Hq, Hkv, D,
                   S_max, sm_scale, out, lse, workspace, workspace_bytes, err_word, PagedArgs{nullptr, 0, 0, 0},
                   stream);
}

extern "C" spec_status spec_tree_attn_verify_f8(const void* q, const void* k_cache, const void* v_cache,
                                                const float* k_scale, const float* v_scale,
                                                const int32_t* prefix_lens, const uint64_t* anc_mask, int B, int N,
                                                int Hq, int Hkv, int D, int S_max, float sm_scale, void* out,
                                                float* lse, void* workspace, size_t workspace_bytes,
                                                uint32_t* err_word, hipStream_t stream) {
  if (!q || !k_cache || !v_cache || !k_scale || !v_scale || !prefix_lens || !anc_mask || !out) return SPEC_ERR_NULL;
  AttnPlan pl;
  if (!make_plan(B, N, Hq, Hkv, D, S_max, &pl) || D != 128) return SPEC_ERR_SHAPE;
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale)) return SPEC_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return SPEC_ERR_ALIGN;
  pl.wt = 1;                                         // whole tiles per wave; same rows, same workspace
  return run_split(pl, kKvF8Mma, q, k_cache, v_cache, k_scale, v_scale, prefix_lens, anc_mask, B, N, Hq, Hkv, D,
                   S_max, sm_scale, out, lse, workspace, workspace_bytes, err_word, PagedArgs{nullptr, 0, 0, 0},
                   stream);
}

namespace spectree {

// Every reason spec_tree_attn_verify_paged can refuse a call before it
// launches anything (the paged verify step checks the same first).
spec_status tree_attn_paged_check(const void* q, spec_dtype q_dtype, const void* k_pages, const void* v_pages,
                                  spec_dtype kv_dtype, const float* k_scale, const float* v_scale,
                                  const int32_t* prefix_lens, const uint64_t* anc_mask, const int32_t* block_table,
                                  int max_pages, int page_size, int num_pages, int B, int N, int Hq, int Hkv, int D,
                                  float sm_scale, const void* out) {
  if (!q || !k_pages || !v_pages || !prefix_lens || !anc_mask || !block_table || !out) return SPEC_ERR_NULL;
  const bool bf16 = (q_dtype == SPEC_BF16 && kv_dtype == SPEC_BF16);
  const bool fp8 = (q_dtype == SPEC_BF16 && kv_dtype == SPEC_FP8_E4M3);
  if (!bf16 && !fp8) return SPEC_ERR_DTYPE;
  if (fp8 && (!k_scale || !v_scale)) return SPEC_ERR_NULL;
  if (page_size < 1 || (page_size & (page_size - 1)) || page_size > 4096) return SPEC_ERR_SHAPE;
  if (max_pages < 1 || max_pages > kMaxPages || num_pages < 1) return SPEC_ERR_SHAPE;
  AttnPlan pl;
  if (!make_plan(B, N, Hq, Hkv, D, max_pages * page_size, &pl)) return SPEC_ERR_SHAPE;
  if ((long long)num_pages * page_size * Hkv * D >= (1ll << 40)) return SPEC_ERR_SHAPE;
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale)) return SPEC_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(out)) return SPEC_ERR_ALIGN;
  return SPEC_OK;
}

spec_status tree_attn_verify_paged_run(const void* q, spec_dtype q_dtype, const void* k_pages, const void* v_pages,
                                       spec_dtype kv_dtype, const float* k_scale, const float* v_scale,
                                       const int32_t* prefix_lens, const uint64_t* anc_mask,
                                       const int32_t* block_table, int max_pages, int page_size, int num_pages, int B,
                                       int N, int Hq, int Hkv, int D, float sm_scale, void* out, float* lse,
                                       void* workspace, size_t workspace_bytes, uint32_t* err_word,
                                       const PrepArgs* prep, hipStream_t stream) {
  const spec_status st = tree_attn_paged_check(q, q_dtype, k_pages, v_pages, kv_dtype, k_scale, v_scale, prefix_lens,
                                               anc_mask, block_table, max_pages, page_size, num_pages, B, N, Hq, Hkv,
                                               D, sm_scale, out);
  if (st != SPEC_OK) return st;
  const int S_max = max_pages * page_size;
  AttnPlan pl;
  make_plan(B, N, Hq, Hkv, D, S_max, &pl);
  int ps_log2 = 0;
  while ((1 << ps_log2) < page_size) ++ps_log2;
  return run_split(pl, kv_dtype, q, k_pages, v_pages, k_scale, v_scale, prefix_lens, anc_mask, B, N, Hq, Hkv, D,
                   S_max, sm_scale, out, lse, workspace, workspace_bytes, err_word,
                   PagedArgs{block_table, max_pages, ps_log2, num_pages}, stream, prep);
}

}  // namespace spectree

extern "C" spec_status spec_tree_attn_verify_paged(const void* q, spec_dtype q_dtype, const void* k_pages,
                                                   const void* v_pages, spec_dtype kv_dtype,
                                                   const float* k_scale, const float* v_scale,
                                                   const int32_t* prefix_lens, const uint64_t* anc_mask,
                                                   const int32_t* block_table, int max_pages, int page_size,
                                                   int num_pages, int B, int N, int Hq, int Hkv, int D,
                                                   float sm_scale, void* out, float* lse, void* workspace,
                                                   size_t workspace_bytes, uint32_t* err_word,
                                                   hipStream_t stream) {
  return tree_attn_verify_paged_run(q, q_dtype, k_pages, v_pages, kv_dtype, k_scale, v_scale, prefix_lens, anc_mask,
                                    block_table, max_pages, page_size, num_pages, B, N, Hq, Hkv, D, sm_scale, out,
                                    lse, workspace, workspace_bytes, err_word, nullptr, stream);
}
