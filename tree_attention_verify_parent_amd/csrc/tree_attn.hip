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
#include <type_traits>

#include "common.h"

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

// s_waitcnt vmcnt(N) with expcnt / lgkmcnt left unconstrained (gfx9 layout).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the memory fence of __syncthreads: that fence
// would force vmcnt(0) and drain the K/V prefetch.  LDS ordering is kept by
// explicit vmcnt waits (DMA writes land before the barrier) and by every LDS
// read being consumed before its wave reaches the next barrier.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

// 8 OCP e4m3 codes (little-endian in lo, hi) -> 8 bf16, exactly, by the
// hardware converter (scale 1.0).
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <int I>
using Int = std::integral_constant<int, I>;

// Device-scope (all XCDs) relaxed 64-bit store / load of two floats.  The
// hardware writes these through to the device coherence point and reads them
// from there, so a partial result written by one workgroup is seen by another
// workgroup of the same launch on any XCD once the writer's store has
// completed (vmcnt) and the reader has observed the split counter.
__device__ __forceinline__ void store_dev(float* p, float a, float b) {
  const uint64_t v = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_dev(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}

// Reductions over the four lanes {l, l^16, l^32, l^48} that share a query
// row.  v_permlane32_swap / v_permlane16_swap hand every lane the pair {its
// own value, its partner's}, in either order; max and + are commutative, so
// all four lanes end with bit-identical results.
__device__ __forceinline__ float row4_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 2^x on the transcendental unit (v_exp_f32): exp2(-inf) = 0, and results
// below the normal range flush to zero, which only drops weights < 2^-126.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

// One wave-wide 16-byte-per-lane DMA from global memory into LDS: lane l's
// 16 bytes land at LDS byte lds_addr + 16*l (lds_addr wave-uniform, via M0).
// Issued as inline assembly so the compiler's wait-count pass does not treat
// every later LDS read as depending on every DMA in flight; the kernel orders
// them itself with s_waitcnt vmcnt(N) before each barrier.
__device__ __forceinline__ void dma16(const void* gptr, const unsigned char* lds_ptr) {
  const uint32_t lds_addr = (uint32_t)(size_t)(lds_void_t*)lds_ptr;
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_addr)
               : "memory", "m0");
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
  static constexpr int ring_bf16 = NSTAGE * 2 * kTile * D * 2;
  static constexpr int fit = (160 * 1024) / ring_bf16;
  static constexpr int wg_per_cu = fit < 1 ? 1 : (fit > 2 ? 2 : fit);
  static constexpr int w = (wg_per_cu * WM * WT + 3) / 4;
  static constexpr int cap = (RB >= 2) ? 2 : 4;
  static constexpr int value = w < 1 ? 1 : (w > cap ? cap : w);
};

template <int D, int KVF, int RB, int WM, int WT, int NSTAGE>
__global__ __launch_bounds__(WM * WT * kWave)
__attribute__((amdgpu_waves_per_eu(SplitOccupancy<D, RB, WM, WT, NSTAGE>::value)))
void tree_attn_split_kernel(
    const __bf16* __restrict__ q, const unsigned char* __restrict__ kc,
    const unsigned char* __restrict__ vc, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ prefix_lens,
    const uint64_t* __restrict__ anc_mask, int B, int N, int Hq, int Hkv, int S_max,
    float sm_scale, int split_len, int n_splits, int n_mt, __bf16* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_o, float2* __restrict__ part_ml,
    uint32_t* __restrict__ counters, uint32_t* __restrict__ err_word) {
  static_assert(WT == 1 || WT == 2, "waves split a 64-token tile in one or two 32-token halves");
  static_assert(NSTAGE >= 2 && NSTAGE <= 8, "ring depth");
  constexpr int NW = WM * WT;
  constexpr int EB = (KVF == SPEC_BF16) ? 2 : 1;     // bytes per cached element
  constexpr int CPT = 2 / WT;                        // 32-token chunks per wave per tile
  constexpr int RBYTES = D * EB;                     // bytes per K/V row
  constexpr int UPR = RBYTES / 16;                   // 16-byte units per row
  constexpr int TB = kTile * RBYTES;                 // bytes per tensor per stage
  constexpr int NLOAD = TB / 1024;                   // 1-KB wave DMA instructions per tensor
  constexpr int KPW = NLOAD / NW;                    // per wave per tensor per stage
  constexpr int PT = 2 * KPW;                        // DMA instructions per wave per tile
  constexpr int RPI = 1024 / RBYTES;                 // rows per DMA instruction
  constexpr int MT = WM * RB * 16;                   // packed rows per workgroup
  constexpr int KC = D / 32;
  constexpr int DB = D / 16;
  static_assert(NLOAD % NW == 0, "DMA instructions must split evenly over the waves");
  static_assert((NSTAGE - 2) * PT < 64, "tiles in flight must fit the vmcnt counter");

  // the ring: stage s holds K at smem + 2s*TB and V at smem + (2s+1)*TB
  __shared__ __align__(1024) unsigned char smem[NSTAGE * 2 * TB];
  auto kst = [&](int st) -> unsigned char* { return smem + (2 * st) * TB; };
  auto vst = [&](int st) -> unsigned char* { return smem + (2 * st + 1) * TB; };

  // ---- work item, XCD-aware: workgroups are dispatched round-robin over the
  // 8 XCDs, so the M-tiles of one KV range get ids congruent mod 8 and share
  // that XCD's L2.
  const int id = blockIdx.x;
  const int per = 8 * n_mt;
  const int mt = (id % per) / 8;
  const int unit = (id / per) * 8 + (id % 8);
  if (unit >= B * Hkv * n_splits) return;
  const int split = unit % n_splits;
  const int kvh = (unit / n_splits) % Hkv;
  const int b = unit / (n_splits * Hkv);
  const int g = Hq / Hkv;
  const int M = g * N;

  // The split's token range as far as it can be known before the prefix
  // length arrives: the first ring tiles are fetched for it right away, so the
  // load of prefix_lens[b] does not delay the K/V stream.
  const int t_begin = split * split_len;
  const int t_spec = min(S_max, t_begin + split_len);
  const int ntiles_spec = (t_spec - t_begin + kTile - 1) / kTile;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM;
  const int wt = wave / WM;
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int row0 = mt * MT + wm * RB * 16;

  float scale_log2 = sm_scale * kLog2e;
  float out_scale = 1.0f;
  if constexpr (KVF == SPEC_FP8_E4M3) {
    scale_log2 *= k_scale[kvh];
    out_scale = v_scale[kvh];
  }

  const size_t head_off = ((size_t)(b * Hkv + kvh) * S_max) * RBYTES;
  const unsigned char* kbase = kc + head_off;
  const unsigned char* vbase = vc + head_off;

  // ---- DMA of tile i into stage S: wave w issues instructions w, w+NW, ...;
  // lane l of instruction j fills LDS bytes j*1024 + 16l, i.e. row
  // j*RPI + l/UPR at swizzled unit l%UPR.
  int t_lim = t_spec;                        // rows at or past t_lim repeat row t_lim - 1
  auto issue = [&](int st, int i) {
    const int t0 = t_begin + i * kTile;
#pragma unroll
    for (int qd = 0; qd < KPW; ++qd) {
      const int j = wave + qd * NW;
      const int row = j * RPI + lane / UPR;
      const int u = (lane % UPR) ^ swz<UPR>(row);
      const size_t c = (size_t)min(t0 + row, t_lim - 1);
      const size_t goff = c * RBYTES + u * 16;
      dma16(kbase + goff, kst(st) + j * 1024);
      dma16(vbase + goff, vst(st) + j * 1024);
    }
  };

  // tiles 0 .. NSTAGE-2 go in flight first, so the start-up latency below
  // is spent fetching the whole ring rather than one tile
#pragma unroll
  for (int i = 0; i < NSTAGE - 1; ++i)
    if (i < ntiles_spec) issue(i, i);

  const int P = prefix_lens[b];

  // ---- Q rows of this wave as MFMA B operands (K-slots 32c + 8lg .. +7)
  bf16x8_t qreg[RB][KC];
  uint64_t anc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = row0 + rb * 16 + l16;
    if (row < M) {
      const int i = row / g, hl = row % g;
      const __bf16* qp = q + ((size_t)(b * N + i) * Hq + kvh * g + hl) * D + 8 * lg;
#pragma unroll
      for (int c = 0; c < KC; ++c) qreg[rb][c] = *reinterpret_cast<const bf16x8_t*>(qp + 32 * c);
      anc[rb] = anc_mask[(size_t)b * N + i];
    } else {
#pragma unroll
      for (int c = 0; c < KC; ++c) qreg[rb][c] = bf16x8_t{};
      anc[rb] = 0ull;
    }
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
  wait_vmcnt<0>();   // usually already met by the wait above; a wave with no Q rows has none
  if (P < 0 || P > S_max - N) {
    if (tid == 0 && split == 0 && mt == 0) flag_error(err_word, SPEC_DERR_PREFIX);
    return;
  }
  const int L = P + N;
  if (t_begin >= L) return;
  const int t_end = min(L, t_spec);
  const int ntiles = (t_end - t_begin + kTile - 1) / kTile;
  const bool direct = (L <= split_len);      // this request has a single split
  if (t_end < t_spec) {
    // The tiles fetched ahead loaded cache rows at or past the request's end,
    // which hold arbitrary bits.  Those tokens get zero weight, but 0 * NaN is
    // NaN in the PV product, so their V rows are cleared.
#pragma unroll
    for (int i = 0; i < NSTAGE - 1; ++i) {
      if (i >= ntiles_spec) break;
      const int first = max(t_end - (t_begin + i * kTile), 0);
      for (int off = first * RBYTES + tid * 16; off < TB; off += NW * kWave * 16)
        *reinterpret_cast<uint4*>(vst(i) + off) = make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();
  }
  t_lim = t_end;

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
    if constexpr (KVF == SPEC_BF16) {
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
    if constexpr (KVF == SPEC_BF16) {
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

  auto compute = [&](int st, int i) {
    const unsigned char* ks = kst(st);
    const unsigned char* vs = vst(st);
    const int t0 = t_begin + i * kTile;
    // ---- S^T = K . Q^T for this wave's chunks of the tile
    f32x4_t sacc[RB][CPT][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cp = 0; cp < CPT; ++cp)
#pragma unroll
        for (int G = 0; G < 2; ++G) sacc[rb][cp][G] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cp = 0; cp < CPT; ++cp) {
      const int ch = wt * CPT + cp;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
#pragma unroll
        for (int G = 0; G < 2; ++G) {
          const bf16x8_t a = read_k(ks, 32 * ch + chunk_token(G, l16), c);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            sacc[rb][cp][G] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[rb][c], sacc[rb][cp][G], 0, 0, 0);
        }
      }
    }
    // ---- mask, online softmax (base 2), P in bf16
    const bool plain = (t0 + kTile <= P);   // the whole tile is prefix: nothing masked
    bf16x8_t pb[RB][CPT];
    float alpha[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      // this lane's 8 tokens of chunk cp sit at bits 32*ch + 8*lg .. +7
      uint32_t vis8[CPT];
      if (!plain) {
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
            float s = sacc[rb][cp][G][r] * scale_log2;
            if (!plain) s = ((vis8[cp] >> (4 * G + r)) & 1u) ? s : -INFINITY;
            sacc[rb][cp][G][r] = s;
            mx = fmaxf(mx, s);
          }
      mx = row4_max(mx);
      const float m_new = fmaxf(m_run[rb], mx);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      alpha[rb] = fast_exp2(m_run[rb] - m_use);
      m_run[rb] = m_new;
      float lsum = 0.0f;
#pragma unroll
      for (int cp = 0; cp < CPT; ++cp)
#pragma unroll
        for (int G = 0; G < 2; ++G)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = fast_exp2(sacc[rb][cp][G][r] - m_use);
            lsum += p;
            pb[rb][cp][4 * G + r] = (__bf16)p;
          }
      l_run[rb] = l_run[rb] * alpha[rb] + lsum;
    }
    // rescale O only when some row's running max moved (alpha != 1): after the
    // first tiles that is rare, and skipping a multiply by exactly 1 changes
    // nothing
    bool moved = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) moved |= (alpha[rb] != 1.0f);
    if (__any(moved)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[rb][db] *= alpha[rb];
    }
    // ---- O^T += V^T . P^T
#pragma unroll
    for (int cp = 0; cp < CPT; ++cp) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8_t a = read_v(vs, wt * CPT + cp, db);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          oacc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[rb][cp], oacc[rb][db], 0, 0, 0);
      }
    }
  };

  // ring: wait for tile i (the tiles after it stay in flight), make it visible
  // to all waves, refill the stage tile i-1 used, compute tile i
  int st = 0;
  for (int i = 0; i < ntiles; ++i) {
    const int ahead = min(NSTAGE - 2, ntiles - 1 - i);
    switch (ahead) {
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
    compute(st, i);
    st = (st + 1 == NSTAGE) ? 0 : st + 1;
  }

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
  const size_t unit_rows = (size_t)(b * Hkv + kvh) * n_splits * (size_t)(n_mt * MT);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (wt != 0) break;                              // the token-split partner waves hold no result
    const float l = row4_sum(l_run[rb]);
    const int row = row0 + rb * 16 + l16;
    if (row >= M) continue;
    const int i = row / g, hl = row % g;
    if (direct) {
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
    } else {
      // partials are read by another workgroup (maybe on another XCD) in this
      // same launch: device-scope stores, written through past this XCD's L2
      const size_t pidx = unit_rows + (size_t)split * (n_mt * MT) + row;
      float* po = part_o + pidx * D + 4 * lg;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4_t v = oacc[rb][db] * out_scale;
        store_dev(po + 16 * db, v[0], v[1]);
        store_dev(po + 16 * db + 2, v[2], v[3]);
      }
      if (lg == 0) store_dev(reinterpret_cast<float*>(part_ml + pidx), m_run[rb], l);
    }
  }
  if (direct) return;

  // ---- split merge, fused: the last workgroup of this (request, kv head,
  // M-tile) to finish combines every split's partial, in split order, so the
  // result does not depend on which workgroup that is.  The per-unit counter
  // lives in the workspace; it starts at zero and the merging workgroup
  // resets it, leaving the workspace ready for the next call.
  wait_vmcnt<0>();                                   // this lane's partial stores have completed
  __syncthreads();                                   // ... for every lane; every wave is done with the ring
  uint32_t* s_last = reinterpret_cast<uint32_t*>(smem);
  const int ns = (L + split_len - 1) / split_len;
  uint32_t* cnt = counters + (size_t)(b * Hkv + kvh) * n_mt + mt;
  if (tid == 0) {
    const uint32_t seen = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    *s_last = (seen == (uint32_t)(ns - 1)) ? 1u : 0u;
  }
  __syncthreads();
  if (!*s_last) return;
  // Every load of the merge is independent and each costs a trip to the
  // device coherence point, so they are issued together: a thread owns IPT
  // (row, column quad) items and loads, per round, BATCH items x SG splits of
  // partial O plus each split's (m, l) for the item's row; rounds over further
  // splits rescale the running sums (online softmax over the splits).
  constexpr int NT = NW * kWave;
  constexpr int QPR = D / 4;                         // column quads per row
  static_assert((MT * QPR) % NT == 0, "merge items split evenly over the threads");
  constexpr int IPT = MT * QPR / NT;                 // items per thread
  constexpr int BATCH = IPT < 8 ? IPT : 8;
  constexpr int SG = 16 / BATCH;                     // splits per load round
  static_assert(IPT % BATCH == 0, "merge batches");
  const size_t split_rows = (size_t)n_mt * MT;       // partial rows per split
  const size_t tile_base = unit_rows + (size_t)mt * MT;
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
    for (int s0 = 0; s0 < ns; s0 += SG) {
      float2 ml[SG][BATCH];
      f32x4_t o[SG][BATCH];
#pragma unroll
      for (int j = 0; j < SG; ++j)
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
          const int item = tid + (k0 + k) * NT;
          const int r = item / QPR, qd = item % QPR;
          ml[j][k] = make_float2(-INFINITY, 0.f);
          o[j][k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          if (s0 + j < ns && mt * MT + r < M) {
            const size_t prow = tile_base + (size_t)(s0 + j) * split_rows + r;
            ml[j][k] = load_dev(reinterpret_cast<const float*>(part_ml + prow));
            const float2 lo = load_dev(part_o + prow * D + 4 * qd);
            const float2 hi = load_dev(part_o + prow * D + 4 * qd + 2);
            o[j][k] = f32x4_t{lo.x, lo.y, hi.x, hi.y};
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
      const int item = tid + (k0 + k) * NT;
      const int r = item / QPR, qd = item % QPR;
      const int row = mt * MT + r;
      if (row >= M) continue;
      const int i = row / g, hl = row % g;
      const size_t orow = (size_t)(b * N + i) * Hq + kvh * g + hl;
      const float inv = 1.0f / den[k];
      bf16x4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[k][e] * inv);
      *reinterpret_cast<bf16x4_t*>(out + orow * D + 4 * qd) = v;
      if (lse && qd == 0) lse[orow] = (m[k] + log2f(den[k])) * kLn2;
    }
  }
  if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// fp32 Q/K/V: one wave per (request, node, head), exact fp32 arithmetic on the
// VALU.  Per 64-key chunk: lane = key for the scores (its K row's loads all in
// flight together), then lane = output column for the PV sum, with the
// chunk's 64 V rows loaded at once.
template <int D>
__global__ __launch_bounds__(kWave) void tree_attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kc, const float* __restrict__ vc,
    const int32_t* __restrict__ prefix_lens, const uint64_t* __restrict__ anc_mask, int N,
    int Hq, int Hkv, int S_max, float sm_scale, float* __restrict__ out, float* __restrict__ lse,
    uint32_t* __restrict__ err_word) {
  constexpr int DPL = D / kWave;                 // output columns per lane
  const int h = blockIdx.x % Hq;
  const int i = (blockIdx.x / Hq) % N;
  const int b = blockIdx.x / (Hq * N);
  const int lane = threadIdx.x;
  const int kvh = h / (Hq / Hkv);
  const int P = prefix_lens[b];
  if (P < 0 || P > S_max - N) {
    if (lane == 0 && i == 0 && h == 0) flag_error(err_word, SPEC_DERR_PREFIX);
    return;
  }
  const int L = P + N;
  const uint64_t anc = anc_mask[(size_t)b * N + i];
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
  __shared__ float sp[kWave];

  for (int c0 = 0; c0 < L; c0 += kWave) {
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
    sp[lane] = p;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      float acc = o[k] * alpha;
#pragma unroll
      for (int j = 0; j < kWave; ++j) acc = fmaf(sp[j], vv[j][k], acc);
      o[k] = acc;
    }
    __syncthreads();
  }
  float* op = out + ((size_t)(b * N + i) * Hq + h) * D;
  const float inv = 1.0f / l_run;
#pragma unroll
  for (int k = 0; k < DPL; ++k) op[lane + k * kWave] = o[k] * inv;
  if (lse && lane == 0) lse[(size_t)(b * N + i) * Hq + h] = (m_run + log2f(l_run)) * kLn2;
}

// ------------------------------------------------------------------ planning

struct AttnPlan {
  int rb, wm, wt, nstage, mt_rows, n_mt, M_pad;
  int split_len, n_splits;
  size_t ws_bytes;
};

// Rows per workgroup follow the packed M = g*N.  Small M (<= 32) lets the
// waves also split each tile's tokens (a 3-stage K/V ring, one workgroup per
// CU); larger M splits rows over the waves (a 2-stage ring, two workgroups per
// CU, so two waves share each SIMD).  KV splits are then added until the grid
// has about one workgroup per resident slot (256 CUs), never below 256
// tokens per split so the partial (O, m, l) traffic stays small against the
// split's K/V bytes.  The split plan does not depend on the cached dtype, so
// one workspace size serves every format.
static bool make_plan(int B, int N, int Hq, int Hkv, int D, int S_max, int kv_bytes, AttnPlan* p) {
  (void)kv_bytes;
  if (B < 1 || N < 1 || N > SPEC_MAX_NODES || Hkv < 1 || Hq < Hkv || Hq % Hkv) return false;
  if (D != 64 && D != 128) return false;
  if (S_max < N) return false;
  const int M = (Hq / Hkv) * N;
  if (M <= 32) { p->rb = 1; p->wm = 2; p->wt = 2; p->nstage = 3; }
  else if (M <= 64) { p->rb = 2; p->wm = 2; p->wt = 1; p->nstage = 2; }
  else { p->rb = 2; p->wm = 4; p->wt = 1; p->nstage = 2; }
  const int stage_bytes = 2 * kTile * D * 2;               // bf16 sizing for the split policy
  const long long per_cu = std::max(1, std::min(2, (160 * 1024) / (p->nstage * stage_bytes)));
  long long target_wgs = 256 * per_cu;
#ifdef SPEC_PLAN_HOOK
  SPEC_PLAN_HOOK(p, M, target_wgs);
#endif
  p->mt_rows = p->rb * p->wm * 16;
  p->n_mt = (M + p->mt_rows - 1) / p->mt_rows;
  p->M_pad = p->n_mt * p->mt_rows;
  const long long units = (long long)B * Hkv * p->n_mt;
  const int want = (int)std::max<long long>(1, (target_wgs + units - 1) / units);
  int split_len = (S_max + want - 1) / want;
  split_len = ((split_len + kTile - 1) / kTile) * kTile;
  if (split_len < 256) split_len = 256;
  p->split_len = split_len;
  p->n_splits = (S_max + split_len - 1) / split_len;
  p->ws_bytes = 0;
  if (p->n_splits > 1) {
    const size_t rows = (size_t)B * Hkv * p->n_splits * p->M_pad;
    const size_t counters = (size_t)B * Hkv * p->n_mt;
    p->ws_bytes = rows * (size_t)D * sizeof(float) + rows * sizeof(float2) + counters * sizeof(uint32_t);
  }
  return true;
}

template <int D, int KVF, int RB, int WM, int WT, int NS>
static void launch_split(const AttnPlan& pl, const void* q, const void* k, const void* v,
                         const float* ks, const float* vs, const int32_t* pre, const uint64_t* anc,
                         int B, int N, int Hq, int Hkv, int S_max, float sm_scale, void* out,
                         float* lse, float* po, float2* pml, uint32_t* cnt, uint32_t* err,
                         hipStream_t st) {
  const int units = B * Hkv * pl.n_splits;
  const int units_pad = ((units + 7) / 8) * 8;
  const unsigned grid = (unsigned)units_pad * (unsigned)pl.n_mt;
  hipLaunchKernelGGL((tree_attn_split_kernel<D, KVF, RB, WM, WT, NS>), dim3(grid), dim3(WM * WT * kWave),
                     0, st, static_cast<const __bf16*>(q), static_cast<const unsigned char*>(k),
                     static_cast<const unsigned char*>(v), ks, vs, pre, anc, B, N, Hq, Hkv, S_max,
                     sm_scale, pl.split_len, pl.n_splits, pl.n_mt, static_cast<__bf16*>(out), lse,
                     po, pml, cnt, err);
}

// Whether an instantiation is buildable: the ring fits the LDS, the tiles in
// flight fit the vmcnt counter, the DMA splits evenly over the waves and the
// token-split combine has scratch room.
template <int D, int KVF, int RB, int WM, int WT, int NS>
constexpr bool split_fits() {
  constexpr int TB = kTile * D * ((KVF == SPEC_BF16) ? 2 : 1);
  constexpr int NW = WM * WT;
  constexpr int NLOAD = TB / 1024;
  if (NS * 2 * TB > 160 * 1024) return false;
  if (NLOAD % NW != 0) return false;
  if ((NS - 2) * 2 * (NLOAD / NW) >= 64) return false;
  if (WT == 2 && WM * RB * (D / 16) * 1024 + WM * RB * 512 > NS * 2 * TB) return false;
  return true;
}

// (RB, WM, WT, NSTAGE) instantiations the planner may pick.
#ifndef SPEC_SPLIT_PLANS
#define SPEC_SPLIT_PLANS(X) X(1, 2, 2, 3) X(2, 2, 1, 2) X(2, 4, 1, 2)
#endif

template <int D, int KVF>
static bool dispatch_shape(const AttnPlan& pl, const void* q, const void* k, const void* v,
                           const float* ks, const float* vs, const int32_t* pre,
                           const uint64_t* anc, int B, int N, int Hq, int Hkv, int S_max,
                           float sm_scale, void* out, float* lse, float* po, float2* pml,
                           uint32_t* cnt, uint32_t* err, hipStream_t st) {
#define SPEC_TRY(RB_, WM_, WT_, NS_)                                                               \
  if constexpr (split_fits<D, KVF, RB_, WM_, WT_, NS_>()) {                                        \
    if (pl.rb == RB_ && pl.wm == WM_ && pl.wt == WT_ && pl.nstage == NS_) {                        \
      launch_split<D, KVF, RB_, WM_, WT_, NS_>(pl, q, k, v, ks, vs, pre, anc, B, N, Hq, Hkv, S_max, \
                                               sm_scale, out, lse, po, pml, cnt, err, st);        \
      return true;                                                                                 \
    }                                                                                              \
  }
  SPEC_SPLIT_PLANS(SPEC_TRY)
#undef SPEC_TRY
  return false;
}

}  // namespace spectree

using namespace spectree;

extern "C" size_t spec_tree_attn_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int S_max) {
  AttnPlan pl;
  if (!make_plan(B, N, Hq, Hkv, D, S_max, 2, &pl)) return 0;
  return pl.ws_bytes;
}

static inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

extern "C" spec_status spec_tree_attn_verify(const void* q, spec_dtype q_dtype, const void* k_cache,
                                             const void* v_cache, spec_dtype kv_dtype,
                                             const float* k_scale, const float* v_scale,
                                             const int32_t* prefix_lens, const uint64_t* anc_mask,
                                             int B, int N, int Hq, int Hkv, int D, int S_max,
                                             float sm_scale, void* out, float* lse,
                                             void* workspace, size_t workspace_bytes,
                                             uint32_t* err_word, hipStream_t stream) {
  if (!q || !k_cache || !v_cache || !prefix_lens || !anc_mask || !out) return SPEC_ERR_NULL;
  const bool f32 = (q_dtype == SPEC_F32 && kv_dtype == SPEC_F32);
  const bool bf16 = (q_dtype == SPEC_BF16 && kv_dtype == SPEC_BF16);
  const bool fp8 = (q_dtype == SPEC_BF16 && kv_dtype == SPEC_FP8_E4M3);
  if (!f32 && !bf16 && !fp8) return SPEC_ERR_DTYPE;
  if (fp8 && (!k_scale || !v_scale)) return SPEC_ERR_NULL;
  AttnPlan pl;
  if (!make_plan(B, N, Hq, Hkv, D, S_max, f32 ? 4 : (bf16 ? 2 : 1), &pl)) return SPEC_ERR_SHAPE;
  if ((long long)B * Hkv * pl.n_splits * pl.n_mt >= (1ll << 31)) return SPEC_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return SPEC_ERR_ALIGN;

  if (f32) {
    const unsigned grid = (unsigned)(B * N * Hq);
    if (D == 64)
      hipLaunchKernelGGL(tree_attn_f32_kernel<64>, dim3(grid), dim3(kWave), 0, stream,
                         static_cast<const float*>(q), static_cast<const float*>(k_cache),
                         static_cast<const float*>(v_cache), prefix_lens, anc_mask, N, Hq, Hkv,
                         S_max, sm_scale, static_cast<float*>(out), lse, err_word);
    else
      hipLaunchKernelGGL(tree_attn_f32_kernel<128>, dim3(grid), dim3(kWave), 0, stream,
                         static_cast<const float*>(q), static_cast<const float*>(k_cache),
                         static_cast<const float*>(v_cache), prefix_lens, anc_mask, N, Hq, Hkv,
                         S_max, sm_scale, static_cast<float*>(out), lse, err_word);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
  }

  float* po = nullptr;
  float2* pml = nullptr;
  uint32_t* cnt = nullptr;
  if (pl.ws_bytes) {
    if (!workspace) return SPEC_ERR_WORKSPACE;
    if (workspace_bytes < pl.ws_bytes) return SPEC_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SPEC_ERR_ALIGN;
    const size_t rows = (size_t)B * Hkv * pl.n_splits * pl.M_pad;
    po = static_cast<float*>(workspace);
    pml = reinterpret_cast<float2*>(static_cast<char*>(workspace) + rows * D * sizeof(float));
    cnt = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + rows * D * sizeof(float) +
                                      rows * sizeof(float2));
  }

  bool launched;
  if (bf16) {
    if (D == 64) launched = dispatch_shape<64, SPEC_BF16>(pl, q, k_cache, v_cache, k_scale, v_scale, prefix_lens, anc_mask, B, N, Hq, Hkv, S_max, sm_scale, out, lse, po, pml, cnt, err_word, stream);
    else launched = dispatch_shape<128, SPEC_BF16>(pl, q, k_cache, v_cache, k_scale, v_scale, prefix_lens, anc_mask, B, N, Hq, Hkv, S_max, sm_scale, out, lse, po, pml, cnt, err_word, stream);
  } else {
    if (D == 64) launched = dispatch_shape<64, SPEC_FP8_E4M3>(pl, q, k_cache, v_cache, k_scale, v_scale, prefix_lens, anc_mask, B, N, Hq, Hkv, S_max, sm_scale, out, lse, po, pml, cnt, err_word, stream);
    else launched = dispatch_shape<128, SPEC_FP8_E4M3>(pl, q, k_cache, v_cache, k_scale, v_scale, prefix_lens, anc_mask, B, N, Hq, Hkv, S_max, sm_scale, out, lse, po, pml, cnt, err_word, stream);
  }
  if (!launched) return SPEC_ERR_SHAPE;
  if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;

  return SPEC_OK;
}
