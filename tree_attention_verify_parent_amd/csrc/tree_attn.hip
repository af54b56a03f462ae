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
// each split writes (O, m, l) partials and the merge kernel combines them in
// split order (deterministic).
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
// Waves per SIMD the kernel is built for: as many workgroups as the LDS ring
// leaves room for on a CU (160 KB), so the compiler keeps the register count
// at or below 512 / that many waves instead of spending it on unrolling.
// The register budget caps it too: two row blocks per wave need about 200+
// registers, so at most 2 waves per SIMD there.
template <int D, int KVF, int RB, int WM, int WT, int NSTAGE>
struct SplitOccupancy {
  static constexpr int lds = NSTAGE * 2 * kTile * D * ((KVF == SPEC_BF16) ? 2 : 1);
  static constexpr int wg_per_cu = (160 * 1024) / lds;
  static constexpr int w = (wg_per_cu * WM * WT + 3) / 4;
  static constexpr int cap = (RB >= 2) ? 2 : 4;
  static constexpr int value = w < 1 ? 1 : (w > cap ? cap : w);
};

template <int D, int KVF, int RB, int WM, int WT, int NSTAGE>
__global__ __launch_bounds__(WM * WT * kWave)
__attribute__((amdgpu_waves_per_eu(SplitOccupancy<D, KVF, RB, WM, WT, NSTAGE>::value)))
void tree_attn_split_kernel(
    const __bf16* __restrict__ q, const unsigned char* __restrict__ kc,
    const unsigned char* __restrict__ vc, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ prefix_lens,
    const uint64_t* __restrict__ anc_mask, int B, int N, int Hq, int Hkv, int S_max,
    float sm_scale, int split_len, int n_splits, int n_mt, __bf16* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_o, float2* __restrict__ part_ml,
    uint32_t* __restrict__ err_word) {
  static_assert(WT == 1 || WT == 2, "waves split a 64-token tile in one or two 32-token halves");
  static_assert(NSTAGE == 2 || NSTAGE == 3, "ring depth");
  constexpr int NW = WM * WT;
  constexpr int EB = (KVF == SPEC_BF16) ? 2 : 1;     // bytes per cached element
  constexpr int CPT = 2 / WT;                        // 32-token chunks per wave per tile
  constexpr int RBYTES = D * EB;                     // bytes per K/V row
  constexpr int UPR = RBYTES / 16;                   // 16-byte units per row
  constexpr int TB = kTile * RBYTES;                 // bytes per tensor per stage
  constexpr int NLOAD = TB / 1024;                   // 1-KB wave DMA instructions per tensor
  constexpr int KPW = NLOAD / NW;                    // per wave per tensor per stage
  constexpr int RPI = 1024 / RBYTES;                 // rows per DMA instruction
  constexpr int MT = WM * RB * 16;                   // packed rows per workgroup
  constexpr int KC = D / 32;
  constexpr int DB = D / 16;
  static_assert(NLOAD % NW == 0, "DMA instructions must split evenly over the waves");

  // one LDS object per stage and tensor, so the compiler can tell the stage
  // being read from the stages still being filled (no forced vmcnt(0))
  __shared__ __align__(1024) unsigned char sk0[TB];
  __shared__ __align__(1024) unsigned char sv0[TB];
  __shared__ __align__(1024) unsigned char sk1[TB];
  __shared__ __align__(1024) unsigned char sv1[TB];
  __shared__ __align__(1024) unsigned char sk2[NSTAGE > 2 ? TB : 16];
  __shared__ __align__(1024) unsigned char sv2[NSTAGE > 2 ? TB : 16];
  auto kst = [&](auto S) -> unsigned char* {
    if constexpr (decltype(S)::value == 0) return sk0;
    else if constexpr (decltype(S)::value == 1) return sk1;
    else return sk2;
  };
  auto vst = [&](auto S) -> unsigned char* {
    if constexpr (decltype(S)::value == 0) return sv0;
    else if constexpr (decltype(S)::value == 1) return sv1;
    else return sv2;
  };

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

  const int P = prefix_lens[b];
  if (P < 0 || P > S_max - N) {
    if (threadIdx.x == 0 && split == 0 && mt == 0) flag_error(err_word, SPEC_DERR_PREFIX);
    return;
  }
  const int L = P + N;
  const int t_begin = split * split_len;
  if (t_begin >= L) return;
  const int t_end = min(L, t_begin + split_len);
  const int ntiles = (t_end - t_begin + kTile - 1) / kTile;
  const bool direct = (L <= split_len);      // this request has a single split

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
  auto issue = [&](auto S, int i) {
    const int t0 = t_begin + i * kTile;
#pragma unroll
    for (int qd = 0; qd < KPW; ++qd) {
      const int j = wave + qd * NW;
      const int row = j * RPI + lane / UPR;
      const int u = (lane % UPR) ^ swz<UPR>(row);
      const size_t c = (size_t)min(t0 + row, t_end - 1);     // rows past the split repeat a valid row
      const size_t goff = c * RBYTES + u * 16;
      dma16(kbase + goff, kst(S) + j * 1024);
      dma16(vbase + goff, vst(S) + j * 1024);
    }
  };

  issue(Int<0>{}, 0);
  if constexpr (NSTAGE > 2) {
    if (ntiles > 1) issue(Int<1>{}, 1);
  }

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
  // inside the tile loop that would happen on every tile.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    asm volatile("" ::"v"(anc[rb]));
#pragma unroll
    for (int c = 0; c < KC; ++c) asm volatile("" ::"v"(qreg[rb][c]));
  }

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

  auto compute = [&](auto S, int i) {
    const unsigned char* ks = kst(S);
    const unsigned char* vs = vst(S);
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
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mx = -INFINITY;
#pragma unroll
      for (int cp = 0; cp < CPT; ++cp)
#pragma unroll
        for (int G = 0; G < 2; ++G)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float s = sacc[rb][cp][G][r] * scale_log2;
            if (!plain) {
              const int c = t0 + 32 * (wt * CPT + cp) + 8 * lg + 4 * G + r;
              const bool ok = (c < t_end) && (c < P || ((anc[rb] >> (c - P)) & 1ull));
              s = ok ? s : -INFINITY;
            }
            sacc[rb][cp][G][r] = s;
            mx = fmaxf(mx, s);
          }
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float m_new = fmaxf(m_run[rb], mx);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = exp2f(m_run[rb] - m_use);
      m_run[rb] = m_new;
      float lsum = 0.0f;
#pragma unroll
      for (int cp = 0; cp < CPT; ++cp)
#pragma unroll
        for (int G = 0; G < 2; ++G)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = exp2f(sacc[rb][cp][G][r] - m_use);
            lsum += p;
            pb[rb][cp][4 * G + r] = (__bf16)p;
          }
      l_run[rb] = l_run[rb] * alpha + lsum;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[rb][db] *= alpha;
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

  // one ring step: wait for tile i (later tiles may stay in flight), make it
  // visible to all waves, refill the stage that tile i-1 used, compute tile i
  auto step = [&](auto S, int i) -> bool {
    if (i >= ntiles) return false;
    if constexpr (NSTAGE == 3) {
      if (i + 1 < ntiles) wait_vmcnt<2 * KPW>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    wg_barrier();
    if (i + NSTAGE - 1 < ntiles) issue(Int<(decltype(S)::value + NSTAGE - 1) % NSTAGE>{}, i + NSTAGE - 1);
    compute(S, i);
    return true;
  };
  for (int i = 0;; i += NSTAGE) {
    if (!step(Int<0>{}, i)) break;
    if (!step(Int<1>{}, i + 1)) break;
    if constexpr (NSTAGE > 2) {
      if (!step(Int<2>{}, i + 2)) break;
    }
  }

  // ---- waves that split the tile's tokens combine their states in LDS
  if constexpr (WT == 2) {
    // scratch: row blocks [0, HB) in stage-0 K, [HB, WM*RB) in stage-1 K, (m, l) in stage-0 V
    constexpr int HB = (WM * RB + 1) / 2;
    static_assert(HB * DB * 64 * 16 <= TB && WM * RB * 64 * 8 <= TB, "combine scratch");
    __syncthreads();                                    // all DMA and LDS stage reads are done
    auto oslot = [&](int blk, int db) -> f32x4_t* {
      f32x4_t* base = reinterpret_cast<f32x4_t*>(blk < HB ? sk0 : sk1);
      return base + ((blk < HB ? blk : blk - HB) * DB + db) * 64 + lane;
    };
    float2* sml = reinterpret_cast<float2*>(sv0);       // [WM*RB][64]
    if (wt == 1) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int db = 0; db < DB; ++db) *oslot(wm * RB + rb, db) = oacc[rb][db];
        sml[(wm * RB + rb) * 64 + lane] = make_float2(m_run[rb], l_run[rb]);
      }
    }
    __syncthreads();
    if (wt == 1) return;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float2 o = sml[(wm * RB + rb) * 64 + lane];
      const float m_new = fmaxf(m_run[rb], o.x);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float a0 = exp2f(m_run[rb] - m_use), a1 = exp2f(o.x - m_use);
      m_run[rb] = m_new;
      l_run[rb] = l_run[rb] * a0 + o.y * a1;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[rb][db] = oacc[rb][db] * a0 + *oslot(wm * RB + rb, db) * a1;
    }
  }

  // ---- epilogue: lane holds O^T[16db + 4lg + r][row l16]
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float l = l_run[rb];
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
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
      const size_t pidx = ((size_t)(b * Hkv + kvh) * n_splits + split) * (size_t)(n_mt * MT) + row;
      float* po = part_o + pidx * D + 4 * lg;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4_t v = oacc[rb][db] * out_scale;
        *reinterpret_cast<f32x4_t*>(po + 16 * db) = v;
      }
      if (lg == 0) part_ml[pidx] = make_float2(m_run[rb], l);
    }
  }
}

// Combine the split partials of requests that needed more than one split:
//   m = max_s m_s,  w_s = 2^(m_s - m),  O = sum_s w_s O_s / sum_s w_s l_s.
// One thread per (packed row, 4 output columns).  Splits are taken in index
// order, eight at a time with all their loads issued together (an online
// max over the groups), so the result is deterministic.
template <int D>
__global__ __launch_bounds__(256) void tree_attn_merge_kernel(
    const int32_t* __restrict__ prefix_lens, int B, int N, int Hq, int Hkv, int S_max,
    int split_len, int n_splits, int M_pad, const float* __restrict__ part_o,
    const float2* __restrict__ part_ml, __bf16* __restrict__ out, float* __restrict__ lse) {
  constexpr int QPR = D / 4;                     // column quads per row
  constexpr int RPB = 256 / QPR;                 // rows per workgroup
  constexpr int GRP = 8;
  const int g = Hq / Hkv, M = g * N;
  const int blocks_per_head = (M + RPB - 1) / RPB;
  const int bh = blockIdx.x / blocks_per_head;
  const int b = bh / Hkv, kvh = bh % Hkv;
  const int row = (blockIdx.x % blocks_per_head) * RPB + threadIdx.x / QPR;
  const int qd = threadIdx.x % QPR;
  if (row >= M) return;
  const int P = prefix_lens[b];
  if (P < 0 || P > S_max - N) return;
  const int L = P + N;
  const int ns = (L + split_len - 1) / split_len;
  if (ns <= 1) return;

  const size_t base = (size_t)(b * Hkv + kvh) * n_splits * (size_t)M_pad + row;
  float m = -INFINITY, den = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < ns; s0 += GRP) {
    float2 ml[GRP];
    f32x4_t o[GRP];
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      if (s0 + j < ns) {
        const size_t idx = base + (size_t)(s0 + j) * M_pad;
        ml[j] = part_ml[idx];
        o[j] = *reinterpret_cast<const f32x4_t*>(part_o + idx * D + 4 * qd);
      } else {
        ml[j] = make_float2(-INFINITY, 0.f);
        o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    float mc = m;
#pragma unroll
    for (int j = 0; j < GRP; ++j) mc = fmaxf(mc, ml[j].x);
    const float m_use = (mc == -INFINITY) ? 0.f : mc;
    const float a = exp2f(m - m_use);
    den *= a;
    acc *= a;
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      const float w = exp2f(ml[j].x - m_use);
      den += w * ml[j].y;
      acc += w * o[j];
    }
    m = mc;
  }
  const int i = row / g, hl = row % g;
  const size_t orow = (size_t)(b * N + i) * Hq + kvh * g + hl;
  const float inv = 1.0f / den;
  bf16x4_t v;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = (__bf16)(acc[r] * inv);
  *reinterpret_cast<bf16x4_t*>(out + orow * D + 4 * qd) = v;
  if (lse && qd == 0) lse[orow] = (m + log2f(den)) * kLn2;
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
  size_t lds_bytes;
  size_t ws_bytes;
};

// Rows per workgroup follow the packed M = g*N.  Small M (<= 32) lets two
// waves split each tile's tokens; larger M splits rows over the waves.  KV
// splits are then added until the grid fills the GPU at the occupancy the
// LDS ring allows (256 CUs x workgroups per CU), never below 256 tokens per
// split so the partial (O, m, l) traffic stays small against the split's
// K/V bytes.
static bool make_plan(int B, int N, int Hq, int Hkv, int D, int S_max, int kv_bytes, AttnPlan* p) {
  if (B < 1 || N < 1 || N > SPEC_MAX_NODES || Hkv < 1 || Hq < Hkv || Hq % Hkv) return false;
  if (D != 64 && D != 128) return false;
  if (S_max < N) return false;
  const int M = (Hq / Hkv) * N;
  if (M <= 32) { p->rb = 2; p->wm = 1; p->wt = 2; p->nstage = 3; }
  else if (M <= 64) { p->rb = 2; p->wm = 2; p->wt = 1; p->nstage = 3; }
  else { p->rb = 2; p->wm = 4; p->wt = 1; p->nstage = 2; }
  p->mt_rows = p->rb * p->wm * 16;
  p->n_mt = (M + p->mt_rows - 1) / p->mt_rows;
  p->M_pad = p->n_mt * p->mt_rows;
  p->lds_bytes = (size_t)p->nstage * 2 * kTile * D * kv_bytes;
  const long long per_cu = std::max<long long>(1, (160 * 1024) / (long long)p->lds_bytes);
  const long long units = (long long)B * Hkv * p->n_mt;
  const long long target = 256 * per_cu;
  const int want = (int)std::max<long long>(1, (target + units - 1) / units);
  int split_len = (S_max + want - 1) / want;
  split_len = ((split_len + kTile - 1) / kTile) * kTile;
  if (split_len < 256) split_len = 256;
  p->split_len = split_len;
  p->n_splits = (S_max + split_len - 1) / split_len;
  p->ws_bytes = 0;
  if (p->n_splits > 1) {
    const size_t rows = (size_t)B * Hkv * p->n_splits * p->M_pad;
    p->ws_bytes = rows * (size_t)D * sizeof(float) + rows * sizeof(float2) + 256;
  }
  return true;
}

template <int D, int KVF, int RB, int WM, int WT, int NS>
static void launch_split(const AttnPlan& pl, const void* q, const void* k, const void* v,
                         const float* ks, const float* vs, const int32_t* pre, const uint64_t* anc,
                         int B, int N, int Hq, int Hkv, int S_max, float sm_scale, void* out,
                         float* lse, float* po, float2* pml, uint32_t* err, hipStream_t st) {
  const int units = B * Hkv * pl.n_splits;
  const int units_pad = ((units + 7) / 8) * 8;
  const unsigned grid = (unsigned)units_pad * (unsigned)pl.n_mt;
  hipLaunchKernelGGL((tree_attn_split_kernel<D, KVF, RB, WM, WT, NS>), dim3(grid), dim3(WM * WT * kWave),
                     0, st, static_cast<const __bf16*>(q), static_cast<const unsigned char*>(k),
                     static_cast<const unsigned char*>(v), ks, vs, pre, anc, B, N, Hq, Hkv, S_max,
                     sm_scale, pl.split_len, pl.n_splits, pl.n_mt, static_cast<__bf16*>(out), lse,
                     po, pml, err);
}

template <int D, int KVF>
static void dispatch_shape(const AttnPlan& pl, const void* q, const void* k, const void* v,
                           const float* ks, const float* vs, const int32_t* pre,
                           const uint64_t* anc, int B, int N, int Hq, int Hkv, int S_max,
                           float sm_scale, void* out, float* lse, float* po, float2* pml,
                           uint32_t* err, hipStream_t st) {
#define SPEC_LAUNCH(RB_, WM_, WT_, NS_)                                                          \
  launch_split<D, KVF, RB_, WM_, WT_, NS_>(pl, q, k, v, ks, vs, pre, anc, B, N, Hq, Hkv, S_max,   \
                                           sm_scale, out, lse, po, pml, err, st)
  if (pl.wt == 2) SPEC_LAUNCH(2, 1, 2, 3);
  else if (pl.wm == 2) SPEC_LAUNCH(2, 2, 1, 3);
  else SPEC_LAUNCH(2, 4, 1, 2);
#undef SPEC_LAUNCH
}

}  // namespace spectree

using namespace spectree;

static int kv_elem_bytes(int D, int S_max) {
  (void)D;
  (void)S_max;
  return 2;
}

extern "C" size_t spec_tree_attn_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int S_max) {
  AttnPlan pl;
  // the split plan does not depend on the cached dtype (the LDS ring of the
  // 2-byte format bounds both), so one workspace size serves every format
  if (!make_plan(B, N, Hq, Hkv, D, S_max, kv_elem_bytes(D, S_max), &pl)) return 0;
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
  if (!make_plan(B, N, Hq, Hkv, D, S_max, kv_elem_bytes(D, S_max), &pl)) return SPEC_ERR_SHAPE;
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
  if (pl.ws_bytes) {
    if (!workspace) return SPEC_ERR_WORKSPACE;
    if (workspace_bytes < pl.ws_bytes) return SPEC_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SPEC_ERR_ALIGN;
    const size_t rows = (size_t)B * Hkv * pl.n_splits * pl.M_pad;
    po = static_cast<float*>(workspace);
    pml = reinterpret_cast<float2*>(static_cast<char*>(workspace) + rows * D * sizeof(float));
  }

  if (bf16) {
    if (D == 64) dispatch_shape<64, SPEC_BF16>(pl, q, k_cache, v_cache, k_scale, v_scale, prefix_lens, anc_mask, B, N, Hq, Hkv, S_max, sm_scale, out, lse, po, pml, err_word, stream);
    else dispatch_shape<128, SPEC_BF16>(pl, q, k_cache, v_cache, k_scale, v_scale, prefix_lens, anc_mask, B, N, Hq, Hkv, S_max, sm_scale, out, lse, po, pml, err_word, stream);
  } else {
    if (D == 64) dispatch_shape<64, SPEC_FP8_E4M3>(pl, q, k_cache, v_cache, k_scale, v_scale, prefix_lens, anc_mask, B, N, Hq, Hkv, S_max, sm_scale, out, lse, po, pml, err_word, stream);
    else dispatch_shape<128, SPEC_FP8_E4M3>(pl, q, k_cache, v_cache, k_scale, v_scale, prefix_lens, anc_mask, B, N, Hq, Hkv, S_max, sm_scale, out, lse, po, pml, err_word, stream);
  }
  if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;

  if (pl.n_splits > 1) {
    const int M = (Hq / Hkv) * N;
    const int rpb = 256 / (D / 4);
    const unsigned grid = (unsigned)(B * Hkv) * (unsigned)((M + rpb - 1) / rpb);
    if (D == 64)
      hipLaunchKernelGGL(tree_attn_merge_kernel<64>, dim3(grid), dim3(256), 0, stream, prefix_lens, B,
                         N, Hq, Hkv, S_max, pl.split_len, pl.n_splits, pl.M_pad, po, pml,
                         static_cast<__bf16*>(out), lse);
    else
      hipLaunchKernelGGL(tree_attn_merge_kernel<128>, dim3(grid), dim3(256), 0, stream, prefix_lens, B,
                         N, Hq, Hkv, S_max, pl.split_len, pl.n_splits, pl.M_pad, po, pml,
                         static_cast<__bf16*>(out), lse);
    if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
  }
  return SPEC_OK;
}
