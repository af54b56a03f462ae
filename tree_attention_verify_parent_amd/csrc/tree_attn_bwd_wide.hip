// Backward pass of the tree-masked attention for more than 128 packed rows
// (gfx950).  The gradients are those of tree_attn_bwd.hip (every accepted and
// rejected branch of a verification trained in one batched forward and
// backward pass under the tree mask: Aurora, section 2, closing paragraph):
//   p[m][c]  = exp(sm_scale * <q[m], K[c]> - lse[m])   on visible keys, else 0
//   D[m]     = <dO[m], O[m]>
//   ds[m][c] = sm_scale * p[m][c] * (<dO[m], V[c]> - D[m])
//   dV[c] = sum_m p[m][c] dO[m],   dK[c] = sum_m ds[m][c] q[m],
//   dq[m] = sum_c ds[m][c] K[c].
// With more rows than one workgroup's LDS holds, dK / dV (sums over rows)
// and dq (sums over keys) cannot both stay on chip in one pass, so there are
// three launches, and no partial sum ever goes to memory:
//   * row statistics: D[m] and lse[m] * log2(e), once per row;
//   * dq, in the forward pass's shape: a workgroup holds 128 packed rows of
//     one (request, kv head) -- their Q and dO as MFMA operands in registers
//     -- and streams the sequence's K / V tiles through a two-stage LDS DMA
//     ring; per 32-key chunk a wave forms S^T = K . Q^T and dP^T = V . dO^T
//     (a lane holds one row), p and ds in registers, and dq^T += K^T . dS^T
//     with K^T from the LDS transpose reads;
//   * dK / dV, in the transposed shape: a workgroup of 8 waves owns a run of
//     128-key tiles; wave w holds K / V of keys 16w .. 16w+15 of the current
//     tile in registers and streams the sequence's packed rows, 64 at a time
//     (Q, dO, their statistics and ancestor masks), through a two-stage LDS
//     DMA ring; dV^T += dO^T . P and dK^T += Q^T . dS accumulate in
//     registers over all rows, and each key's gradients are written once.
// S and dP are formed in both passes; in exchange each pass keeps only its
// own accumulators.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "gfx950.h"
#include "bwd_wide.h"

namespace spectree {
namespace bwd_wide {

constexpr int kTile = 64;                          // keys per K / V tile of the dq pass
constexpr int kWavesDq = 4;
constexpr int kRowsDq = kWavesDq * 2 * 16;         // packed rows per dq workgroup (two 16-row blocks a wave)
constexpr int kWavesKv = 8;
constexpr int kKeysKv = kWavesKv * 16;             // keys per dK / dV tile
constexpr int kRowStep = 64;                       // packed rows per streamed step of the dK / dV pass
// operand fragments a wave keeps in flight: the product loops read them in
// batches, the next batch's reads issued before the current batch's products
constexpr int kFragBatch = 4;
constexpr float kLog2e = 1.4426950408889634f;

// ---- dq pass: K / V tiles, row-major with XOR-swizzled 16-byte units.  The
// natural operand reads of a 16-lane group touch rows {0-3, 8-11, 16-19,
// 24-27} (+4G) at one unit, the transpose reads the same row set at two
// adjacent units; the swizzle gives those rows distinct bank groups.
template <int UPR>
__device__ __forceinline__ int kv_swz(int row) {
  if constexpr (UPR >= 16) return (row & 3) | (((row >> 3) & 3) << 2);
  else return ((row >> 1) & 1) | (((row >> 3) & 3) << 1);
}
// key of MFMA A-row m of key group G within a 32-key chunk: lane group lg
// then holds keys 8lg .. 8lg+7 of the chunk in its S^T accumulators, the
// contraction run its dS^T operand needs
__device__ __forceinline__ int chunk_key(int G, int m) { return 8 * (m >> 2) + 4 * G + (m & 3); }

// ---- dK / dV pass: Q / dO rows, row-major with XOR-swizzled 16-byte units.
// The operand reads take 16 consecutive rows at one unit, the transpose
// reads 4 consecutive (4-aligned) rows at two adjacent units.
template <int UPR>
__device__ __forceinline__ int row_swz(int row) {
  if constexpr (UPR == 16) return ((row & 7) << 1) | ((row >> 3) & 1);
  else return (((row >> 1) & 3) << 1) | ((row >> 3) & 1);
}

// 8 bf16 at logical unit `unit` of row `row` of a swizzled row-major buffer
template <int RBYTES, typename F>
__device__ __forceinline__ bf16x8_t read_unit(const unsigned char* buf, int row, int unit, F swz) {
  return *reinterpret_cast<const bf16x8_t*>(buf + row * RBYTES + ((unit ^ swz(row)) << 4));
}

// Transpose read: lane (l16, lg) receives column 16*cb + l16 of rows
// r0 + 0..3 (first read) and r1 + 0..3 (second); lanes 4k..4k+3 of a 16-lane
// group point at the 16 columns of row k.
template <int RBYTES, typename F>
__device__ __forceinline__ bf16x8_t read_cols(const unsigned char* buf, int r0, int r1, int cb, int l16, F swz) {
  i16x4_t t[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = (h ? r1 : r0) + (l16 >> 2);
    const int u = 2 * cb + ((l16 >> 1) & 1);
    const int off = row * RBYTES + ((u ^ swz(row)) << 4) + ((l16 & 1) << 3);
    t[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(buf + off));
  }
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// Visibility of keys t0 .. t0+63 to a row with ancestor-or-self set anc:
// bit k is set iff key t0+k is a prefix token or a tree node on the row's
// path, and lies before the sequence end L.
__device__ __forceinline__ uint64_t key_visibility(uint64_t anc, int t0, int P, int L) {
  const int pre = P - t0;
  const uint64_t prefix = pre <= 0 ? 0ull : (pre >= 64 ? ~0ull : ((1ull << pre) - 1ull));
  const uint64_t tree = pre >= 64 ? 0ull : (pre >= 0 ? (anc << pre) : (anc >> (-pre)));
  const int lim = L - t0;
  const uint64_t inside = lim >= 64 ? ~0ull : (lim <= 0 ? 0ull : ((1ull << lim) - 1ull));
  return (prefix | tree) & inside;
}

// D[r] = <dO[r], O[r]> and lse[r] * log2(e) for every (request, node, head)
// row r, in the rows' own order: 16 lanes a row.
template <int D>
__global__ __launch_bounds__(256) void bwd_rowstat_kernel(const __bf16* __restrict__ out,
                                                         const __bf16* __restrict__ dout,
                                                         const float* __restrict__ lse, long long rows,
                                                         float* __restrict__ dm, float* __restrict__ lse2) {
  constexpr int EPL = D / 16;                      // elements per lane
  const long long r = ((long long)blockIdx.x * 256 + threadIdx.x) / 16;
  const int part = threadIdx.x & 15;
  float acc = 0.f;
  if (r < rows) {
    const __bf16* o = out + r * D + part * EPL;
    const __bf16* d = dout + r * D + part * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc = fmaf((float)d[e], (float)o[e], acc);
  }
#pragma unroll
  for (int s = 8; s > 0; s >>= 1) acc += __shfl_xor(acc, s, kWave);
  if (part == 0 && r < rows) {
    dm[r] = acc;
    lse2[r] = lse[r] * kLog2e;
  }
}

// dq of 128 packed rows of one (request, kv head) per workgroup.  The M-tiles
// of a sequence get workgroup ids congruent mod 8, so they share an XCD's L2.
template <int D>
__global__ __launch_bounds__(kWavesDq * kWave) __attribute__((amdgpu_waves_per_eu(2)))
void tree_attn_bwd_dq_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ kc,
                             const __bf16* __restrict__ vc, const int32_t* __restrict__ prefix_lens,
                             const uint64_t* __restrict__ anc_mask, const float* __restrict__ lse2,
                             const float* __restrict__ dm, const __bf16* __restrict__ dout, int n_seq, int N,
                             int Hq, int Hkv, int S_max, float sm_scale, int n_mt, __bf16* __restrict__ dq,
                             uint32_t* __restrict__ err_word) {
  constexpr int RBYTES = D * 2, UPR = RBYTES / 16, TB = kTile * RBYTES, NLOAD = TB / 1024;
  constexpr int KPW = NLOAD / kWavesDq, RPI = 1024 / RBYTES, KC = D / 32, DB = D / 16, RB = 2;
  static_assert(NLOAD % kWavesDq == 0, "DMA instructions split evenly over the waves");
  __shared__ __align__(1024) unsigned char ring[2 * 2 * TB];

  const int id = blockIdx.x, per = 8 * n_mt;
  const int mt = (id % per) / 8;
  const int seq = (id / per) * 8 + id % 8;
  if (seq >= n_seq) return;
  const int b = seq / Hkv, kvh = seq % Hkv, g = Hq / Hkv, M = g * N;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int P = prefix_lens[b];
  if (P < 0 || P > S_max - N) {
    if (mt == 0 && kvh == 0 && threadIdx.x == 0) flag_error(err_word, SPEC_DERR_PREFIX);
    return;
  }
  const int L = P + N;
  const int ntiles = (L + kTile - 1) / kTile;
  const unsigned char* kb = reinterpret_cast<const unsigned char*>(kc + (size_t)seq * S_max * D);
  const unsigned char* vb = reinterpret_cast<const unsigned char*>(vc + (size_t)seq * S_max * D);
  auto swz = [](int row) { return kv_swz<UPR>(row); };

  // tile i into stage st: wave w issues instructions w, w+4, ...; lane l of
  // instruction j fills row j*RPI + l/UPR at physical unit l%UPR; keys at or
  // past L repeat key L-1
  auto dma_tile = [&](int i, int st) {
#pragma unroll
    for (int qd = 0; qd < KPW; ++qd) {
      const int j = w + qd * kWavesDq;
      const int row = j * RPI + lane / UPR;
      const int c = min(i * kTile + row, L - 1);
      const size_t goff = (size_t)c * RBYTES + (((lane % UPR) ^ kv_swz<UPR>(row)) << 4);
      dma16(kb + goff, LDS_ADDR(ring) + (2 * st) * TB + j * 1024);
      dma16(vb + goff, LDS_ADDR(ring) + (2 * st + 1) * TB + j * 1024);
    }
  };
  dma_tile(0, 0);

  // this wave's rows: lane (l16, lg) of row block rb holds row row0 + 16rb +
  // l16 at K-slots 32c + 8lg .. +7 of its B operands
  const int row0 = mt * kRowsDq + w * RB * 16;
  bf16x8_t qreg[RB][KC], doreg[RB][KC];
  float l2r[RB], dmr[RB];
  uint64_t anc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = row0 + rb * 16 + l16;
    if (row < M) {
      const int i = row / g;
      const size_t r = (size_t)(b * N + i) * Hq + kvh * g + row % g;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        qreg[rb][c] = *reinterpret_cast<const bf16x8_t*>(q + r * D + 32 * c + 8 * lg);
        doreg[rb][c] = *reinterpret_cast<const bf16x8_t*>(dout + r * D + 32 * c + 8 * lg);
      }
      l2r[rb] = lse2[r];
      dmr[rb] = dm[r];
      anc[rb] = anc_mask[(size_t)b * N + i];
    } else {
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        qreg[rb][c] = bf16x8_t{};
        doreg[rb][c] = bf16x8_t{};
      }
      l2r[rb] = INFINITY;                          // p = 0 on the padding rows
      dmr[rb] = 0.f;
      anc[rb] = 0ull;
    }
  }
  // complete these loads here, once (the compiler's own wait for them,
  // placed in the loop, would drain the ring on every tile)
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    asm volatile("" ::"v"(anc[rb]), "v"(l2r[rb]), "v"(dmr[rb]));
#pragma unroll
    for (int c = 0; c < KC; ++c) asm volatile("" ::"v"(qreg[rb][c]), "v"(doreg[rb][c]));
  }

  f32x4_t dqacc[RB][DB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int db = 0; db < DB; ++db) dqacc[rb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const float scale_log2 = sm_scale * kLog2e;

  auto tile = [&](int i, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value != 0;
    wait_vmcnt<0>();                               // tile i (and, at i = 0, the rows' operands)
    wg_barrier();                                  // ... visible to all; tile i-1's stage free
    const int st = i & 1;
    if (i + 1 < ntiles) dma_tile(i + 1, st ^ 1);
    const unsigned char* ks = ring + (2 * st) * TB;
    const unsigned char* vs = ring + (2 * st + 1) * TB;
    uint64_t vis[RB];
    if constexpr (MASKED)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) vis[rb] = key_visibility(anc[rb], i * kTile, P, L);
#pragma unroll
    for (int cp = 0; cp < 2; ++cp) {
      // S^T and dP^T of the chunk's 32 keys: lane holds keys 32cp + 8lg + 4G + r
      f32x4_t sacc[RB][2], pacc[RB][2];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int G = 0; G < 2; ++G) {
          sacc[rb][G] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          pacc[rb][G] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      {
        constexpr int NF = KC * 2 * 2, PB = kFragBatch;
        bf16x8_t fr[NF];
        auto rd = [&](int x) {
          const int c = x / 4, G = (x / 2) % 2;
          fr[x] = read_unit<RBYTES>((x & 1) ? vs : ks, 32 * cp + chunk_key(G, l16), 4 * c + lg, swz);
        };
        auto mm = [&](int x) {
          const int c = x / 4, G = (x / 2) % 2;
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            if (x & 1) pacc[rb][G] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[x], doreg[rb][c], pacc[rb][G], 0, 0, 0);
            else sacc[rb][G] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[x], qreg[rb][c], sacc[rb][G], 0, 0, 0);
          }
        };
        batched_products<NF, PB>(rd, mm);
      }
      // p and ds in registers, ds in bf16 as the dq product's B operand
      bf16x8_t dsb[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        uint32_t v8 = 0xFFu;
        if constexpr (MASKED) v8 = (uint32_t)(vis[rb] >> (32 * cp + 8 * lg)) & 0xFFu;
#pragma unroll
        for (int G = 0; G < 2; ++G)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float p = fast_exp2(__builtin_fmaf(sacc[rb][G][r], scale_log2, -l2r[rb]));
            if constexpr (MASKED) p = ((v8 >> (4 * G + r)) & 1u) ? p : 0.f;
            dsb[rb][4 * G + r] = (__bf16)(p * (pacc[rb][G][r] - dmr[rb]) * sm_scale);
          }
      }
      // dq^T += K^T . dS^T over the chunk's keys
      {
        constexpr int PB = kFragBatch < DB ? kFragBatch : DB;
        bf16x8_t fr[DB];
        auto rd = [&](int db) {
          i16x4_t t[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int row = 32 * cp + 8 * lg + 4 * h + (l16 >> 2);
            const int u = 2 * db + ((l16 >> 1) & 1);
            const int off = row * RBYTES + ((u ^ kv_swz<UPR>(row)) << 4) + ((l16 & 1) << 3);
            t[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(ks + off));
          }
          fr[db] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7));
        };
        auto mm = [&](int db) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            dqacc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[db], dsb[rb], dqacc[rb][db], 0, 0, 0);
        };
        batched_products<DB, PB>(rd, mm);
      }
    }
  };
  // tiles wholly inside the prefix need no mask
  const int n_plain = min(ntiles, P / kTile);
  for (int i = 0; i < n_plain; ++i) tile(i, std::integral_constant<int, 0>{});
  for (int i = n_plain; i < ntiles; ++i) tile(i, std::integral_constant<int, 1>{});

  // dq: lane holds dq^T[16db + 4lg + r][row l16]
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = row0 + rb * 16 + l16;
    if (row >= M) continue;
    __bf16* op = dq + ((size_t)(b * N + row / g) * Hq + kvh * g + row % g) * D + 4 * lg;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      bf16x4_t v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (__bf16)dqacc[rb][db][r];
      *reinterpret_cast<bf16x4_t*>(op + 16 * db) = v;
    }
  }
}

// dK / dV of a run of 128-key tiles of one (request, kv head) per workgroup.
// The runs of a sequence get workgroup ids congruent mod 8 (one XCD's L2
// holds the rows they all stream).
template <int D>
__global__ __launch_bounds__(kWavesKv * kWave) __attribute__((amdgpu_waves_per_eu(2)))
void tree_attn_bwd_dkdv_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ kc,
                               const __bf16* __restrict__ vc, const int32_t* __restrict__ prefix_lens,
                               const uint64_t* __restrict__ anc_mask, const float* __restrict__ lse2,
                               const float* __restrict__ dm, const __bf16* __restrict__ dout, int n_seq, int N,
                               int Hq, int Hkv, int S_max, float sm_scale, int n_runs, int run_len,
                               __bf16* __restrict__ dk, __bf16* __restrict__ dv) {
  constexpr int RBYTES = D * 2, UPR = RBYTES / 16, RPI = 1024 / RBYTES, KC = D / 32, DB = D / 16;
  constexpr int MB = kRowStep / 16, KS = kRowStep / 32;
  constexpr int QB = kRowStep * RBYTES;            // bytes of Q (or dO) rows per stage
  constexpr int QI = QB / 1024;                    // 1-KB DMA instructions per tensor per stage
  // a stage: Q and dO rows, then the rows' lse2 and D (4 B a row) and masks
  // (8 B), by NSD wave-wide dword DMAs (64 dwords each)
  constexpr int SB = 2 * QB + 16 * kRowStep;
  constexpr int NSD = 4 * kRowStep / kWave;
  static_assert(QI % kWavesKv == 0 || kWavesKv % QI == 0, "row DMAs split over the waves");
  static_assert(kRowStep % kWave == 0 && NSD <= kWavesKv, "a step's statistics: one dword DMA per wave");
  __shared__ __align__(1024) unsigned char ring[2 * SB];

  const int id = blockIdx.x, per = 8 * n_runs;
  const int run = (id % per) / 8;
  const int seq = (id / per) * 8 + id % 8;
  if (seq >= n_seq) return;
  const int b = seq / Hkv, kvh = seq % Hkv, g = Hq / Hkv, M = g * N;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int P = prefix_lens[b];
  if (P < 0 || P > S_max - N) return;              // flagged by the dq pass
  const int L = P + N;
  const int T = (L + kKeysKv - 1) / kKeysKv;
  const int kt0 = run * run_len;
  const int ntk = min(run_len, T - kt0);
  if (ntk <= 0) return;
  const int n_rs = (M + kRowStep - 1) / kRowStep;
  const int F = ntk * n_rs;                        // steps: (key tile, row step) pairs, row step fastest
  auto swz = [](int row) { return row_swz<UPR>(row); };

  // packed row m's (request, node, head) row index, rows past M repeating row M-1
  auto row_of = [&](int m) -> size_t {
    const int mm = min(m, M - 1);
    return (size_t)(b * N + mm / g) * Hq + kvh * g + mm % g;
  };
  // row step rs into stage st: Q and dO rows (instruction j lands row j*RPI +
  // l/UPR at physical unit l%UPR), then one dword a row of lse2 (wave 0) and
  // D (wave 1), and the rows' masks (waves 2, 3)
  auto dma_rows = [&](int rs, int st) {
    const uint32_t base = LDS_ADDR(ring) + st * SB;
    for (int j = w; j < QI; j += kWavesKv) {
      const int r = j * RPI + lane / UPR;
      const size_t e = row_of(rs * kRowStep + r) * D + 8 * ((lane % UPR) ^ row_swz<UPR>(r));
      dma16(q + e, base + j * 1024);
      dma16(dout + e, base + QB + j * 1024);
    }
    // dword DMA w of the statistics: lse2 rows, D rows, then the masks
    constexpr int NS1 = kRowStep / kWave;          // DMAs per 4-byte statistic
    if (w < NS1) {
      dma4(lse2 + row_of(rs * kRowStep + kWave * w + lane), base + 2 * QB + 256 * w);
    } else if (w < 2 * NS1) {
      dma4(dm + row_of(rs * kRowStep + kWave * (w - NS1) + lane), base + 2 * QB + 256 * w);
    } else if (w < NSD) {
      const int idx = kWave * (w - 2 * NS1) + lane;   // dword idx of the step's masks
      const int mm = min(rs * kRowStep + (idx >> 1), M - 1);
      dma4(reinterpret_cast<const uint32_t*>(anc_mask) + 2 * ((size_t)b * N + mm / g) + (idx & 1),
           base + 2 * QB + 256 * w);
    }
  };
  // K / V of this wave's 16 keys of tile kt, as the B operands of S = Q . K^T
  // and dP = dO . V^T: lane (l16, lg) holds key 16w + l16 at K-slots 32c +
  // 8lg .. +7 (keys at or past L repeat key L-1)
  const __bf16* kseq = kc + (size_t)seq * S_max * D;
  const __bf16* vseq = vc + (size_t)seq * S_max * D;
  auto load_kv = [&](int kt, bf16x8_t* kd, bf16x8_t* vd) {
    const int key = min(kt * kKeysKv + 16 * w + l16, L - 1);
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      kd[c] = *reinterpret_cast<const bf16x8_t*>(kseq + (size_t)key * D + 32 * c + 8 * lg);
      vd[c] = *reinterpret_cast<const bf16x8_t*>(vseq + (size_t)key * D + 32 * c + 8 * lg);
    }
  };
  // the gradients leave through buffer stores bounded to L rows: keys at or
  // past L are dropped without a branch
  const __amdgpu_buffer_rsrc_t rdk = dev_rsrc(dk + (size_t)seq * S_max * D, L * RBYTES);
  const __amdgpu_buffer_rsrc_t rdv = dev_rsrc(dv + (size_t)seq * S_max * D, L * RBYTES);

  bf16x8_t kf[KC], vf[KC];
  load_kv(kt0, kf, vf);
  dma_rows(0, 0);
  f32x4_t dkacc[DB], dvacc[DB];
  const float scale_log2 = sm_scale * kLog2e;

  auto step = [&](int f, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value != 0;
    const int rs = f % n_rs;
    const int kt = kt0 + f / n_rs;
    const unsigned char* sq = ring + (f & 1) * SB;
    const unsigned char* sdo = sq + QB;
    const float* s_l2 = reinterpret_cast<const float*>(sq + 2 * QB);
    const float* s_dm = s_l2 + kRowStep;
    const uint64_t* s_anc = reinterpret_cast<const uint64_t*>(s_dm + kRowStep);
    // ---- S = Q . K^T and dP = dO . V^T for the wave's 16 keys (lane = key)
    f32x4_t sacc[MB], pacc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      sacc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      pacc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    {
      // fragments (c, mb, Q or dO) in batches of PB, the next batch's reads
      // issued before the current batch's products
      constexpr int NF = KC * MB * 2, PB = kFragBatch;
      bf16x8_t fr[NF];
      auto rd = [&](int x) {
        const int c = x / (MB * 2), mb = (x / 2) % MB;
        fr[x] = read_unit<RBYTES>((x & 1) ? sdo : sq, 16 * mb + l16, 4 * c + lg, swz);
      };
      auto mm = [&](int x) {
        const int c = x / (MB * 2), mb = (x / 2) % MB;
        if (x & 1) pacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[x], vf[c], pacc[mb], 0, 0, 0);
        else sacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[x], kf[c], sacc[mb], 0, 0, 0);
      };
      batched_products<NF, PB>(rd, mm);
    }
    // ---- p and ds of rows 16mb + 4lg + r at this lane's key; K-slot t of
    // k-step s holds row 32s + 4lg + t (t < 4) or 32s + 16 + 4lg + t - 4
    const int key = kt * kKeysKv + 16 * w + l16;
    const int j = key - P;                         // tree node of the key, if >= 0
    bf16x8_t pb[KS], dsb[KS];
    f32x4_t l2s[MB], dms[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      l2s[mb] = *reinterpret_cast<const f32x4_t*>(s_l2 + 16 * mb + 4 * lg);
      dms[mb] = *reinterpret_cast<const f32x4_t*>(s_dm + 16 * mb + 4 * lg);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const f32x4_t l2 = l2s[mb];
      const f32x4_t dmv = dms[mb];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float p = fast_exp2(__builtin_fmaf(sacc[mb][r], scale_log2, -l2[r]));
        if constexpr (MASKED) {
          const int rl = 16 * mb + 4 * lg + r;
          const bool vis = (rs * kRowStep + rl < M) && (key < L) && (j < 0 || ((s_anc[rl] >> j) & 1ull));
          p = vis ? p : 0.f;
        }
        pb[mb >> 1][4 * (mb & 1) + r] = (__bf16)p;
        dsb[mb >> 1][4 * (mb & 1) + r] = (__bf16)(p * (pacc[mb][r] - dmv[r]) * sm_scale);
      }
    }
    // ---- dV^T += dO^T . P and dK^T += Q^T . dS (rows d, column = key)
    {
      // fragments (s, db, dO or Q), two transpose reads each, batched as above
      constexpr int NF = KS * DB * 2, PB = kFragBatch;
      bf16x8_t fr[NF];
      auto rd = [&](int x) {
        const int sx = x / (DB * 2), db = (x / 2) % DB;
        fr[x] = read_cols<RBYTES>((x & 1) ? sq : sdo, 32 * sx + 4 * lg, 32 * sx + 16 + 4 * lg, db, l16, swz);
      };
      auto mm = [&](int x) {
        const int sx = x / (DB * 2), db = (x / 2) % DB;
        if (x & 1) dkacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[x], dsb[sx], dkacc[db], 0, 0, 0);
        else dvacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[x], pb[sx], dvacc[db], 0, 0, 0);
      };
      batched_products<NF, PB>(rd, mm);
    }
  };

  for (int f = 0; f < F; ++f) {
    const int rs = f % n_rs;
    const int kt = kt0 + f / n_rs;
    wait_vmcnt<0>();                               // this step's rows (and the key tile's K / V)
    wg_barrier();                                  // ... visible to all; the other stage is free
    if (rs == 0) {
      // a new key tile: its K / V (the first tile's came with the prologue).
      // Loaded here rather than prefetched a step ahead: the 32 registers a
      // prefetch holds cost the loop more than this wait, once a tile.
      if (f > 0) {
        load_kv(kt, kf, vf);
        wait_vmcnt<0>();
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dkacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        dvacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    if (f + 1 < F) dma_rows((f + 1) % n_rs, (f + 1) & 1);
    const bool plain = (kt + 1) * kKeysKv <= P && (rs + 1) * kRowStep <= M;
    if (plain) step(f, std::integral_constant<int, 0>{});
    else step(f, std::integral_constant<int, 1>{});
    if (rs == n_rs - 1) {
      // lane holds dK^T / dV^T[16db + 4lg + r][key 16w + l16]
      const int key = kt * kKeysKv + 16 * w + l16;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        bf16x4_t a, v;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          a[r] = (__bf16)dkacc[db][r];
          v[r] = (__bf16)dvacc[db][r];
        }
        const int off = (key * D + 16 * db + 4 * lg) * 2;
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, a), rdk, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), rdv, off, 0, 0);
      }
    }
  }
  wait_vmcnt<0>();
}

}  // namespace bwd_wide

// Workspace of the wide backward: D and lse * log2(e) per (request, node,
// head) row, 256-byte aligned each.
size_t bwd_wide_workspace_bytes(int B, int N, int Hq) {
  const size_t one = ((size_t)B * N * Hq * sizeof(float) + 255) & ~(size_t)255;
  return 2 * one;
}

spec_status bwd_wide_launch(const void* q, const void* k, const void* v, const int32_t* prefix_lens,
                            const uint64_t* anc_mask, const void* out, const float* lse, const void* dout, int B,
                            int N, int Hq, int Hkv, int D, int S_max, float sm_scale, void* dq, void* dk, void* dv,
                            void* workspace, uint32_t* err_word, hipStream_t stream) {
  using namespace bwd_wide;
  const long long rows = (long long)B * N * Hq;
  const size_t one = ((size_t)rows * sizeof(float) + 255) & ~(size_t)255;
  float* dm = static_cast<float*>(workspace);
  float* lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + one);
  const int n_seq = B * Hkv;
  const int seq_pad = (n_seq + 7) / 8 * 8;
  const int M = (Hq / Hkv) * N;
  const int n_mt = (M + kRowsDq - 1) / kRowsDq;
  // dK / dV runs: about one workgroup per CU (8 waves each) in all
  const int t_max = (S_max + kKeysKv - 1) / kKeysKv;
  const int want = std::max(1, (256 + n_seq - 1) / n_seq);
  const int run_len = (t_max + want - 1) / want;
  const int n_runs = (t_max + run_len - 1) / run_len;
  const auto* qb = static_cast<const __bf16*>(q);
  const auto* kb = static_cast<const __bf16*>(k);
  const auto* vb = static_cast<const __bf16*>(v);
  const auto* ob = static_cast<const __bf16*>(out);
  const auto* db = static_cast<const __bf16*>(dout);
#define SPEC_WIDE(D_)                                                                                          \
  hipLaunchKernelGGL(bwd_rowstat_kernel<D_>, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, ob, db, lse, \
                     rows, dm, lse2);                                                                          \
  hipLaunchKernelGGL(tree_attn_bwd_dq_kernel<D_>, dim3((unsigned)(seq_pad * n_mt)), dim3(kWavesDq * kWave), 0,  \
                     stream, qb, kb, vb, prefix_lens, anc_mask, lse2, dm, db, n_seq, N, Hq, Hkv, S_max, sm_scale,  \
                     n_mt, static_cast<__bf16*>(dq), err_word);                                                \
  hipLaunchKernelGGL(tree_attn_bwd_dkdv_kernel<D_>, dim3((unsigned)(seq_pad * n_runs)), dim3(kWavesKv * kWave), 0, \
                     stream, qb, kb, vb, prefix_lens, anc_mask, lse2, dm, db, n_seq, N, Hq, Hkv, S_max, sm_scale,  \
                     n_runs, run_len, static_cast<__bf16*>(dk), static_cast<__bf16*>(dv))
  if (D == 128) {
    SPEC_WIDE(128);
  } else {
    SPEC_WIDE(64);
  }
#undef SPEC_WIDE
  return launch_status();
}

}  // namespace spectree
