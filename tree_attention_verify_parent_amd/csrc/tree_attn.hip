// Tree-masked split-KV attention for the verify step (gfx950).
//
// Every draft node's query attends to its request's KV-cache prefix plus its
// own ancestors and itself (the custom tree mask of Aurora, section 2, closing
// paragraph; all proposed tokens are verified in one parallel pass, Runtime
// Draft Model Training, "Overview").  The pass is bound by streaming K/V from
// HBM (the same page notes that verification is memory- rather than
// compute-bound), so each K/V byte is read once per (request, kv head): the
// g = Hq/Hkv query heads of a kv head and the N tree nodes are packed into the
// M dimension of small dense MFMA tiles.
//
// Kernel layout (bf16 / e4m3 KV):
//   workgroup = NW waves = one (request b, kv head, M-tile, KV split);
//   wave w owns RB blocks of 16 packed query rows (row = node * g + head);
//   the split's tokens go through LDS 64 at a time: K as [token][d] bf16 and
//   V transposed to [d][token] bf16, both XOR-swizzled against bank conflicts;
//   S^T = K . Q^T and O^T = V^T . P^T run on v_mfma_f32_16x16x32_bf16, so a
//   lane holds one query row of S and of O and the online-softmax statistics
//   of a row live in the 4 lanes {l, l^16, l^32, l^48};
//   the 64-bit ancestor mask of each row is applied in registers, only on
//   tiles that reach the tree rows.
// A request whose tokens fit one split writes its output directly; otherwise
// each split writes (O, m, l) partials and spec_tree_attn_merge combines them
// in split order (deterministic).
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

// 16-byte unit swizzles.  K rows: lanes 0..7 of an A-operand read hit tokens
// {0,1,2,3,8,9,10,11} (+4G); XOR with (t&3)|((t>>3)&1)<<2 spreads them over 8
// distinct units.  V^T rows (d-major): lanes 0..7 read 8 consecutive d rows at
// one unit; XOR with (d&7)^((d>>3)&7) spreads those and keeps the transposed
// writes at most 2-way conflicted.
__device__ __forceinline__ int swz_k(int t) { return (t & 3) | (((t >> 3) & 1) << 2); }
__device__ __forceinline__ int swz_v(int d) { return (d & 7) ^ ((d >> 3) & 7); }

template <int KVF>
struct KvFormat;
template <>
struct KvFormat<SPEC_BF16> {
  static constexpr int kElem = 2;   // bytes per element in HBM
  static constexpr int kEpl = 8;    // elements per 16-byte load
};
template <>
struct KvFormat<SPEC_FP8_E4M3> {
  static constexpr int kElem = 1;
  static constexpr int kEpl = 16;
};

// bf16 bits of element k of a 16-byte load
template <int KVF>
__device__ __forceinline__ uint32_t elem_bits(const uint4& w, int k) {
  constexpr int per_word = (KVF == SPEC_BF16) ? 2 : 4;
  const int wi = k / per_word;
  const uint32_t word = (wi == 0) ? w.x : (wi == 1) ? w.y : (wi == 2) ? w.z : w.w;
  if constexpr (KVF == SPEC_BF16) {
    return (word >> (16 * (k & 1))) & 0xFFFFu;
  } else {
    const uint32_t byte = (word >> (8 * (k & 3))) & 0xFFu;
    return e4m3_to_bf16_bits(byte);
  }
}

template <int D, int KVF, int RB, int NW>
__global__ __launch_bounds__(NW * kWave) void tree_attn_split_kernel(
    const __bf16* __restrict__ q, const unsigned char* __restrict__ kc,
    const unsigned char* __restrict__ vc, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ prefix_lens,
    const uint64_t* __restrict__ anc_mask, int B, int N, int Hq, int Hkv, int S_max,
    float sm_scale, int split_len, int n_splits, int n_mt, __bf16* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_o, float2* __restrict__ part_ml,
    uint32_t* __restrict__ err_word) {
  using F = KvFormat<KVF>;
  constexpr int NT = NW * kWave;
  constexpr int MT = NW * RB * 16;          // packed rows per workgroup
  constexpr int KC = D / 32;                // 32-wide contraction chunks of QK^T
  constexpr int DB = D / 16;                // 16-wide output column blocks
  constexpr int KROW = D * 2;               // bytes per K row in LDS
  constexpr int VROW = kTile * 2;           // bytes per V^T row in LDS
  constexpr int UPR = D / F::kEpl;          // 16-byte loads per cache row
  constexpr int KTASKS = kTile * UPR;       // K: one load each
  constexpr int VTASKS = (kTile / 4) * UPR; // V: 4 tokens x one load-width each
  constexpr int KPT = (KTASKS + NT - 1) / NT;
  constexpr int VPT = (VTASKS + NT - 1) / NT;
  static_assert(KTASKS % NT == 0, "K staging must divide evenly");

  __shared__ __align__(16) unsigned char lds_k[kTile * KROW];
  __shared__ __align__(16) unsigned char lds_v[D * VROW];

  // ---- work item: XCD-aware order.  Workgroups are dispatched round-robin
  // over the 8 XCDs, so the M-tiles of one KV range get ids congruent mod 8 and
  // share that XCD's L2.
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
  const bool direct = (L <= split_len);      // this request has a single split

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int row0 = mt * MT + wave * RB * 16;

  float scale_log2 = sm_scale * kLog2e;
  float out_scale = 1.0f;
  if constexpr (KVF == SPEC_FP8_E4M3) {
    scale_log2 *= k_scale[kvh];
    out_scale = v_scale[kvh];
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

  f32x4_t oacc[RB][DB];
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[rb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const size_t head_off = ((size_t)(b * Hkv + kvh) * S_max) * D;
  const unsigned char* kbase = kc + head_off * F::kElem;
  const unsigned char* vbase = vc + head_off * F::kElem;

  uint4 kbuf[KPT];
  uint4 vbuf[VPT][4];

  auto load_tile = [&](int t0) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int task = tid + j * NT;
      const int tok = task / UPR, u = task % UPR;
      const int c = t0 + tok;
      kbuf[j] = (c < t_end) ? *reinterpret_cast<const uint4*>(kbase + ((size_t)c * D + u * F::kEpl) * F::kElem)
                            : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int task = tid + j * NT;
      const int tg = task / UPR, u = task % UPR;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = t0 + 4 * tg + r;
        vbuf[j][r] = (task < VTASKS && c < t_end)
                         ? *reinterpret_cast<const uint4*>(vbase + ((size_t)c * D + u * F::kEpl) * F::kElem)
                         : uint4{0u, 0u, 0u, 0u};
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int task = tid + j * NT;
      const int tok = task / UPR, u = task % UPR;
      if constexpr (KVF == SPEC_BF16) {
        *reinterpret_cast<uint4*>(lds_k + tok * KROW + ((u ^ swz_k(tok)) << 4)) = kbuf[j];
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint4 w;
          w.x = elem_bits<KVF>(kbuf[j], 8 * h + 0) | (elem_bits<KVF>(kbuf[j], 8 * h + 1) << 16);
          w.y = elem_bits<KVF>(kbuf[j], 8 * h + 2) | (elem_bits<KVF>(kbuf[j], 8 * h + 3) << 16);
          w.z = elem_bits<KVF>(kbuf[j], 8 * h + 4) | (elem_bits<KVF>(kbuf[j], 8 * h + 5) << 16);
          w.w = elem_bits<KVF>(kbuf[j], 8 * h + 6) | (elem_bits<KVF>(kbuf[j], 8 * h + 7) << 16);
          const int ub = 2 * u + h;
          *reinterpret_cast<uint4*>(lds_k + tok * KROW + ((ub ^ swz_k(tok)) << 4)) = w;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int task = tid + j * NT;
      if (task < VTASKS) {
        const int tg = task / UPR, u = task % UPR;
#pragma unroll
        for (int k = 0; k < F::kEpl; ++k) {
          const int d = u * F::kEpl + k;
          uint2 w;
          w.x = elem_bits<KVF>(vbuf[j][0], k) | (elem_bits<KVF>(vbuf[j][1], k) << 16);
          w.y = elem_bits<KVF>(vbuf[j][2], k) | (elem_bits<KVF>(vbuf[j][3], k) << 16);
          const int t = 4 * tg;
          *reinterpret_cast<uint2*>(lds_v + d * VROW + (((t >> 3) ^ swz_v(d)) << 4) + ((t & 7) << 1)) = w;
        }
      }
    }
  };

  load_tile(t_begin);
  for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
    __syncthreads();            // previous tile fully consumed
    store_tile();
    __syncthreads();
    if (t0 + kTile < t_end) load_tile(t0 + kTile);

    // ---- S^T = K . Q^T for the 64 tokens of the tile
    f32x4_t sacc[RB][2][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int ch = 0; ch < 2; ++ch)
#pragma unroll
        for (int G = 0; G < 2; ++G) sacc[rb][ch][G] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
      for (int c = 0; c < KC; ++c) {
#pragma unroll
        for (int G = 0; G < 2; ++G) {
          const int tok = 32 * ch + chunk_token(G, l16);
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
              lds_k + tok * KROW + (((4 * c + lg) ^ swz_k(tok)) << 4));
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            sacc[rb][ch][G] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[rb][c], sacc[rb][ch][G], 0, 0, 0);
        }
      }
    }

    // ---- mask, online softmax (base 2), P in bf16
    const bool plain = (t0 + kTile <= P);   // the whole tile is prefix: nothing masked
    bf16x8_t pb[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mx = -INFINITY;
#pragma unroll
      for (int ch = 0; ch < 2; ++ch)
#pragma unroll
        for (int G = 0; G < 2; ++G)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float s = sacc[rb][ch][G][r] * scale_log2;
            if (!plain) {
              const int c = t0 + 32 * ch + 8 * lg + 4 * G + r;
              const bool ok = (c < t_end) && (c < P || ((anc[rb] >> (c - P)) & 1ull));
              s = ok ? s : -INFINITY;
            }
            sacc[rb][ch][G][r] = s;
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
      for (int ch = 0; ch < 2; ++ch)
#pragma unroll
        for (int G = 0; G < 2; ++G)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = exp2f(sacc[rb][ch][G][r] - m_use);
            lsum += p;
            pb[rb][ch][4 * G + r] = (__bf16)p;
          }
      l_run[rb] = l_run[rb] * alpha + lsum;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[rb][db] *= alpha;
    }

    // ---- O^T += V^T . P^T
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = 16 * db + l16;
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            lds_v + d * VROW + (((4 * ch + lg) ^ swz_v(d)) << 4));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          oacc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[rb][ch], oacc[rb][db], 0, 0, 0);
      }
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
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
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
        f32x4_t v = oacc[rb][db] * out_scale;
        *reinterpret_cast<f32x4_t*>(po + 16 * db) = v;
      }
      if (lg == 0) part_ml[pidx] = make_float2(m_run[rb], l);
    }
  }
}

// Combine the split partials of requests that needed more than one split:
//   m = max_s m_s,  w_s = 2^(m_s - m),  O = sum_s w_s O_s / sum_s w_s l_s.
// One thread per (packed row, 4 output columns); splits in index order.
template <int D>
__global__ __launch_bounds__(256) void tree_attn_merge_kernel(
    const int32_t* __restrict__ prefix_lens, int B, int N, int Hq, int Hkv, int S_max,
    int split_len, int n_splits, int M_pad, const float* __restrict__ part_o,
    const float2* __restrict__ part_ml, __bf16* __restrict__ out, float* __restrict__ lse) {
  constexpr int QPR = D / 4;                     // column quads per row
  constexpr int RPB = 256 / QPR;                 // rows per workgroup
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
  float m = -INFINITY;
  for (int s = 0; s < ns; ++s) m = fmaxf(m, part_ml[base + (size_t)s * M_pad].x);
  float den = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < ns; ++s) {
    const size_t idx = base + (size_t)s * M_pad;
    const float2 ml = part_ml[idx];
    const float w = exp2f(ml.x - m);
    den += w * ml.y;
    const f32x4_t o = *reinterpret_cast<const f32x4_t*>(part_o + idx * D + 4 * qd);
    acc += w * o;
  }
  const int i = row / g, hl = row % g;
  const size_t orow = (size_t)(b * N + i) * Hq + kvh * g + hl;
  const float inv = 1.0f / den;
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  bf16x4_t v;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = (__bf16)(acc[r] * inv);
  *reinterpret_cast<bf16x4_t*>(out + orow * D + 4 * qd) = v;
  if (lse && qd == 0) lse[orow] = (m + log2f(den)) * kLn2;
}

// fp32 Q/K/V: one wave per (request, node, head), exact fp32 arithmetic on the
// VALU.  Lane = key within a 64-key chunk for the scores, lane = output column
// for the PV accumulation.
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

  for (int c0 = 0; c0 < L; c0 += kWave) {
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
    for (int k = 0; k < DPL; ++k) o[k] *= alpha;
    const int cmax = min(kWave, L - c0);
    for (int j = 0; j < cmax; ++j) {
      const float pj = __shfl(p, j, kWave);
      if (pj != 0.f) {
        const float* vr = vb + (size_t)(c0 + j) * D;
#pragma unroll
        for (int k = 0; k < DPL; ++k) o[k] = fmaf(pj, vr[lane + k * kWave], o[k]);
      }
    }
  }
  float* op = out + ((size_t)(b * N + i) * Hq + h) * D;
  const float inv = 1.0f / l_run;
#pragma unroll
  for (int k = 0; k < DPL; ++k) op[lane + k * kWave] = o[k] * inv;
  if (lse && lane == 0) lse[(size_t)(b * N + i) * Hq + h] = (m_run + log2f(l_run)) * kLn2;
}

// ------------------------------------------------------------------ planning

struct AttnPlan {
  int rb, nw, mt_rows, n_mt, M_pad;
  int split_len, n_splits;
  size_t ws_bytes;
};

// Rows per workgroup follow the packed M = g*N; KV splits are added until the
// grid has about two workgroups per CU (256 CUs), but never below 256 tokens
// per split so the partial (O, m, l) traffic stays small against the K/V
// bytes of the split.
static bool make_plan(int B, int N, int Hq, int Hkv, int D, int S_max, AttnPlan* p) {
  if (B < 1 || N < 1 || N > SPEC_MAX_NODES || Hkv < 1 || Hq < Hkv || Hq % Hkv) return false;
  if (D != 64 && D != 128) return false;
  if (S_max < N) return false;
  const int M = (Hq / Hkv) * N;
  if (M <= 32) { p->rb = 1; p->nw = 2; }
  else if (M <= 64) { p->rb = 1; p->nw = 4; }
  else { p->rb = 2; p->nw = 4; }
  p->mt_rows = p->rb * p->nw * 16;
  p->n_mt = (M + p->mt_rows - 1) / p->mt_rows;
  p->M_pad = p->n_mt * p->mt_rows;
  const long long units = (long long)B * Hkv * p->n_mt;
  const long long target = 512;
  const int want = (int)((target + units - 1) / units);
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

template <int D, int KVF, int RB, int NW>
static void launch_split(const AttnPlan& pl, const void* q, const void* k, const void* v,
                         const float* ks, const float* vs, const int32_t* pre, const uint64_t* anc,
                         int B, int N, int Hq, int Hkv, int S_max, float sm_scale, void* out,
                         float* lse, float* po, float2* pml, uint32_t* err, hipStream_t st) {
  const int units = B * Hkv * pl.n_splits;
  const int units_pad = ((units + 7) / 8) * 8;
  const unsigned grid = (unsigned)units_pad * (unsigned)pl.n_mt;
  hipLaunchKernelGGL((tree_attn_split_kernel<D, KVF, RB, NW>), dim3(grid), dim3(NW * kWave), 0, st,
                     static_cast<const __bf16*>(q), static_cast<const unsigned char*>(k),
                     static_cast<const unsigned char*>(v), ks, vs, pre, anc, B, N, Hq, Hkv, S_max,
                     sm_scale, pl.split_len, pl.n_splits, pl.n_mt, static_cast<__bf16*>(out), lse,
                     po, pml, err);
}

template <int D, int KVF>
static void dispatch_rows(const AttnPlan& pl, const void* q, const void* k, const void* v,
                          const float* ks, const float* vs, const int32_t* pre,
                          const uint64_t* anc, int B, int N, int Hq, int Hkv, int S_max,
                          float sm_scale, void* out, float* lse, float* po, float2* pml,
                          uint32_t* err, hipStream_t st) {
  if (pl.rb == 1 && pl.nw == 2)
    launch_split<D, KVF, 1, 2>(pl, q, k, v, ks, vs, pre, anc, B, N, Hq, Hkv, S_max, sm_scale, out, lse, po, pml, err, st);
  else if (pl.rb == 1)
    launch_split<D, KVF, 1, 4>(pl, q, k, v, ks, vs, pre, anc, B, N, Hq, Hkv, S_max, sm_scale, out, lse, po, pml, err, st);
  else
    launch_split<D, KVF, 2, 4>(pl, q, k, v, ks, vs, pre, anc, B, N, Hq, Hkv, S_max, sm_scale, out, lse, po, pml, err, st);
}

}  // namespace spectree

using namespace spectree;

extern "C" size_t spec_tree_attn_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int S_max) {
  AttnPlan pl;
  if (!make_plan(B, N, Hq, Hkv, D, S_max, &pl)) return 0;
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
  if (!make_plan(B, N, Hq, Hkv, D, S_max, &pl)) return SPEC_ERR_SHAPE;
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
    if (D == 64) dispatch_rows<64, SPEC_BF16>(pl, q, k_cache, v_cache, k_scale, v_scale, prefix_lens, anc_mask, B, N, Hq, Hkv, S_max, sm_scale, out, lse, po, pml, err_word, stream);
    else dispatch_rows<128, SPEC_BF16>(pl, q, k_cache, v_cache, k_scale, v_scale, prefix_lens, anc_mask, B, N, Hq, Hkv, S_max, sm_scale, out, lse, po, pml, err_word, stream);
  } else {
    if (D == 64) dispatch_rows<64, SPEC_FP8_E4M3>(pl, q, k_cache, v_cache, k_scale, v_scale, prefix_lens, anc_mask, B, N, Hq, Hkv, S_max, sm_scale, out, lse, po, pml, err_word, stream);
    else dispatch_rows<128, SPEC_FP8_E4M3>(pl, q, k_cache, v_cache, k_scale, v_scale, prefix_lens, anc_mask, B, N, Hq, Hkv, S_max, sm_scale, out, lse, po, pml, err_word, stream);
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
