// Backward pass of the tree-masked attention (gfx950).
//
// The draft model is trained on every accepted and rejected branch of a
// verification in one batched forward and backward pass under the tree mask
// (Aurora, section 2, closing paragraph on tree attention).  This is that
// backward pass for the attention of the verify step: for request b, kv head
// kvh, the g query heads x N nodes packed into M rows (row m = node * g +
// head, as in the forward pass), keys c < L = P + N, and the forward pass's
// output O and log-sum-exp lse:
//   p[m][c]  = exp(sm_scale * <q[m], K[c]> - lse[m])   on visible keys, else 0
//   D[m]     = <dO[m], O[m]>
//   ds[m][c] = sm_scale * p[m][c] * (<dO[m], V[c]> - D[m])
//   dV[c] = sum_m p[m][c] dO[m],   dK[c] = sum_m ds[m][c] q[m],
//   dq[m] = sum_c ds[m][c] K[c].
//
// bf16 kernel: workgroup = one (request, kv head, run of 64-key tiles), four
// waves.  K/V tiles stream HBM -> LDS by direct DMA into a ring, as in the
// forward pass; Q and dO of all M rows sit in LDS (and, for M <= 32, in
// registers) for the whole run.  Wave w
// owns keys 16w .. 16w+15 of a tile:
//   S  = Q . K^T,  dP = dO . V^T                     (M x 16, lane = key)
//   dV^T = dO^T . P,  dK^T = Q^T . dS                (D x 16, lane = key)
// so dK and dV of a key are finished inside one wave; they go to HBM as
// whole rows, turned around through the wave's own rows of the V stage.  dS^T goes through LDS, and wave w then
// accumulates dq^T = K^T . dS^T for its quarter of the D columns over the
// whole run.  A run that covers its whole sequence writes dq directly;
// otherwise each run writes an fp32 partial and the last run of the sequence
// to finish adds them up in run order (deterministic), in the same launch.
// MFMA v_mfma_f32_16x16x32_bf16 throughout; operands that contract over
// keys or rows come from the LDS transpose reads (ds_read_b64_tr_b16).
//
// More than 128 packed rows do not fit one workgroup's LDS: that case runs
// as separate dq and dK / dV passes (tree_attn_bwd_wide.hip).
//
// fp32 path: one plain launch of 4-wave workgroups (dq per row, dK / dV per key), exact fp32
// arithmetic, for small problems.
#include <cmath>

#include "gfx950.h"
#include "bwd_wide.h"

namespace spectree {

namespace bwd {

constexpr int kTile = 64;                          // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr float kLog2e = 1.4426950408889634f;

// XOR swizzle of the 16-byte units of an LDS row of UPR units.  Two access
// shapes touch these rows: 16 consecutive rows at one unit (the operand
// reads of Q, dO, K, V rows), and 4 consecutive rows (4-aligned) at two
// adjacent units (the transpose reads).  For 256-byte rows the swizzle is a
// bijection of the 16 units over any 16 consecutive rows, and keeps the two
// adjacent units of the 4 rows on 8 distinct units; 128-byte rows do the
// same on the (row parity, unit) pairs.
template <int UPR>
__device__ __forceinline__ int swz(int row) {
  if constexpr (UPR == 16) return ((row & 7) << 1) | ((row >> 3) & 1);
  else return (((row >> 1) & 3) << 1) | ((row >> 3) & 1);
}

// XOR swizzle of the 16-byte units of the 16-row staging area that turns
// dK / dV from the MFMA C layout into whole rows: the writes put 16 rows x 2
// halves of one unit pair on distinct banks, the row reads touch one row.
template <int UPR>
__device__ __forceinline__ int sws(int row) {
  if constexpr (UPR == 16) return row & 15;
  else return (row >> 1) & 7;
}

// s_waitcnt lgkmcnt(0) with vmcnt / expcnt unconstrained: LDS writes done,
// the K/V DMAs still in flight.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4)); }

// s_waitcnt vmcnt(A * PT + S * SPT) for wave-uniform A in [0, AMAX], S in [0, SMAX]
template <int PT, int SPT, int A, int S>
__device__ __forceinline__ void wait_stores(int s) {
  if constexpr (S >= 0) {
    if (s == S) {
      wait_vmcnt<A * PT + S * SPT>();
      return;
    }
    wait_stores<PT, SPT, A, S - 1>(s);
  }
}
template <int PT, int SPT, int A, int SMAX>
__device__ __forceinline__ void wait_ring(int a, int s) {
  if constexpr (A >= 0) {
    if (a == A) {
      wait_stores<PT, SPT, A, SMAX>(s);
      return;
    }
    wait_ring<PT, SPT, A - 1, SMAX>(a, s);
  }
}

template <int D, int MP, int NSTAGE>
struct Shape {
  static constexpr int RBYTES = D * 2;             // bytes per K/V/Q row
  static constexpr int UPR = RBYTES / 16;
  static constexpr int TB = kTile * RBYTES;        // bytes per tensor per stage
  static constexpr int NLOAD = TB / 1024;          // 1-KB wave DMA instructions per tensor
  static constexpr int KPW = NLOAD / kWaves;
  static constexpr int PT = 2 * KPW;               // DMA instructions per wave per tile
  static constexpr int RPI = 1024 / RBYTES;        // rows per DMA instruction
  static constexpr int KC = D / 32;                // MFMA k-steps over D
  static constexpr int DB = D / 16;                // 16-column blocks of D
  static constexpr int MB = MP / 16;               // 16-row blocks of M
  static constexpr int KS = MP / 32;               // MFMA k-steps over M
  static constexpr int DN = DB / kWaves;           // dq column blocks per wave
  static constexpr int SPT = 2 * (16 * RBYTES / 1024);   // dK + dV row stores per wave per tile
  static constexpr int DS_STRIDE = MP * 2 + 8;     // bytes per dS^T row (padded)
  static constexpr int LDS = NSTAGE * 2 * TB + 2 * MP * RBYTES + kTile * DS_STRIDE + MP * 16 + 16;
  // every wave's DMAs and stores in flight fit the 6-bit vmcnt counter
  static constexpr bool fits = (LDS <= 160 * 1024) && ((NSTAGE - 2) * PT + (NSTAGE - 1) * SPT < 64) &&
                               (NLOAD % kWaves == 0) && (MP % 32 == 0) && (MP <= 128);
};

template <int D, int MP, int NSTAGE>
__global__ __launch_bounds__(kThreads) void tree_attn_bwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kc, const __bf16* __restrict__ vc,
    const int32_t* __restrict__ prefix_lens, const uint64_t* __restrict__ anc_mask,
    const __bf16* __restrict__ out, const float* __restrict__ lse, const __bf16* __restrict__ dout,
    int B, int N, int Hq, int Hkv, int S_max, float sm_scale, int split_len, int n_splits,
    __bf16* __restrict__ dq, __bf16* __restrict__ dk, __bf16* __restrict__ dv,
    float* __restrict__ part, uint32_t* __restrict__ counters, uint32_t* __restrict__ err_word) {
  using SH = Shape<D, MP, NSTAGE>;
  static_assert(SH::fits, "shape does not fit the LDS or the vmcnt counter");
  constexpr int RBYTES = SH::RBYTES, UPR = SH::UPR, TB = SH::TB, KPW = SH::KPW, PT = SH::PT;
  constexpr int RPI = SH::RPI, KC = SH::KC, DB = SH::DB, MB = SH::MB, KS = SH::KS, DN = SH::DN;
  constexpr int DS_STRIDE = SH::DS_STRIDE;
  constexpr int SPT = SH::SPT;                     // dK / dV row stores per wave per tile

  __shared__ __align__(1024) unsigned char ring[NSTAGE * 2 * TB];
  __shared__ __align__(16) unsigned char sq[MP * RBYTES];
  __shared__ __align__(16) unsigned char sdo[MP * RBYTES];
  __shared__ __align__(16) unsigned char sds[kTile * DS_STRIDE];
  __shared__ __align__(16) float s_lse2[MP];
  __shared__ __align__(16) float s_dm[MP];
  __shared__ uint64_t s_anc[MP];
  __shared__ uint32_t s_last;
  __shared__ int s_hist[kWave];
  __shared__ int s_pick[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- The run this workgroup takes.  The runs of every (request, kv head)
  // sequence are ordered longest first: all full runs (split_len tiles), in
  // sequence order, then the partial last runs by decreasing length (ties in
  // sequence order).  Workgroups are dispatched in id order as CUs free up,
  // so on ragged batches this approximates a longest-first schedule.  Wave 0
  // derives the order from the prefix lengths; a length out of range gives
  // its request no runs (flagged once, by workgroup 0).
  if (w == 0) {
    const int R = split_len;
    s_hist[lane] = 0;
    __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0)
    auto tiles_of = [&](int bb) -> int {
      const int pb = prefix_lens[bb];
      if (pb < 0 || pb > S_max - N) {
        if (blockIdx.x == 0) flag_error(err_word, SPEC_DERR_PREFIX);
        return 0;
      }
      return (pb + N + kTile - 1) / kTile;
    };
    int F = 0;                                     // full runs in all
    for (int c0 = 0; c0 < B; c0 += kWave) {
      const int bb = c0 + lane;
      const int T = bb < B ? tiles_of(bb) : 0;
      int f = T / R;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) f += __shfl_xor(f, o, kWave);
      F += Hkv * f;
      if (T % R) atomicAdd(&s_hist[T % R], Hkv);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    const int id = (int)blockIdx.x;
    int pick_seq = -1, pick_split = 0;
    if (id < F) {
      // the id-th full run: sequence order, then run order
      int before = 0;
      for (int c0 = 0; c0 < B && pick_seq < 0; c0 += kWave) {
        const int bb = c0 + lane;
        int pb = 0, f = 0;
        if (bb < B) {
          pb = prefix_lens[bb];
          f = (pb < 0 || pb > S_max - N) ? 0 : ((pb + N + kTile - 1) / kTile) / R;
        }
        int incl = Hkv * f;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
          const int t = __shfl_up(incl, d);
          if (lane >= d) incl += t;
        }
        const int excl = before + incl - Hkv * f;
        const uint64_t hit = __ballot(f > 0 && excl <= id && id < before + incl);
        if (hit) {
          const int src = __builtin_ctzll(hit);
          const int fb = __shfl(f, src), eb = __shfl(excl, src);
          const int r = id - eb;                   // kvh-major, then run
          pick_seq = (c0 + src) * Hkv + r / fb;
          pick_split = r % fb;
        }
        before += __shfl(incl, kWave - 1);
      }
    } else {
      // the k-th partial run, by decreasing length: lengths above lane's own
      const int k = id - F;
      const int cnt = s_hist[lane];                // runs whose partial length is lane
      int suf = cnt;                               // suffix sum over lengths >= lane
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const int t = __shfl_down(suf, d);
        if (lane + d < kWave) suf += t;
      }
      const int above = suf - cnt;                 // runs with a longer partial length
      const uint64_t in = __ballot(cnt > 0 && above <= k && k < above + cnt);
      if (in) {
        const int len = __builtin_ctzll(in);       // the partial length that holds rank k
        const int kk = k - __shfl(above, len);     // rank among runs of that length
        const int nb = kk / Hkv;                   // the nb-th request with that partial length
        int seen = 0;
        for (int c0 = 0; c0 < B && pick_seq < 0; c0 += kWave) {
          const int bb = c0 + lane;
          int T = 0;
          if (bb < B) {
            const int pb = prefix_lens[bb];
            T = (pb < 0 || pb > S_max - N) ? 0 : (pb + N + kTile - 1) / kTile;
          }
          const uint64_t m = __ballot(bb < B && T % R == len);
          const int c = __popcll(m);
          if (nb < seen + c) {
            // the (nb - seen)-th set bit of m
            uint64_t mm = m;
            for (int j = 0; j < nb - seen; ++j) mm &= mm - 1;
            const int src = __builtin_ctzll(mm);
            const int Tb = __shfl(T, src);
            pick_seq = (c0 + src) * Hkv + kk % Hkv;
            pick_split = Tb / R;
          }
          seen += c;
        }
      }
    }
    if (lane == 0) {
      s_pick[0] = pick_seq;
      s_pick[1] = pick_split;
    }
  }
  __syncthreads();
  const int seq = s_pick[0];
  if (seq < 0) return;                             // past the last run
  const int split = s_pick[1];
  const int b = seq / Hkv;
  const int kvh = seq % Hkv;
  const int g = Hq / Hkv;
  const int M = g * N;
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  const int P = prefix_lens[b];                    // in range: the pick skips the others
  const int L = P + N;
  const int T = (L + kTile - 1) / kTile;           // tiles of the sequence
  const int n_act = (T + split_len - 1) / split_len;   // runs with work
  if (split >= n_act) return;
  const int tile0 = split * split_len;
  const int ntiles = min(split_len, T - tile0);
  const bool direct = (n_act == 1);

  const size_t kv_off = (size_t)seq * S_max * D;   // element offset of the sequence's rows
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(kc + kv_off);
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(vc + kv_off);

  // ---- DMA of tile i of the run into stage st: wave w issues instructions
  // w, w+4, ...; lane l of instruction j fills LDS bytes j*1024 + 16l, i.e.
  // row j*RPI + l/UPR at physical unit l%UPR, holding logical unit
  // (l%UPR) ^ swz(row).  Rows at or past L repeat row L-1.
  auto dma_tile = [&](int i, int st) {
    const int t0 = (tile0 + i) * kTile;
#pragma unroll
    for (int qd = 0; qd < KPW; ++qd) {
      const int j = w + qd * kWaves;
      const int row = j * RPI + lane / UPR;
      const int c = min(t0 + row, L - 1);
      const size_t goff = (size_t)c * RBYTES + (((lane % UPR) ^ swz<UPR>(row)) << 4);
      dma16(kbase + goff, LDS_ADDR(ring) + (2 * st) * TB + j * 1024);
      dma16(vbase + goff, LDS_ADDR(ring) + (2 * st + 1) * TB + j * 1024);
    }
  };
  // ---- prologue, by DMA ahead of the first K/V tiles: Q and dO rows into
  // LDS (swizzled like the tiles), O rows into the last ring stage (not used
  // before the loop starts), the forward pass's lse and each row's ancestor
  // mask.  Rows m >= M repeat row M-1; their lse becomes +inf, so p = 0.
  {
    auto row_of = [&](int m) -> size_t {
      const int mm = min(m, M - 1);
      return (size_t)(b * N + mm / g) * Hq + kvh * g + mm % g;
    };
    constexpr int QI = MP * RBYTES / 1024;         // 1-KB DMA instructions per tensor
    for (int j = w; j < QI; j += kWaves) {
      const int m = j * RPI + lane / UPR;
      const size_t e = row_of(m) * D + 8 * ((lane % UPR) ^ swz<UPR>(m));
      dma16(q + e, LDS_ADDR(sq) + j * 1024);
      dma16(dout + e, LDS_ADDR(sdo) + j * 1024);
      dma16(out + e, LDS_ADDR(ring) + (2 * (NSTAGE - 1)) * TB + j * 1024);
    }
    if (w == 0) {
#pragma unroll
      for (int j = 0; j < (MP + 63) / 64; ++j)
        if (64 * j + lane < MP) dma4(lse + row_of(64 * j + lane), LDS_ADDR(s_lse2) + 256 * j);
#pragma unroll
      for (int j = 0; j < (2 * MP + 63) / 64; ++j) {
        const int idx = 64 * j + lane;             // dword idx of the per-row masks
        const int m = min(idx >> 1, M - 1);
        if ((idx >> 1) < MP)
          dma4(reinterpret_cast<const uint32_t*>(anc_mask) + 2 * ((size_t)b * N + m / g) + (idx & 1),
               LDS_ADDR(s_anc) + 256 * j);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NSTAGE - 1; ++i)
    if (i < ntiles) dma_tile(i, i);
  // the prologue's DMAs have landed once at most the K/V tiles' are in flight
  wait_ring<PT, 0, NSTAGE - 1, 0>(min(NSTAGE - 1, ntiles), 0);
  wg_barrier();
  {
    // D[m] = <dO[m], O[m]>: the UPR chunks of a row sit in UPR consecutive lanes
    constexpr int NCH = MP * UPR;
    static_assert(NCH % kThreads == 0, "chunks split evenly over the threads");
    const unsigned char* otmp = ring + (2 * (NSTAGE - 1)) * TB;
#pragma unroll
    for (int k = 0; k < NCH / kThreads; ++k) {
      const int c = tid + k * kThreads;
      const int m = c / UPR, u = c % UPR;
      const int off = m * RBYTES + ((u ^ swz<UPR>(m)) << 4);
      const bf16x8_t dov = *reinterpret_cast<const bf16x8_t*>(sdo + off);
      const bf16x8_t ov = *reinterpret_cast<const bf16x8_t*>(otmp + off);
      float dm = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dm = fmaf((float)dov[e], (float)ov[e], dm);
#pragma unroll
      for (int o = UPR / 2; o > 0; o >>= 1) dm += __shfl_xor(dm, o, kWave);
      if (u == 0) s_dm[m] = dm;
    }
    for (int m = tid; m < MP; m += kThreads) s_lse2[m] = (m < M) ? s_lse2[m] * kLog2e : INFINITY;
  }
  wait_lgkm0();
  wg_barrier();

  const float scale_log2 = sm_scale * kLog2e;

  // 8 bf16 of row `row`, logical unit `unit`, of a swizzled row-major buffer
  auto read_row = [&](const unsigned char* buf, int row, int unit) -> bf16x8_t {
    return *reinterpret_cast<const bf16x8_t*>(buf + row * RBYTES + ((unit ^ swz<UPR>(row)) << 4));
  };
  // Transpose read of a swizzled row-major buffer: lane (l16, lg) receives
  // column 16*cb + l16 of rows r0(lg) + 0..3 (first read) and r1(lg) + 0..3
  // (second): lanes 4k..4k+3 of a 16-lane group point at the 16 columns of
  // row k.
  auto read_tr = [&](const unsigned char* buf, int r0, int r1, int cb) -> bf16x8_t {
    i16x4_t t[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = (h ? r1 : r0) + (l16 >> 2);
      const int u = 2 * cb + ((l16 >> 1) & 1);
      const int off = row * RBYTES + ((u ^ swz<UPR>(row)) << 4) + ((l16 & 1) << 3);
      t[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(buf + off));
    }
    const i16x8_t both = __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, both);
  };

  // With 32 packed rows the Q and dO operands of every tile (natural and
  // transposed, 128 registers) stay in registers; larger M reads them from LDS.
  constexpr bool CACHE = (MP == 32);
  bf16x8_t qn[CACHE ? MB : 1][CACHE ? KC : 1], don[CACHE ? MB : 1][CACHE ? KC : 1];
  bf16x8_t qt[CACHE ? KS : 1][CACHE ? DB : 1], dot[CACHE ? KS : 1][CACHE ? DB : 1];
  if constexpr (CACHE) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        qn[mb][c] = read_row(sq, 16 * mb + l16, 4 * c + lg);
        don[mb][c] = read_row(sdo, 16 * mb + l16, 4 * c + lg);
      }
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        qt[s][db] = read_tr(sq, 32 * s + 4 * lg, 32 * s + 16 + 4 * lg, db);
        dot[s][db] = read_tr(sdo, 32 * s + 4 * lg, 32 * s + 16 + 4 * lg, db);
      }
  }
  // A operands: Q / dO rows 16mb.. at d-step c; Q^T / dO^T columns 16db.. at row step s
  auto q_nat = [&](int mb, int c) -> bf16x8_t {
    if constexpr (CACHE) return qn[mb][c];
    else return read_row(sq, 16 * mb + l16, 4 * c + lg);
  };
  auto do_nat = [&](int mb, int c) -> bf16x8_t {
    if constexpr (CACHE) return don[mb][c];
    else return read_row(sdo, 16 * mb + l16, 4 * c + lg);
  };
  auto q_tr = [&](int s, int db) -> bf16x8_t {
    if constexpr (CACHE) return qt[s][db];
    else return read_tr(sq, 32 * s + 4 * lg, 32 * s + 16 + 4 * lg, db);
  };
  auto do_tr = [&](int s, int db) -> bf16x8_t {
    if constexpr (CACHE) return dot[s][db];
    else return read_tr(sdo, 32 * s + 4 * lg, 32 * s + 16 + 4 * lg, db);
  };

  // dq^T accumulators: rows d = 16*(w*DN + dn) + 4lg + r, column m = 16mb + l16
  f32x4_t dqacc[DN][MB];
#pragma unroll
  for (int dn = 0; dn < DN; ++dn)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) dqacc[dn][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // dK / dV of the run's keys go out through buffer stores: bounds L rows, so
  // the keys of the last tile at or past L are dropped without a branch (and
  // every wave issues exactly SPT stores per tile, which the ring's vmcnt
  // waits count on)
  const __amdgpu_buffer_rsrc_t rdk = dev_rsrc(dk + kv_off, L * RBYTES);
  const __amdgpu_buffer_rsrc_t rdv = dev_rsrc(dv + kv_off, L * RBYTES);

  int st = 0;
  for (int i = 0; i < ntiles; ++i) {
    // wait for tile i: issued after it by this wave are the DMAs of the
    // `ahead` tiles after it and the stores of the last `sb` tiles
    const int ahead = min(NSTAGE - 2, ntiles - 1 - i);
    const int sb = min(i, NSTAGE - 1);
    wait_ring<PT, SPT, NSTAGE - 2, NSTAGE - 1>(ahead, sb);
    wg_barrier();                                  // tile i visible; tile i-1 and its dS done
    if (i + NSTAGE - 1 < ntiles) {
      int nst = st + NSTAGE - 1;
      if (nst >= NSTAGE) nst -= NSTAGE;
      dma_tile(i + NSTAGE - 1, nst);
    }
    const unsigned char* ks = ring + (2 * st) * TB;
    const unsigned char* vs = ring + (2 * st + 1) * TB;
    const int t0 = (tile0 + i) * kTile;
    const int key = 16 * w + l16;                  // this lane's key within the tile

    // ---- S = Q . K^T and dP = dO . V^T for the wave's 16 keys
    f32x4_t sacc[MB], pacc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      sacc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      pacc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const bf16x8_t kf = read_row(ks, key, 4 * c + lg);
      const bf16x8_t vf = read_row(vs, key, 4 * c + lg);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        sacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q_nat(mb, c), kf, sacc[mb], 0, 0, 0);
        pacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(do_nat(mb, c), vf, pacc[mb], 0, 0, 0);
      }
    }

    // ---- p and ds for rows m = 16mb + 4lg + r at this lane's key; the
    // K-slot t of k-step s holds row 32s + 4lg + t (t < 4) or 32s + 16 + 4lg
    // + t - 4, the run a lane gets from the C layout of blocks 2s and 2s+1
    const int tk = t0 + key;
    const bool plain = (t0 + kTile <= P);          // the whole tile is prefix
    const int j = tk - P;                          // tree node of the key, if >= 0
    bf16x8_t pb[KS], dsb[KS];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const f32x4_t l2 = *reinterpret_cast<const f32x4_t*>(s_lse2 + 16 * mb + 4 * lg);
      const f32x4_t dm = *reinterpret_cast<const f32x4_t*>(s_dm + 16 * mb + 4 * lg);
      bf16x4_t dsv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float p = fast_exp2(__builtin_fmaf(sacc[mb][r], scale_log2, -l2[r]));
        if (!plain) {
          const bool vis = (j < 0) || (j < N && ((s_anc[16 * mb + 4 * lg + r] >> j) & 1ull));
          p = vis ? p : 0.f;
        }
        const float ds = p * (pacc[mb][r] - dm[r]) * sm_scale;
        pb[mb >> 1][4 * (mb & 1) + r] = (__bf16)p;
        dsb[mb >> 1][4 * (mb & 1) + r] = (__bf16)ds;
        dsv[r] = (__bf16)ds;
      }
      // dS^T row `key`, columns 16mb + 4lg .. +3
      *reinterpret_cast<bf16x4_t*>(sds + key * DS_STRIDE + (16 * mb + 4 * lg) * 2) = dsv;
    }

    // ---- dV^T = dO^T . P and dK^T = Q^T . dS (rows d, column = key)
    f32x4_t dvacc[DB], dkacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      dvacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      dkacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dvacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(do_tr(s, db), pb[s], dvacc[db], 0, 0, 0);
        dkacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q_tr(s, db), dsb[s], dkacc[db], 0, 0, 0);
      }
    }
    // ---- dV and dK of the wave's 16 keys leave through the wave's own 16
    // rows of the V stage (free once its dP is done, and read by no other
    // wave): 8-byte LDS writes from the C layout, then contiguous 16-byte-
    // per-lane stores of whole rows.  Keys at or past L fall outside the
    // buffer bounds and are dropped.
    unsigned char* stg = ring + (2 * st + 1) * TB + 16 * w * RBYTES;
    auto stage_out = [&](const f32x4_t* acc, __amdgpu_buffer_rsrc_t rsrc) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        bf16x4_t v4;
#pragma unroll
        for (int r = 0; r < 4; ++r) v4[r] = (__bf16)acc[db][r];
        *reinterpret_cast<bf16x4_t*>(stg + l16 * RBYTES + (((2 * db + (lg >> 1)) ^ sws<UPR>(l16)) << 4) +
                                     ((lg & 1) << 3)) = v4;
      }
#pragma unroll
      for (int k = 0; k < SPT / 2; ++k) {
        const int row = k * RPI + lane / UPR;
        const int u = lane % UPR;
        const u32x4_t d = *reinterpret_cast<const u32x4_t*>(stg + row * RBYTES + ((u ^ sws<UPR>(row)) << 4));
        __builtin_amdgcn_raw_buffer_store_b128(d, rsrc, (t0 + 16 * w + row) * RBYTES + u * 16, 0, 0);
      }
    };
    stage_out(dvacc, rdv);
    stage_out(dkacc, rdk);

    // ---- dq^T += K^T . dS^T over the tile's 64 keys, this wave's columns
    wait_lgkm0();
    wg_barrier();                                  // every wave's dS^T rows written
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8_t ak[DN];
#pragma unroll
      for (int dn = 0; dn < DN; ++dn)
        ak[dn] = read_tr(ks, 32 * s2 + 8 * lg, 32 * s2 + 8 * lg + 4, w * DN + dn);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        // lane (m = 16mb + l16, lg): dS[m][32*s2 + 8lg + t], t = 0..7
        i16x4_t t[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int row = 32 * s2 + 8 * lg + 4 * h + (l16 >> 2);
          t[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4_t*)(sds + row * DS_STRIDE + (16 * mb + 4 * (l16 & 3)) * 2));
        }
        const bf16x8_t bds = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int dn = 0; dn < DN; ++dn)
          dqacc[dn][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[dn], bds, dqacc[dn][mb], 0, 0, 0);
      }
    }
    st = (st + 1 == NSTAGE) ? 0 : st + 1;
  }
  wait_vmcnt<0>();

  // ---- dq: rows d = 16*(w*DN + dn) + 4lg + r of column m = 16mb + l16
  auto dq_row = [&](int m) -> size_t { return ((size_t)(b * N + m / g) * Hq + kvh * g + m % g) * D; };
  if (direct) {
#pragma unroll
    for (int dn = 0; dn < DN; ++dn)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int m = 16 * mb + l16;
        if (m >= M) continue;
        bf16x4_t v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (__bf16)dqacc[dn][mb][r];
        *reinterpret_cast<bf16x4_t*>(dq + dq_row(m) + 16 * (w * DN + dn) + 4 * lg) = v;
      }
    return;
  }
  // partial of this run in the lanes' own order: chunk ((w*DN + dn)*MB + mb)*64 + lane
  constexpr int NCH = DB * MB * kWave;             // 16-byte chunks per partial
  const size_t slot_floats = (size_t)MP * D;
  {
    const __amdgpu_buffer_rsrc_t rp = dev_rsrc(part + ((size_t)seq * n_splits + split) * slot_floats, NCH * 16);
#pragma unroll
    for (int dn = 0; dn < DN; ++dn)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) store_dev4(rp, (((w * DN + dn) * MB + mb) * kWave + lane) * 16, dqacc[dn][mb]);
  }
  wait_vmcnt<0>();
  __syncthreads();
  uint32_t* cnt = counters + seq;
  if (tid == 0) {
    const uint32_t seen = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    s_last = (seen == (uint32_t)(n_act - 1)) ? 1u : 0u;
  }
  __syncthreads();
  if (!s_last) return;
  // last run: sum the runs' partials in run order; a thread owns chunks
  // tid + k*256, and issues KG chunks x 4 runs of loads at a time
  constexpr int CPTH = NCH / kThreads;             // chunks per thread
  constexpr int KG = CPTH < 4 ? CPTH : 4;
  static_assert(NCH % kThreads == 0 && CPTH % KG == 0, "merge chunks");
  const float* pbase = part + (size_t)seq * n_splits * slot_floats;
#pragma unroll 1
  for (int k0 = 0; k0 < CPTH; k0 += KG) {
    f32x4_t acc[KG];
#pragma unroll
    for (int k = 0; k < KG; ++k) acc[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n_act; s0 += 4) {
      f32x4_t x[4][KG];
#pragma unroll
      for (int sp = 0; sp < 4; ++sp) {
        const __amdgpu_buffer_rsrc_t rp = dev_rsrc(pbase + (size_t)(s0 + sp) * slot_floats, NCH * 16);
#pragma unroll
        for (int k = 0; k < KG; ++k) {
          x[sp][k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          if (s0 + sp < n_act) x[sp][k] = load_dev4(rp, (tid + (k0 + k) * kThreads) * 16);
        }
      }
#pragma unroll
      for (int sp = 0; sp < 4; ++sp)
#pragma unroll
        for (int k = 0; k < KG; ++k)
          if (s0 + sp < n_act) acc[k] += x[sp][k];
    }
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      const int c = tid + (k0 + k) * kThreads;
      const int ln = c & 63;
      const int mb = (c >> 6) % MB;
      const int dblk = (c >> 6) / MB;
      const int m = 16 * mb + (ln & 15);
      if (m >= M) continue;
      bf16x4_t v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (__bf16)acc[k][r];
      *reinterpret_cast<bf16x4_t*>(dq + dq_row(m) + 16 * dblk + 4 * (ln >> 4)) = v;
    }
  }
  if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ---------------------------------------------------------------- fp32
// One launch, two roles, kBwdF32Waves waves a workgroup; each wave sums its
// share and the shares are added in LDS.
//  - Workgroups [0, B*N*Hq): dq of one (request, node, head).  Wave w takes
//    the key chunks w, w + kBwdF32Waves, ...: lane = key for the scores, then
//    lane = column for the sum over the chunk's keys, each key's ds read from
//    its lane.
//  - The rest: dK and dV of one (request, kv head, key), lane = column.  Wave
//    w takes the (node, head) rows w, w + kBwdF32Waves, ... that see the key.
constexpr int kBwdF32Waves = 4;

template <int D>
__global__ __launch_bounds__(kBwdF32Waves * kWave) void tree_attn_bwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kc, const float* __restrict__ vc,
    const int32_t* __restrict__ prefix_lens, const uint64_t* __restrict__ anc_mask,
    const float* __restrict__ out, const float* __restrict__ lse, const float* __restrict__ dout, int B, int N,
    int Hq, int Hkv, int S_max, float sm_scale, float* __restrict__ dq, float* __restrict__ dk,
    float* __restrict__ dv, uint32_t* __restrict__ err_word) {
  constexpr int DPL = D / kWave;
  constexpr int NWV = kBwdF32Waves;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  __shared__ float s_acc[2][NWV][D];
  const int n_dq = B * N * Hq;
  if ((int)blockIdx.x < n_dq) {
    const int h = blockIdx.x % Hq;
    const int i = (blockIdx.x / Hq) % N;
    const int b = blockIdx.x / (Hq * N);
    const int kvh = h / (Hq / Hkv);
    const int P = prefix_lens[b];
    if (P < 0 || P > S_max - N) {
      if (threadIdx.x == 0 && i == 0 && h == 0) flag_error(err_word, SPEC_DERR_PREFIX);
      return;
    }
    const int L = P + N;
    const uint64_t anc = anc_mask[(size_t)b * N + i];
    const size_t row = ((size_t)(b * N + i) * Hq + h) * D;
    float dm = 0.f;
#pragma unroll
    for (int k = 0; k < DPL; ++k) dm = fmaf(dout[row + lane + k * kWave], out[row + lane + k * kWave], dm);
    dm = wave_sum(dm);
    const float l = lse[(size_t)(b * N + i) * Hq + h];
    const float* kb = kc + (size_t)(b * Hkv + kvh) * S_max * D;
    const float* vb = vc + (size_t)(b * Hkv + kvh) * S_max * D;
    float acc[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
    for (int c0 = wave * kWave; c0 < L; c0 += NWV * kWave) {
      const int c = c0 + lane;
      const bool ok = (c < L) && (c < P || ((anc >> (c - P)) & 1ull));
      float ds = 0.f;
      if (ok) {
        float s = 0.f, dp = 0.f;
        for (int d = 0; d < D; ++d) {
          s = fmaf(q[row + d], kb[(size_t)c * D + d], s);
          dp = fmaf(dout[row + d], vb[(size_t)c * D + d], dp);
        }
        const float p = expf(s * sm_scale - l);
        ds = p * (dp - dm) * sm_scale;
      }
      const int cmax = min(kWave, L - c0);
#pragma unroll
      for (int jj = 0; jj < kWave; ++jj) {
        if (jj >= cmax) break;
        const float x = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ds), jj));
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[k] = fmaf(x, kb[(size_t)(c0 + jj) * D + lane + k * kWave], acc[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k) s_acc[0][wave][lane + k * kWave] = acc[k];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      float t = s_acc[0][0][lane + k * kWave];
#pragma unroll
      for (int w = 1; w < NWV; ++w) t += s_acc[0][w][lane + k * kWave];
      dq[row + lane + k * kWave] = t;
    }
    return;
  }
  const int blk = (int)blockIdx.x - n_dq;
  const int c = blk % S_max;
  const int kvh = (blk / S_max) % Hkv;
  const int b = blk / (S_max * Hkv);
  const int P = prefix_lens[b];
  if (P < 0 || P > S_max - N) return;              // flagged by the dq role
  const int L = P + N;
  if (c >= L) return;
  const int g = Hq / Hkv;
  const size_t krow = ((size_t)(b * Hkv + kvh) * S_max + c) * D;
  float kv[DPL], vv[DPL], gk[DPL], gv[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    kv[k] = kc[krow + lane + k * kWave];
    vv[k] = vc[krow + lane + k * kWave];
    gk[k] = 0.f;
    gv[k] = 0.f;
  }
  for (int t = wave; t < N * g; t += NWV) {
    const int i = t / g, hl = t % g;
    if (c >= P && !((anc_mask[(size_t)b * N + i] >> (c - P)) & 1ull)) continue;
    const int h = kvh * g + hl;
    const size_t row = ((size_t)(b * N + i) * Hq + h) * D;
    float s = 0.f, dp = 0.f, dm = 0.f;
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      const int d = lane + k * kWave;
      s = fmaf(q[row + d], kv[k], s);
      dp = fmaf(dout[row + d], vv[k], dp);
      dm = fmaf(dout[row + d], out[row + d], dm);
    }
    s = wave_sum(s);
    dp = wave_sum(dp);
    dm = wave_sum(dm);
    const float p = expf(s * sm_scale - lse[(size_t)(b * N + i) * Hq + h]);
    const float ds = p * (dp - dm) * sm_scale;
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      const int d = lane + k * kWave;
      gv[k] = fmaf(p, dout[row + d], gv[k]);
      gk[k] = fmaf(ds, q[row + d], gk[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    s_acc[0][wave][lane + k * kWave] = gk[k];
    s_acc[1][wave][lane + k * kWave] = gv[k];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    float tk = s_acc[0][0][lane + k * kWave], tv = s_acc[1][0][lane + k * kWave];
#pragma unroll
    for (int w = 1; w < NWV; ++w) {
      tk += s_acc[0][w][lane + k * kWave];
      tv += s_acc[1][w][lane + k * kWave];
    }
    dk[krow + lane + k * kWave] = tk;
    dv[krow + lane + k * kWave] = tv;
  }
}

// ---------------------------------------------------------------- host
struct BwdPlan {
  int mp, nstage, split_len, n_splits;
  bool wide;                     // more than 128 packed rows: the separate dq and dK / dV passes
  size_t part_bytes;             // dq partials of the runs (0 when every run covers its sequence)
  size_t cnt_off;                // byte offset of the per-sequence run counters
  size_t ws_bytes;
};

// Runs of tiles, sized from the largest possible sequence (S_max keys): at
// least one workgroup per CU (a workgroup fills a CU's LDS), and no run
// longer than kMaxRun tiles, which bounds the tail of the longest-first
// schedule when prefix lengths differ.  Longer runs pay the prologue and the
// dq merge less often: at 16-node trees over 512..8192-token prefixes, 64
// gave 397 us, 32 388 us and 24 375 us (and 345 / 354 / 355 us with every
// prefix at the mean length).
constexpr int kCUs = 256;
constexpr int kMaxRun = 24;

static bool make_bwd_plan(int B, int N, int Hq, int Hkv, int D, int S_max, BwdPlan* p) {
  if (B < 1 || N < 1 || N > SPEC_MAX_NODES || Hkv < 1 || Hq < 1 || Hq % Hkv) return false;
  if (D != 64 && D != 128) return false;
  if (S_max < N || (long long)B * Hkv * S_max >= (1ll << 31) / 2 || (long long)S_max * D * 2 >= (1ll << 31))
    return false;
  if ((long long)B * N * Hq >= (1ll << 31)) return false;   // query rows index in int
  const int M = (Hq / Hkv) * N;
  p->wide = M > 128;
  if (p->wide) {
    p->mp = 0;
    p->nstage = 0;
    p->split_len = 0;
    p->n_splits = 1;
    p->part_bytes = p->cnt_off = 0;
    p->ws_bytes = bwd_wide_workspace_bytes(B, N, Hq);
    return true;
  }
  p->mp = M <= 32 ? 32 : (M <= 64 ? 64 : 128);
  p->nstage = (D == 128 && p->mp == 128) ? 2 : 3;
  const long long seqs = (long long)B * Hkv;
  const int n_tiles = (S_max + kTile - 1) / kTile;
  const long long want = std::max<long long>((kCUs + seqs - 1) / seqs, (n_tiles + kMaxRun - 1) / kMaxRun);
  int split_len = (int)((n_tiles + want - 1) / want);
  p->split_len = split_len;
  p->n_splits = (n_tiles + split_len - 1) / split_len;
  if (seqs * p->n_splits >= (1ll << 31)) return false;
  // workspace: dq partials and run counters when runs split a sequence
  p->part_bytes = p->n_splits > 1 ? (size_t)seqs * p->n_splits * p->mp * D * sizeof(float) : 0;
  p->cnt_off = p->part_bytes;
  p->ws_bytes = p->n_splits > 1 ? p->cnt_off + (size_t)seqs * sizeof(uint32_t) : 0;
  return true;
}

template <int D, int MP, int NS>
static void launch_bwd(const BwdPlan& pl, const void* q, const void* k, const void* v, const int32_t* pre,
                       const uint64_t* anc, const void* out, const float* lse, const void* dout, int B, int N,
                       int Hq, int Hkv, int S_max, float sm_scale, void* dq, void* dk, void* dv, float* part,
                       uint32_t* cnt, uint32_t* err, hipStream_t st) {
  const unsigned grid = (unsigned)(B * Hkv) * (unsigned)pl.n_splits;
  hipLaunchKernelGGL((tree_attn_bwd_kernel<D, MP, NS>), dim3(grid), dim3(kThreads), 0, st,
                     static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
                     pre, anc, static_cast<const __bf16*>(out), lse, static_cast<const __bf16*>(dout), B, N, Hq,
                     Hkv, S_max, sm_scale, pl.split_len, pl.n_splits, static_cast<__bf16*>(dq),
                     static_cast<__bf16*>(dk), static_cast<__bf16*>(dv), part, cnt, err);
}

}  // namespace bwd
}  // namespace spectree

using namespace spectree;
using namespace spectree::bwd;

extern "C" size_t spec_tree_attn_backward_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int S_max) {
  BwdPlan pl;
  if (!make_bwd_plan(B, N, Hq, Hkv, D, S_max, &pl)) return 0;
  return pl.ws_bytes;
}

extern "C" spec_status spec_tree_attn_backward(const void* q, const void* k_cache, const void* v_cache,
                                               spec_dtype dtype, const int32_t* prefix_lens,
                                               const uint64_t* anc_mask, const void* out, const float* lse,
                                               const void* d_out, int B, int N, int Hq, int Hkv, int D,
                                               int S_max, float sm_scale, void* dq, void* dk, void* dv,
                                               void* workspace, size_t workspace_bytes, uint32_t* err_word,
                                               hipStream_t stream) {
  if (!q || !k_cache || !v_cache || !prefix_lens || !anc_mask || !out || !lse || !d_out || !dq || !dk || !dv)
    return SPEC_ERR_NULL;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
  BwdPlan pl;
  if (!make_bwd_plan(B, N, Hq, Hkv, D, S_max, &pl)) return SPEC_ERR_SHAPE;
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale)) return SPEC_ERR_SHAPE;
  for (const void* p : {q, k_cache, v_cache, out, d_out, (const void*)dq, (const void*)dk, (const void*)dv})
    if (reinterpret_cast<uintptr_t>(p) & 15u) return SPEC_ERR_ALIGN;

  hip_clear_error();
  if (dtype == SPEC_F32) {
    const long long grid = (long long)B * N * Hq + (long long)B * Hkv * S_max;
    if (grid >= (1ll << 31)) return SPEC_ERR_SHAPE;
#define SPEC_F32_BWD(D_)                                                                                      \
  hipLaunchKernelGGL(tree_attn_bwd_f32_kernel<D_>, dim3((unsigned)grid), dim3(kBwdF32Waves * kWave), 0, stream, \
                     static_cast<const float*>(q), static_cast<const float*>(k_cache),                        \
                     static_cast<const float*>(v_cache), prefix_lens, anc_mask, static_cast<const float*>(out), \
                     lse, static_cast<const float*>(d_out), B, N, Hq, Hkv, S_max, sm_scale,                   \
                     static_cast<float*>(dq), static_cast<float*>(dk), static_cast<float*>(dv), err_word)
    if (D == 64) { SPEC_F32_BWD(64); } else { SPEC_F32_BWD(128); }
#undef SPEC_F32_BWD
    return launch_status();
  }

  float* part = nullptr;
  uint32_t* cnt = nullptr;
  if (pl.ws_bytes) {
    if (!workspace || workspace_bytes < pl.ws_bytes) return SPEC_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 15u) return SPEC_ERR_ALIGN;
    char* ws = static_cast<char*>(workspace);
    if (!pl.wide && pl.n_splits > 1) {
      part = reinterpret_cast<float*>(ws);
      cnt = reinterpret_cast<uint32_t*>(ws + pl.cnt_off);
    }
  }
  if (pl.wide)
    return bwd_wide_launch(q, k_cache, v_cache, prefix_lens, anc_mask, out, lse, d_out, B, N, Hq, Hkv, D, S_max,
                           sm_scale, dq, dk, dv, workspace, err_word, stream);
#define SPEC_BWD(D_, MP_, NS_)                                                                                 \
  if (D == D_ && pl.mp == MP_ && pl.nstage == NS_) {                                                           \
    launch_bwd<D_, MP_, NS_>(pl, q, k_cache, v_cache, prefix_lens, anc_mask, out, lse, d_out, B, N, Hq, Hkv,    \
                             S_max, sm_scale, dq, dk, dv, part, cnt, err_word, stream);                          \
    return launch_status();                                                                                    \
  }
  SPEC_BWD(128, 32, 3)
  SPEC_BWD(128, 64, 3)
  SPEC_BWD(128, 128, 2)
  SPEC_BWD(64, 32, 3)
  SPEC_BWD(64, 64, 3)
  SPEC_BWD(64, 128, 3)
#undef SPEC_BWD
  return SPEC_ERR_SHAPE;
}
