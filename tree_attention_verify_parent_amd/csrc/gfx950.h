// gfx950 building blocks shared by the attention kernels: explicit wait
// counts and barriers, LDS DMA, device-scope partial-result stores and loads,
// the reductions over the four lanes of a 16x16 MFMA column, and vector types.
#pragma once

#include "common.h"

namespace spectree {

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

// Device-scope (all XCDs) stores and loads of partial results through buffer
// instructions with the SC1 cache policy: the hardware writes these through
// to the device coherence point and reads them from there, so data written by
// one workgroup is seen by another workgroup of the same launch on any XCD
// once the writer's store has completed (vmcnt) and the reader has observed
// the split counter.  Out-of-range offsets read zero and drop stores.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kSC1 = 16;                           // cache-policy bit: device scope
constexpr int kRsrcWord3 = 0x00020000;             // raw 32-bit buffer, gfx9 family
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRsrcWord3);
}
__device__ __forceinline__ void store_dev4(__amdgpu_buffer_rsrc_t r, int off, f32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, kSC1);
}
__device__ __forceinline__ void store_dev2(__amdgpu_buffer_rsrc_t r, int off, float a, float b) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{__float_as_uint(a), __float_as_uint(b)}, r, off, 0, kSC1);
}
__device__ __forceinline__ f32x4_t load_dev4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSC1));
}
__device__ __forceinline__ float2 load_dev2(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kSC1);
  return make_float2(__uint_as_float(v[0]), __uint_as_float(v[1]));
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

// One wave-wide 16-byte-per-lane DMA from global memory into LDS: lane l's
// 16 bytes land at LDS byte lds_addr + 16*l (lds_addr wave-uniform, via M0).
// Issued as inline assembly so the compiler's wait-count pass does not treat
// every later LDS read as depending on every DMA in flight; the kernel orders
// them itself with s_waitcnt vmcnt(N) before each barrier.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_addr)
               : "memory", "m0");
}
// The same with a wave-uniform global base (held in SGPRs) and a 32-bit lane
// offset: the saddr form of the DMA, which needs no 64-bit per-lane address
// arithmetic.  Lane l's 16 bytes come from sbase + voff.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  const uint64_t b = (uint64_t)sbase;
  // the builtin returns int: take each half back as unsigned before widening
  // (a sign-extended low half would corrupt the upper address bits)
  const uint64_t bu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(bu), "s"(lds_addr)
               : "memory", "m0");
}
// NF operand fragments read in batches of PB: batch j+1's reads are issued
// before batch j's products, so PB fragments stay in flight.  rd(x) issues the
// LDS reads of fragment x and mm(x) its products; scheduling barriers pin that
// order (left to itself the compiler issues each fragment's read right before
// its products and waits for it).
template <int NF, int PB, typename R, typename F>
__device__ __forceinline__ void batched_products(R rd, F mm) {
  static_assert(NF % PB == 0, "whole batches");
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int x = 0; x < PB; ++x) rd(x);
#pragma unroll
  for (int j = 0; j < NF / PB; ++j) {
    __builtin_amdgcn_sched_barrier(0);
    if (j + 1 < NF / PB) {
#pragma unroll
      for (int x = 0; x < PB; ++x) rd((j + 1) * PB + x);
    }
#pragma unroll
    for (int x = 0; x < PB; ++x) mm(j * PB + x);
  }
  __builtin_amdgcn_sched_barrier(0);
}
// LDS byte address of a __shared__ object (the cast of the object itself
// folds to a constant; callers add byte offsets to it)
#define LDS_ADDR(obj) ((uint32_t)(size_t)(lds_void_t*)(obj))

// The same for 4 bytes per lane: lane l's dword lands at lds_addr + 4*l.
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_addr) {
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(gptr), "s"(lds_addr)
               : "memory", "m0");
}

}  // namespace spectree
