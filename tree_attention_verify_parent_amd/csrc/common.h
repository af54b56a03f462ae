// Shared device helpers for the spectree kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spectree.h"

namespace spectree {

constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Wave-wide reductions.  __shfl_xor lowers to DPP / ds_swizzle / permlane
// moves on gfx950; all 64 lanes take part.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t x, int src) {
  uint32_t lo = __shfl((uint32_t)x, src, kWave);
  uint32_t hi = __shfl((uint32_t)(x >> 32), src, kWave);
  return ((uint64_t)hi << 32) | lo;
}

// HIP keeps a thread's last error until it is read, so a failure of some
// unrelated earlier call would come back from the next check.  Each entry
// point clears it right before its launches and then reads only theirs.
inline void hip_clear_error() { (void)hipGetLastError(); }
inline spec_status launch_status() { return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP; }

__device__ __forceinline__ void flag_error(uint32_t* err_word, uint32_t bits) {
  if (err_word) atomicOr(err_word, bits);
}

// bf16 bit pattern of an OCP FP8 E4M3 code (exact: every e4m3 value is a
// bf16 value).  Sign | 4-bit exponent (bias 7) | 3-bit mantissa; exponent 0
// holds the subnormals m * 2^-9.  NaN codes are a precondition violation.
__device__ __forceinline__ uint32_t e4m3_to_bf16_bits(uint32_t code) {
  const uint32_t sign = (code & 0x80u) << 8;
  const uint32_t e = (code >> 3) & 0xFu;
  const uint32_t m = code & 0x7u;
  // normal: bf16 exponent = e - 7 + 127, mantissa m in the top 3 of 7 bits
  const uint32_t normal = ((e + 120u) << 7) | (m << 4);
  // subnormal m * 2^-9: leading one of m at bit p -> exponent 118 + p
  const uint32_t p = (m >= 4u) ? 2u : ((m >= 2u) ? 1u : 0u);
  const uint32_t sub = (m == 0u) ? 0u : (((118u + p) << 7) | ((m << (7u - p)) & 0x7Fu));
  return sign | (e != 0u ? normal : sub);
}

}  // namespace spectree
