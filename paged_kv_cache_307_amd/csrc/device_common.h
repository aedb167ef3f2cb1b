// Device-side helpers shared by the libpa kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace pa {

// bfloat16 bits <-> fp32.  Widening is exact; narrowing rounds to nearest
// even (NaN stays NaN).
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x0040u);  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// Read-only int32 data of a launch (block tables, context lengths): read
// through the constant address space, so that a wave-uniform index becomes
// a scalar-cache load even in kernels that also store to memory.
typedef __attribute__((address_space(4))) const int32_t ro_int32_t;
__device__ __forceinline__ int32_t load_ro(const int32_t* p, int64_t i) {
  return ((const ro_int32_t*)p)[i];
}

// Effective context length of sequence s: clamped to [0, max_context_len]
// and to the capacity of its table row.
__device__ __forceinline__ int effective_len(const DecodeArgs& a, int s, int block_size) {
  int L = load_ro(a.context_lens, s);
  L = L < 0 ? 0 : L;
  L = L > a.max_context_len ? a.max_context_len : L;
  const int cap = a.max_blocks_per_seq * block_size;
  return L > cap ? cap : L;
}

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t wave_uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(x)));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(x) >> 32));
  return int64_t((uint64_t(hi) << 32) | lo);
}

}  // namespace pa
