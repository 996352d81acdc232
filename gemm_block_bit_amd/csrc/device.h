// Device-side helpers for gfx950 (CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gbb {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The fp16 pattern 0x6400 is 1024.0 with a zero 10-bit mantissa, so OR-ing a
// code q < 1024 into the mantissa gives the fp16 value 1024 + q exactly.
constexpr uint32_t kMagicPair = 0x64006400u;

__device__ __forceinline__ f32x4 mfma16(const half8& a, const half8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ i32x4 mfma16_i8(const i32x4& a, const i32x4& b, const i32x4& c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8 as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(half8, v);
}

__device__ __forceinline__ half2v as_half2(uint32_t a) { return __builtin_bit_cast(half2v, a); }
__device__ __forceinline__ uint32_t as_u32(half2v h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ float lo_half(uint32_t e) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(e & 0xffffu));
}
__device__ __forceinline__ float hi_half(uint32_t e) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(e >> 16));
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// 16-byte global load/store through the vector memory path.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace gbb
