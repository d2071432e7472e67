// Device helpers shared by the gfx950 kernels of the paged-KV library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedattn.h"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;

// 16-byte global load / store (one dwordx4 per lane).
__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void store16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ float exp2_fast(float x) {
  // v_exp_f32: 2^x; exact 0 for -inf and 1 for 0.
  return __builtin_amdgcn_exp2f(x);
}

// Butterfly partner across the four 16-lane rows of a wave64.
__device__ __forceinline__ float xor16(float x) { return __shfl_xor(x, 16, 64); }
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// bfloat16 <-> float32 (round to nearest even on the way down).
__device__ __forceinline__ float bf16_to_f32(__bf16 h) { return static_cast<float>(h); }
__device__ __forceinline__ __bf16 f32_to_bf16(float x) { return static_cast<__bf16>(x); }

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

template <typename T>
struct ElemTraits;

template <>
struct ElemTraits<uint16_t> {            // bfloat16 bit patterns
  static constexpr int kBytes = 2;
  static constexpr int kX = 8;            // elements per 16-byte chunk
  static constexpr bool kBf16 = true;
};

template <>
struct ElemTraits<float> {
  static constexpr int kBytes = 4;
  static constexpr int kX = 4;
  static constexpr bool kBf16 = false;
};

}  // namespace pa
