// Device helpers shared by the gfx950 kernels of the paged-KV library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedattn.h"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;

// 16-byte global load / store (one dwordx4 per lane).
__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void store16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
// Streaming loads (the nt policy): data read once.  On gfx950 a gather of scattered 4 KB
// tiles reaches ~15% more bandwidth with them than with default-policy loads.
__device__ __forceinline__ u32x4 load16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ uint2 load8_nt(const void* p) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v[0], v[1]);
}

__device__ __forceinline__ float exp2_fast(float x) {
  // v_exp_f32: 2^x; exact 0 for -inf and 1 for 0.
  return __builtin_amdgcn_exp2f(x);
}

// Reductions across the four 16-lane rows of a wave64 (lanes n, n + 16, n + 32, n + 48)
// with gfx950's VALU lane swaps instead of an LDS permute.  v_permlane16_swap exchanges
// odd rows of its first operand with even rows of its second; given x twice, one result
// holds x and the other the partner row's x (lane l ^ 16), in an order that depends on the
// row -- so a symmetric op of the two results is x op x[l ^ 16] in every lane.
// v_permlane32_swap does the same across the two halves of the wave (lane l ^ 32).
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Reductions across the 16 lanes of each row with DPP moves: after quad_perm xor 1 and
// xor 2 every lane of a quad holds its quad's result, the half-row mirror (lane i reads
// lane 7 - i of its half-row) pairs the two quads of each half-row and the row mirror
// (lane i reads lane 15 - i) the two halves.  Each step combines a lane with its partner
// symmetrically, so all 16 lanes end with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm(1, 0, 3, 2)
constexpr int kDppXor2 = 0x4E;          // quad_perm(2, 3, 0, 1)
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_f32<kDppXor1>(x));
  x = fmaxf(x, dpp_f32<kDppXor2>(x));
  x = fmaxf(x, dpp_f32<kDppHalfMirror>(x));
  return fmaxf(x, dpp_f32<kDppMirror>(x));
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f32<kDppXor1>(x);
  x += dpp_f32<kDppXor2>(x);
  x += dpp_f32<kDppHalfMirror>(x);
  return x + dpp_f32<kDppMirror>(x);
}

// Word w of a 16-byte chunk as a pair of bf16.  The word is copied out first: clang
// lowers __builtin_bit_cast of an ext_vector element subscript (v[w]) to element 0.
__device__ __forceinline__ bf16x2 bf16_pair(u32x4 v, int w) {
  const uint32_t u = v[w];
  return __builtin_bit_cast(bf16x2, u);
}

// x of lane `src` (0..63) of the wave (ds_bpermute: no LDS storage is used).
__device__ __forceinline__ float lane_read(float x, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(4 * src, __float_as_int(x)));
}

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

template <>
struct ElemTraits<uint8_t> {             // OCP FP8 E4M3 codes (K/V cache storage only)
  static constexpr int kBytes = 1;
  static constexpr int kX = 16;
  static constexpr bool kBf16 = false;
};

// V cache tile of one (block, kv head): the block's BS tokens in groups of
// Xv = min(elements per 16 bytes, BS) tokens, each group channel-major, so that Xv
// consecutive tokens of one channel are one 16-byte chunk (an appended token touches one
// 16-byte chunk per channel, 8 channels per 128-byte line).  Element (token o, channel d)
// sits at ((o / Xv) * D + d) * Xv + o % Xv.
template <typename T>
__host__ __device__ constexpr int v_group(int BS) {
  return ElemTraits<T>::kX < BS ? ElemTraits<T>::kX : BS;
}
__host__ __device__ inline size_t v_offset(int o, int d, int D, int Xv) {
  return ((size_t)(o / Xv) * D + d) * Xv + o % Xv;
}

// ---- FP8 E4M3 (OCP): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
// holds subnormals m * 2^-9; S.1111.111 is NaN; no infinities; largest finite 448. ----

// Code of a float32 value: nearest E4M3 value, ties to the even code; magnitudes above 448
// and infinities saturate to +-448; NaN keeps its sign as S.1111.111.  Branch-free: both
// the subnormal and the normal candidate are formed (clamped, so no conversion leaves its
// range) and the right one is selected.
__device__ __forceinline__ uint32_t e4m3_code(float q) {
  const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
  const float a = fabsf(q);
  // below 2^-6 the grid is 2^-9: code = round(a * 2^9), 0 .. 8 (8 = smallest normal)
  const uint32_t sub = static_cast<uint32_t>(fminf(rintf(a * 512.f), 8.f));
  // normal: a = 2^e * (m / 8) with m in [8, 16]; m = 16 carries into the exponent
  const int e = min(max(static_cast<int>((__float_as_uint(a) >> 23) & 0xFFu) - 127, -6), 8);
  const uint32_t m = static_cast<uint32_t>(fminf(rintf(ldexpf(a, 3 - e)), 16.f));
  const uint32_t nrm = static_cast<uint32_t>(e + 7) * 8u + m - 8u;
  uint32_t code = a < 0.015625f ? sub : nrm;
  code = a >= 448.f ? 0x7Eu : code;                      // saturate (and +-inf)
  code = (a == a) ? code : 0x7Fu;                        // NaN
  return sign | code;
}

// Eight E4M3 codes (bytes of w0 then w1, lowest byte first) as an MFMA bf16 operand.
// Every E4M3 value is a bfloat16 value, so the conversion (scale 1) is exact.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, true));
  return __builtin_bit_cast(bf16x8, r);
}

}  // namespace pa
