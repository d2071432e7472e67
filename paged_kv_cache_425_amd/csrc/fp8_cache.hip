// Write path into FP8 (E4M3) K/V pools for gfx950.
//
// The pages list FP8 E4M3 as an 8-bit float precision with about half the
// memory of 16-bit formats (page "vLLM core features", section 4.3, the table
// of quantisation formats); here it is the storage format of the paged K/V
// pools.  A new token's K and V are quantised with one scale per tensor and
// scattered into its slot, as reshape_and_cache does for 16/32-bit pools
// (page "vLLM core features", section 4.1: a new token only adds one entry).
//
// Quantisation of element x with scale s: the float32 quotient x / s
// (correctly rounded), then the nearest E4M3 code (e4m3_code: ties to even,
// saturating at 448).  A NaN element gives the NaN code with its own sign.
#include "common.h"

namespace pa {

constexpr int kFp8Threads = 256;

// 8 source elements starting at p, as float32.
template <typename T>
__device__ __forceinline__ void load8_elems(const T* p, float (&x)[8]) {
  if constexpr (ElemTraits<T>::kBf16) {
    const u32x4 w = load16(p);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(w[k] << 16);
      x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 w = load16(p + 4 * h);
#pragma unroll
      for (int k = 0; k < 4; ++k) x[4 * h + k] = __uint_as_float(w[k]);
    }
  }
}

// One workgroup per token.  Thread c quantises 8 consecutive channels of the token's K
// (c < Hkv*D/8) or V (the rest): K codes are one 8-byte store into the token's K row,
// V codes are 8 byte stores, one into each channel's token group.
template <typename T>
__global__ void __launch_bounds__(kFp8Threads)
reshape_and_cache_fp8_kernel(const T* __restrict__ key, const T* __restrict__ value,
                             const int64_t* __restrict__ slot_mapping,
                             uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                             int Hkv, int D, int BS, int NB, float k_scale, float v_scale) {
  const int i = blockIdx.x;
  const int groups = D / 8;                 // 8-channel groups per head
  const int ngroup = Hkv * groups;          // per token, for K and for V
  const size_t src0 = (size_t)i * Hkv * D;
  for (int c = threadIdx.x; c < 2 * ngroup; c += kFp8Threads) {
    const bool is_v = c >= ngroup;
    const int cc = is_v ? c - ngroup : c;
    float x[8];
    load8_elems((is_v ? value : key) + src0 + (size_t)cc * 8, x);
    const int64_t slot = slot_mapping[i];
    if (slot < 0 || slot >= (int64_t)NB * BS) continue;
    const float sc = is_v ? v_scale : k_scale;
    uint32_t codes[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      // a NaN element keeps its own sign (that of a NaN quotient is not fixed by IEEE 754)
      const uint32_t code = x[k] != x[k] ? (((__float_as_uint(x[k]) >> 24) & 0x80u) | 0x7Fu)
                                         : e4m3_code(__fdiv_rn(x[k], sc));
      codes[k >> 2] |= code << (8 * (k & 3));
    }
    const int64_t blk = slot / BS;
    const int off = (int)(slot % BS);
    const int h = cc / groups;
    const int d0 = (cc % groups) * 8;         // first channel of the group
    if (!is_v) {
      uint8_t* dst = k_cache + (((size_t)blk * Hkv + h) * BS + off) * D + d0;
      *reinterpret_cast<uint2*>(dst) = make_uint2(codes[0], codes[1]);
    } else {
      const int Xv = v_group<uint8_t>(BS);
      uint8_t* dst = v_cache + ((size_t)blk * Hkv + h) * D * BS + v_offset(off, d0, D, Xv);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        dst[(size_t)k * Xv] = static_cast<uint8_t>(codes[k >> 2] >> (8 * (k & 3)));
    }
  }
}

}  // namespace pa

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool good_scale(float s) { return s > 0.f && s <= 3.4028234663852886e38f; }

}  // namespace

extern "C" pa_status pa_reshape_and_cache_fp8(const void* key, const void* value,
                                              const int64_t* slot_mapping, void* k_cache,
                                              void* v_cache, int num_tokens, int num_kv_heads,
                                              int head_dim, int block_size, int num_blocks,
                                              pa_dtype dtype, float k_scale, float v_scale,
                                              void* stream) {
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != 8 && block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || !good_scale(k_scale) || !good_scale(v_scale)) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !slot_mapping || !k_cache || !v_cache) return PA_ERR_INVALID_ARG;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(slot_mapping, 8))
    return PA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* kc = static_cast<uint8_t*>(k_cache);
  uint8_t* vc = static_cast<uint8_t*>(v_cache);
  if (dtype == PA_DTYPE_BF16) {
    hipLaunchKernelGGL(pa::reshape_and_cache_fp8_kernel<uint16_t>, dim3(num_tokens),
                       dim3(pa::kFp8Threads), 0, s, static_cast<const uint16_t*>(key),
                       static_cast<const uint16_t*>(value), slot_mapping, kc, vc, num_kv_heads,
                       head_dim, block_size, num_blocks, k_scale, v_scale);
  } else {
    hipLaunchKernelGGL(pa::reshape_and_cache_fp8_kernel<float>, dim3(num_tokens),
                       dim3(pa::kFp8Threads), 0, s, static_cast<const float*>(key),
                       static_cast<const float*>(value), slot_mapping, kc, vc, num_kv_heads,
                       head_dim, block_size, num_blocks, k_scale, v_scale);
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}
