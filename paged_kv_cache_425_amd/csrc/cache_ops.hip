// Write path, copy-on-write and diagnostic read path of the paged KV cache (gfx950).
//
// reshape_and_cache: a new token only adds one entry to its sequence's
// mapping (page "vLLM core features", section 4.1); here its K and V are
// copied into the slot (physical block, offset) the scheduler chose for it.
// gather_kv: the inverse, reassembling each sequence through its block table
// (page "vLLM core architecture", section 2.2.2) as plain copies.
//
// Both are bit-exact copies; K moves in 16-byte chunks (a token's K row is
// contiguous in the token-major K pool), V element by element (a token holds one
// element of each channel's 16-byte token group).
#include "common.h"

namespace pa {

constexpr int kCopyThreads = 256;

// One workgroup per token.  Thread c moves 16-byte chunk c of the token's K
// (c < Hkv*D/X) or V (the rest): K chunks land whole in the cache, V chunks
// are split into X single-element stores, one per channel's token group.  The
// source chunk is loaded before the slot is looked at, so the two loads are
// in flight together.
template <typename T>
__global__ void __launch_bounds__(kCopyThreads)
reshape_and_cache_kernel(const T* __restrict__ key, const T* __restrict__ value,
                         const int64_t* __restrict__ slot_mapping, T* __restrict__ k_cache,
                         T* __restrict__ v_cache, int Hkv, int D, int BS, int NB) {
  constexpr int X = ElemTraits<T>::kX;
  const int i = blockIdx.x;
  const int chunks = D / X;                 // 16-byte chunks per head
  const int nchunk = Hkv * chunks;          // per token, for K and for V
  const size_t src0 = (size_t)i * Hkv * D;
  for (int c = threadIdx.x; c < 2 * nchunk; c += kCopyThreads) {
    const bool is_v = c >= nchunk;
    const int cc = is_v ? c - nchunk : c;
    const u32x4 val = load16((is_v ? value : key) + src0 + (size_t)cc * X);
    const int64_t slot = slot_mapping[i];
    if (slot < 0 || slot >= (int64_t)NB * BS) continue;
    const int64_t blk = slot / BS;
    const int off = (int)(slot % BS);
    const int h = cc / chunks;
    const int dc = cc % chunks;
    if (!is_v) {
      store16(k_cache + (((size_t)blk * Hkv + h) * BS + off) * D + (size_t)dc * X, val);
    } else {
      const int Xv = v_group<T>(BS);
      T* dst = v_cache + ((size_t)blk * Hkv + h) * D * BS + v_offset(off, dc * X, D, Xv);
      const T* e = reinterpret_cast<const T*>(&val);
#pragma unroll
      for (int k = 0; k < X; ++k) dst[(size_t)k * Xv] = e[k];
    }
  }
}

// One workgroup per (sequence, logical block).
template <typename T>
__global__ void __launch_bounds__(kCopyThreads)
gather_kv_kernel(T* __restrict__ k_out, T* __restrict__ v_out,
                 const int64_t* __restrict__ seq_offsets, const int32_t* __restrict__ block_table,
                 const int32_t* __restrict__ context_lens, const T* __restrict__ k_cache,
                 const T* __restrict__ v_cache, int Hkv, int D, int BS, int MB, int NB,
                 int blocks_per_seq) {
  constexpr int X = ElemTraits<T>::kX;
  const int s = blockIdx.x / blocks_per_seq;
  const int b = blockIdx.x % blocks_per_seq;
  int L = context_lens[s];
  L = L < 0 ? 0 : (L > MB * BS ? MB * BS : L);
  const int t0 = b * BS;
  if (t0 >= L) return;
  const int nt = min(BS, L - t0);
  const unsigned raw = static_cast<unsigned>(block_table[(size_t)s * MB + b]);
  const size_t phys = min(raw, static_cast<unsigned>(NB - 1));
  const size_t row0 = (size_t)seq_offsets[s] + t0;
  const int chunks = D / X;
  for (int c = threadIdx.x; c < nt * Hkv * chunks; c += kCopyThreads) {
    const int o = c / (Hkv * chunks);
    const int r = c % (Hkv * chunks);
    const int h = r / chunks;
    const int dc = r % chunks;
    const T* src = k_cache + ((phys * Hkv + h) * BS + o) * D + (size_t)dc * X;
    store16(k_out + ((row0 + o) * Hkv + h) * D + dc * X, load16(src));
  }
  for (int e = threadIdx.x; e < nt * Hkv * D; e += kCopyThreads) {
    const int o = e / (Hkv * D);
    const int r = e % (Hkv * D);
    const int h = r / D;
    const int d = r % D;
    v_out[((row0 + o) * Hkv + h) * D + d] =
        v_cache[(phys * Hkv + h) * D * BS + v_offset(o, d, D, v_group<T>(BS))];
  }
}

// Copy-on-write: block dst becomes a copy of block src.  One workgroup per
// (pair, kv head, K or V): a (block, kv head) tile of D * BS elements is
// contiguous in both pools, so the copy is a run of 16-byte chunks.  Pairs
// naming a block outside the pool are skipped.
template <typename T>
__global__ void __launch_bounds__(kCopyThreads)
copy_blocks_kernel(T* __restrict__ k_cache, T* __restrict__ v_cache,
                   const int64_t* __restrict__ pairs, int Hkv, int D, int BS, int NB) {
  constexpr int X = ElemTraits<T>::kX;
  const int id = blockIdx.x;
  const int is_v = id & 1;
  const int h = (id >> 1) % Hkv;
  const int pr = (id >> 1) / Hkv;
  const int64_t src = pairs[2 * (size_t)pr], dst = pairs[2 * (size_t)pr + 1];
  if (src < 0 || src >= NB || dst < 0 || dst >= NB) return;
  T* pool = is_v ? v_cache : k_cache;
  const size_t tile = (size_t)D * BS;
  const T* from = pool + ((size_t)src * Hkv + h) * tile;
  T* to = pool + ((size_t)dst * Hkv + h) * tile;
  const int chunks = (int)(tile / X);
  for (int c = threadIdx.x; c < chunks; c += kCopyThreads)
    store16(to + (size_t)c * X, load16(from + (size_t)c * X));
}

}  // namespace pa

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

pa_status check_cache_shapes(int num_kv_heads, int head_dim, int block_size, int num_blocks,
                             pa_dtype dtype) {
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != 8 && block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

}  // namespace

extern "C" pa_status pa_reshape_and_cache(const void* key, const void* value,
                                          const int64_t* slot_mapping, void* k_cache,
                                          void* v_cache, int num_tokens, int num_kv_heads,
                                          int head_dim, int block_size, int num_blocks,
                                          pa_dtype dtype, void* stream) {
  pa_status st = check_cache_shapes(num_kv_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !slot_mapping || !k_cache || !v_cache) return PA_ERR_INVALID_ARG;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(slot_mapping, 8))
    return PA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == PA_DTYPE_BF16) {
    hipLaunchKernelGGL(pa::reshape_and_cache_kernel<uint16_t>, dim3(num_tokens),
                       dim3(pa::kCopyThreads), 0, s, static_cast<const uint16_t*>(key),
                       static_cast<const uint16_t*>(value), slot_mapping,
                       static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                       num_kv_heads, head_dim, block_size, num_blocks);
  } else {
    hipLaunchKernelGGL(pa::reshape_and_cache_kernel<float>, dim3(num_tokens),
                       dim3(pa::kCopyThreads), 0, s, static_cast<const float*>(key),
                       static_cast<const float*>(value), slot_mapping,
                       static_cast<float*>(k_cache), static_cast<float*>(v_cache), num_kv_heads,
                       head_dim, block_size, num_blocks);
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

extern "C" pa_status pa_gather_kv(void* k_out, void* v_out, const int64_t* seq_offsets,
                                  const int32_t* block_table, const int32_t* context_lens,
                                  const void* k_cache, const void* v_cache, int num_seqs,
                                  int num_kv_heads, int head_dim, int block_size,
                                  int max_blocks_per_seq, int num_blocks, int max_context_len,
                                  pa_dtype dtype, void* stream) {
  pa_status st = check_cache_shapes(num_kv_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_context_len < 0) return PA_ERR_INVALID_ARG;
  if ((long)max_context_len > (long)max_blocks_per_seq * block_size) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0 || max_context_len == 0) return PA_OK;
  if (!k_out || !v_out || !seq_offsets || !block_table || !context_lens || !k_cache || !v_cache)
    return PA_ERR_INVALID_ARG;
  if (!aligned(k_out, 16) || !aligned(v_out, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(seq_offsets, 8) || !aligned(block_table, 4) ||
      !aligned(context_lens, 4))
    return PA_ERR_INVALID_ARG;
  const int bps = (max_context_len + block_size - 1) / block_size;
  const long grid = (long)num_seqs * bps;
  if (grid > 0x7FFFFFFFL) return PA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == PA_DTYPE_BF16) {
    hipLaunchKernelGGL(pa::gather_kv_kernel<uint16_t>, dim3((unsigned)grid), dim3(pa::kCopyThreads),
                       0, s, static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(v_out),
                       seq_offsets, block_table, context_lens,
                       static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache),
                       num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, bps);
  } else {
    hipLaunchKernelGGL(pa::gather_kv_kernel<float>, dim3((unsigned)grid), dim3(pa::kCopyThreads), 0,
                       s, static_cast<float*>(k_out), static_cast<float*>(v_out), seq_offsets,
                       block_table, context_lens, static_cast<const float*>(k_cache),
                       static_cast<const float*>(v_cache), num_kv_heads, head_dim, block_size,
                       max_blocks_per_seq, num_blocks, bps);
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

extern "C" pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping,
                                    int num_pairs, int num_kv_heads, int head_dim, int block_size,
                                    int num_blocks, pa_dtype dtype, void* stream) {
  // FP8 pools copy like any other: whole 16-byte chunks
  pa_status st = check_cache_shapes(num_kv_heads, head_dim, block_size, num_blocks,
                                    dtype == PA_DTYPE_FP8_E4M3 ? PA_DTYPE_BF16 : dtype);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_mapping, 8))
    return PA_ERR_INVALID_ARG;
  const long grid = (long)num_pairs * num_kv_heads * 2;
  if (grid > 0x7FFFFFFFL) return PA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == PA_DTYPE_FP8_E4M3) {
    hipLaunchKernelGGL(pa::copy_blocks_kernel<uint8_t>, dim3((unsigned)grid),
                       dim3(pa::kCopyThreads), 0, s, static_cast<uint8_t*>(k_cache),
                       static_cast<uint8_t*>(v_cache), block_mapping, num_kv_heads, head_dim,
                       block_size, num_blocks);
  } else if (dtype == PA_DTYPE_BF16) {
    hipLaunchKernelGGL(pa::copy_blocks_kernel<uint16_t>, dim3((unsigned)grid),
                       dim3(pa::kCopyThreads), 0, s, static_cast<uint16_t*>(k_cache),
                       static_cast<uint16_t*>(v_cache), block_mapping, num_kv_heads, head_dim,
                       block_size, num_blocks);
  } else {
    hipLaunchKernelGGL(pa::copy_blocks_kernel<float>, dim3((unsigned)grid), dim3(pa::kCopyThreads),
                       0, s, static_cast<float*>(k_cache), static_cast<float*>(v_cache),
                       block_mapping, num_kv_heads, head_dim, block_size, num_blocks);
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

extern "C" int pa_abi_version(void) { return PA_ABI_VERSION; }

extern "C" const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG: invalid argument";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: shape or dtype not supported";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: HIP launch failed";
  }
  return "unknown pa_status";
}
