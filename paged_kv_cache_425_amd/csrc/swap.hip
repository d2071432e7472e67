// Block swapping between the HBM pool and a pool in pinned host memory (gfx950).
//
// When GPU memory runs short the scheduler moves a request's KV out block by
// block, not the request as a whole, and can write the blocks to CPU memory;
// they come back when there is room (page "vLLM core architecture", section
// 2.3.2, which also notes that the CPU-GPU link then bounds throughput).
//
// One launch moves every block of the call: workgroup (pair, K or V) copies one
// block's contiguous (Hkv x D x BS) tile in 16-byte chunks, reading from one
// pool and writing to the other.  The pinned host pool is reached through its
// device mapping, so the GPU's own loads and stores cross the PCIe link (no
// copy-engine call per block); four chunks per thread are in flight at once to
// cover the link's latency.
#include "common.h"

namespace pa {

constexpr int kSwapThreads = 256;
constexpr int kSwapUnroll = 4;

__global__ void __launch_bounds__(kSwapThreads)
swap_blocks_kernel(const u32x4* __restrict__ src_k, const u32x4* __restrict__ src_v,
                   u32x4* __restrict__ dst_k, u32x4* __restrict__ dst_v,
                   const int64_t* __restrict__ pairs, int chunks, int src_nb, int dst_nb) {
  const int pr = blockIdx.x >> 1;
  const int is_v = blockIdx.x & 1;
  const int64_t s = pairs[2 * (size_t)pr], d = pairs[2 * (size_t)pr + 1];
  if (s < 0 || s >= src_nb || d < 0 || d >= dst_nb) return;
  const u32x4* from = (is_v ? src_v : src_k) + (size_t)s * chunks;
  u32x4* to = (is_v ? dst_v : dst_k) + (size_t)d * chunks;
  for (int c0 = threadIdx.x; c0 < chunks; c0 += kSwapThreads * kSwapUnroll) {
    u32x4 v[kSwapUnroll];
#pragma unroll
    for (int u = 0; u < kSwapUnroll; ++u) {
      const int c = c0 + u * kSwapThreads;
      if (c < chunks) v[u] = from[c];
    }
#pragma unroll
    for (int u = 0; u < kSwapUnroll; ++u) {
      const int c = c0 + u * kSwapThreads;
      if (c < chunks) to[c] = v[u];
    }
  }
}

}  // namespace pa

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Device address of a pool or table: device memory as is, pinned host memory through its
// device mapping.  Anything else (pageable host memory, unknown pointers) gives nullptr,
// so nothing is launched on memory the GPU cannot reach.
const void* device_address(const void* p) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();                 // leave no error behind for later calls
    return nullptr;
  }
  if (attr.type == hipMemoryTypeDevice) return p;
  if (attr.type == hipMemoryTypeHost && attr.devicePointer != nullptr) {
    // the pointer may sit inside the allocation: keep its offset
    const char* host_base = static_cast<const char*>(attr.hostPointer);
    if (host_base == nullptr) return attr.devicePointer;
    return static_cast<const char*>(attr.devicePointer) +
           (static_cast<const char*>(p) - host_base);
  }
  return nullptr;
}

int element_bytes(pa_dtype dt) {
  return dt == PA_DTYPE_F32 ? 4 : dt == PA_DTYPE_BF16 ? 2 : dt == PA_DTYPE_FP8_E4M3 ? 1 : 0;
}

}  // namespace

extern "C" pa_status pa_swap_blocks(const void* src_k, const void* src_v, void* dst_k,
                                    void* dst_v, const int64_t* block_mapping, int num_pairs,
                                    int num_kv_heads, int head_dim, int block_size,
                                    int src_num_blocks, int dst_num_blocks, pa_dtype dtype,
                                    void* stream) {
  const int elt = element_bytes(dtype);
  if (elt == 0) return PA_ERR_UNSUPPORTED;
  if (num_kv_heads <= 0 || src_num_blocks <= 0 || dst_num_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != 8 && block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
  if (num_pairs < 0) return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !block_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned(src_k, 16) || !aligned(src_v, 16) || !aligned(dst_k, 16) ||
      !aligned(dst_v, 16) || !aligned(block_mapping, 8))
    return PA_ERR_INVALID_ARG;
  const long grid = 2L * num_pairs;
  if (grid > 0x7FFFFFFFL) return PA_ERR_INVALID_ARG;
  const long block_bytes = (long)num_kv_heads * head_dim * block_size * elt;
  if (block_bytes / 16 > 0x7FFFFFFFL) return PA_ERR_INVALID_ARG;
  const void* sk = device_address(src_k);
  const void* sv = device_address(src_v);
  const void* dk = device_address(dst_k);
  const void* dv = device_address(dst_v);
  const void* bm = device_address(block_mapping);
  if (!sk || !sv || !dk || !dv || !bm) return PA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(pa::swap_blocks_kernel, dim3((unsigned)grid), dim3(pa::kSwapThreads), 0, s,
                     static_cast<const pa::u32x4*>(sk), static_cast<const pa::u32x4*>(sv),
                     static_cast<pa::u32x4*>(const_cast<void*>(dk)),
                     static_cast<pa::u32x4*>(const_cast<void*>(dv)),
                     static_cast<const int64_t*>(bm), (int)(block_bytes / 16), src_num_blocks,
                     dst_num_blocks);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}
