// Read-bandwidth probe for gfx950: how fast the memory system delivers the paged
// decode's access pattern when nothing else is done with the bytes.
//
// A paged decode streams each sequence's K and V as whole (block, kv head) tiles
// scattered through the pool -- 4 KB each at block size 16, bf16, head size 128.
// This kernel reads such pieces (at offsets the caller lists: in order, for a
// streaming read, or shuffled, for the paged gather) and keeps only a checksum, so
// its rate is the ceiling the decode's loads can reach on this part, with default or
// streaming (nt) loads.  It is a diagnostic next to the decode path, not a step of it.
//
// A second diagnostic, the co-execution probe, times matrix-core and vector-ALU work on
// one SIMD: how far the VALU instructions of one wave run while the MFMAs of the same
// wave, or of another wave on the SIMD, are in flight.  It bounds what a kernel whose
// steps alternate the two (the paged prefill) can gain from overlapping them.
#include "common.h"

namespace pa {

constexpr int kProbeThreads = 256;

// Workgroup b takes pieces [U*b, U*b + U), then [U*(b + grid), ...), and so on.  For a
// group of U pieces each thread loads its 16-byte chunk of every piece before it uses
// any of them, so U loads per thread are in flight.  Pieces past the end are skipped.
template <int U, bool NT>
__global__ void __launch_bounds__(kProbeThreads)
read_probe_kernel(const unsigned char* __restrict__ buf, const int64_t* __restrict__ offs,
                  int npieces, int piece_bytes, uint32_t* __restrict__ sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int chunks = piece_bytes / 16;
  for (long p0 = (long)blockIdx.x * U; p0 < npieces; p0 += (long)gridDim.x * U) {
    const int live = (int)min((long)U, npieces - p0);
    for (int c = threadIdx.x; c < chunks; c += kProbeThreads) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const long p = p0 + (u < live ? u : 0);
        const unsigned char* a = buf + offs[p] + (size_t)c * 16;
        v[u] = NT ? load16_nt(a) : load16(a);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) acc ^= v[u];
    }
  }
  sink[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Co-execution probe.  Every wave runs `iters` iterations of its work: MFMA work is 8
// independent chains of v_mfma_f32_16x16x32_bf16 (one MFMA each per iteration), VALU work
// is 32 fused multiply-adds over 8 independent chains.  Mode 0: MFMA work only; 1: VALU
// work only; 2: both in every wave, one MFMA then four FMAs (held in that order by
// scheduling barriers); 3: MFMA work in the first half of the workgroup's waves and VALU
// work in the second half.  A workgroup's waves go to the compute unit's four SIMDs in
// turn (wave w to SIMD w % 4), so at 8 waves every SIMD runs one wave of each kind; mode
// 4 checks that placement: no work, and every thread writes the SIMD its wave runs on
// (bits 5:4 of the hardware wave id register, HW_ID).  Otherwise one float per thread is
// written so that no work is removed.
constexpr int kCoexecMaxThreads = 512;

__global__ void __launch_bounds__(kCoexecMaxThreads)
coexec_probe_kernel(int mode, int iters, float seed, float* __restrict__ out) {
  const int wave = threadIdx.x >> 6;
  if (mode == 4) {
    const unsigned hw_id = __builtin_amdgcn_s_getreg(4 | (0 << 6) | (31 << 11));
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = static_cast<float>((hw_id >> 4) & 3u);
    return;
  }
  bool do_m = mode == 0 || mode == 2, do_v = mode == 1 || mode == 2;
  if (mode == 3) {
    do_m = 2 * wave < (int)(blockDim.x >> 6);
    do_v = !do_m;
  }
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(seed * static_cast<float>(threadIdx.x + i));
    b[i] = static_cast<__bf16>(seed - static_cast<float>(i));
  }
  f32x4 acc[8];
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    acc[k] = f32x4{seed, seed, seed, seed};
    v[k] = seed * static_cast<float>(k + 1) + static_cast<float>(threadIdx.x);
  }
  const float mul = 0.999f + seed * 1e-7f, add = 1e-3f * seed;
  if (do_m && do_v) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        __builtin_amdgcn_sched_barrier(0);
        acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[k], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[(k + q) & 7] = fmaf(v[(k + q) & 7], mul, add);
      }
    }
  } else if (do_m) {
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[k], 0, 0, 0);
  } else {
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int q = 0; q < 4; ++q) v[(k + q) & 7] = fmaf(v[(k + q) & 7], mul, add);
  }
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) sum += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3] + v[k];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

}  // namespace pa

namespace {
template <int U>
void launch_probe(bool nt, int workgroups, hipStream_t s, const unsigned char* b,
                  const int64_t* offs, int n, int piece_bytes, uint32_t* sink) {
  if (nt)
    hipLaunchKernelGGL((pa::read_probe_kernel<U, true>), dim3(workgroups), dim3(pa::kProbeThreads),
                       0, s, b, offs, n, piece_bytes, sink);
  else
    hipLaunchKernelGGL((pa::read_probe_kernel<U, false>), dim3(workgroups),
                       dim3(pa::kProbeThreads), 0, s, b, offs, n, piece_bytes, sink);
}
}  // namespace

extern "C" pa_status pa_read_probe(const void* buf, const int64_t* piece_offsets, int num_pieces,
                                   int piece_bytes, int workgroups, int in_flight,
                                   int nontemporal, uint32_t* sink, void* stream) {
  if (num_pieces < 0 || workgroups <= 0 || piece_bytes <= 0 || piece_bytes % 4096 ||
      (nontemporal != 0 && nontemporal != 1))
    return PA_ERR_INVALID_ARG;
  if (in_flight != 4 && in_flight != 8 && in_flight != 16) return PA_ERR_UNSUPPORTED;
  if (num_pieces == 0) return PA_OK;
  if (!buf || !piece_offsets || !sink) return PA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(buf) % 16 || reinterpret_cast<uintptr_t>(piece_offsets) % 8 ||
      reinterpret_cast<uintptr_t>(sink) % 4)
    return PA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned char* b = static_cast<const unsigned char*>(buf);
  const bool nt = nontemporal == 1;
  if (in_flight == 4)
    launch_probe<4>(nt, workgroups, s, b, piece_offsets, num_pieces, piece_bytes, sink);
  else if (in_flight == 8)
    launch_probe<8>(nt, workgroups, s, b, piece_offsets, num_pieces, piece_bytes, sink);
  else
    launch_probe<16>(nt, workgroups, s, b, piece_offsets, num_pieces, piece_bytes, sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

extern "C" pa_status pa_coexec_probe(int mode, int workgroups, int waves_per_workgroup,
                                     int iters, float* out, void* stream) {
  if (mode < 0 || mode > 4 || workgroups <= 0 || iters <= 0 || iters > (1 << 20) ||
      (waves_per_workgroup != 4 && waves_per_workgroup != 8))
    return PA_ERR_INVALID_ARG;
  if (!out || reinterpret_cast<uintptr_t>(out) % 4) return PA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(pa::coexec_probe_kernel, dim3((unsigned)workgroups),
                     dim3((unsigned)(waves_per_workgroup * 64)), 0,
                     static_cast<hipStream_t>(stream), mode, iters, 1.0f, out);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}
