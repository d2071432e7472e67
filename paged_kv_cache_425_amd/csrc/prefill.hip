// Paged prefill for gfx950 (MI355X): causal attention of a chunk of new query
// tokens per sequence over the sequence's paged K/V.
//
// What is computed: sequence s owns query rows query_start_loc[s] ..
// query_start_loc[s+1] - 1 (n tokens); with L = context_lens[s], row i is the
// token at position p = L - n + i and attends to positions 0 .. p of the K/V
// reassembled through the block table (page "vLLM core architecture", section
// 2.2.2).  Only the new tokens of a request are computed; its earlier, cached
// context -- e.g. a system prompt shared in physical blocks (page "core
// inference engine", section 2.2; prefix caching, page "core features",
// sections 4.2 and 4.6) -- is read through the table.  n = 1 is a decode step.
//
// Work decomposition
//   workgroup = (kv head, sequence, query tile).  A tile holds 128 query rows:
//     128 / g tokens x the g query heads of the kv head (row r = token r / g,
//     head r % g).  4 waves; wave w owns rows [32 w, 32 w + 32) as two 16-row
//     column blocks.
//   The workgroup streams the keys 0 .. (last position of the tile) in steps of
//   32 keys (bf16) or 16 keys (f32).  Each step's K and V tiles are loaded once
//   into LDS (every thread one 16-byte chunk of K and of V per 256 chunks) and
//   read by all waves.  LDS holds two tile buffers: step st is computed from one
//   while step st + 1 is staged into the other (one barrier per step), and the
//   global loads run two steps ahead in registers.
//   Q.K^T per column block is [keys x D] . [D x 16 rows] on MFMA (the K tile is the
//   A operand, the query rows the B operand), P.V is [D x keys] . [keys x 16 rows]
//   -- the same lane mapping as the decode kernel; each K or V fragment read from
//   LDS feeds both column blocks of the wave.  For bf16 the softmax weights enter
//   P.V as two bf16 MFMAs, p = hi + lo, accumulated into one output.
//   Rows keep a running max and sum (online softmax, base 2, the scale applied in
//   the exponent); the max moves only when a step raises it by more than kLazy, so
//   the accumulators are rescaled on few steps.  Key t counts for a row at position
//   p only if t <= p; steps wholly below the tile's first position skip the mask.
//   V rows at positions >= L are zeroed in LDS (their weight is 0, and 0 * NaN is
//   NaN).
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace pa {

struct PrefillParams {
  void* out;
  const void* q;
  const int32_t* qsl;            // query_start_loc [S + 1]
  const int32_t* block_table;
  const int32_t* context_lens;
  const void* k_cache;
  const void* v_cache;
  int S, Hq, Hkv, g, MB, NB, T, tiles;
  float scale_log2;
};

template <typename T, int D>
struct PrefillShape {
  static constexpr bool kBf16 = ElemTraits<T>::kBf16;
  static constexpr int kX = ElemTraits<T>::kX;               // elements per 16-byte chunk
  static constexpr int kStep = kBf16 ? 32 : 16;              // keys per step
  static constexpr int kTpl = kBf16 ? 8 : 4;                 // logits per lane per step
  static constexpr int kTiles = kBf16 ? 2 : 1;               // 16-key K tiles per step
  static constexpr int kNc = D / (kBf16 ? 32 : 16);          // K chunks per lane per tile
  static constexpr int kNs = D / 16;                         // 16-channel output slices
  static constexpr int kKChunks = kStep * (D / kX);          // 16-byte K chunks per step
  static constexpr int kVChunks = D * (kStep / kX);          // 16-byte V chunks per step
  // LDS rows: K [key][chunk] with a 16-byte pad, V [channel][keys] with a 16-byte pad
  static constexpr int kKRow = D / kX + 1;                   // in 16-byte units
  static constexpr int kVRow = kStep / kX + 1;               // in 16-byte units
  static constexpr int kKBytes = kStep * kKRow * 16;
  static constexpr int kVBytes = D * kVRow * 16;
};

constexpr int kPrefillWaves = 4;
constexpr int kPrefillRows = 128;                            // query rows per workgroup
constexpr int kPrefillBlocks = 2;                            // 16-row column blocks per wave
constexpr float kLazy = 8.f;                                 // lazy-rescale threshold (log2)

template <typename T, int D, int BS>
__global__ void __launch_bounds__(kPrefillWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
paged_prefill_kernel(const PrefillParams a) {
  using Sh = PrefillShape<T, D>;
  constexpr bool kBf16 = Sh::kBf16;
  constexpr int kX = Sh::kX;
  constexpr int kStep = Sh::kStep;
  constexpr int kTpl = Sh::kTpl;
  constexpr int kNc = Sh::kNc;
  constexpr int kNs = Sh::kNs;
  constexpr int kThreads = kPrefillWaves * 64;
  constexpr int kLoadsK = (Sh::kKChunks + kThreads - 1) / kThreads;
  constexpr int kLoadsV = (Sh::kVChunks + kThreads - 1) / kThreads;

  // two K/V tile buffers: step st is computed from buffer st % 2 while step st + 1 is
  // staged into the other
  __shared__ __align__(16) unsigned char kt[2 * Sh::kKBytes];
  __shared__ __align__(16) unsigned char vt[2 * Sh::kVBytes];
  __shared__ int tbl_lds[1024];                              // block-table window (<= 1024)

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int j = lane >> 4;

  int id = blockIdx.x;
  const int kvh = id % a.Hkv;
  id /= a.Hkv;
  const int s = id % a.S;
  const int tile = id / a.S;

  const int g = a.g;
  const int tile_tokens = kPrefillRows / g;
  int L = a.context_lens[s];
  L = L < 0 ? 0 : (L > a.MB * BS ? a.MB * BS : L);
  const int r0 = min(max(a.qsl[s], 0), a.T);
  int nq = min(max(a.qsl[s + 1], 0), a.T) - r0;
  nq = nq < 0 ? 0 : (nq > L ? L : nq);
  const int t0 = tile * tile_tokens;                         // first token of the tile
  if (t0 >= nq) return;
  const int t1 = min(nq, t0 + tile_tokens);
  const int pos0 = L - nq;                                   // position of chunk token 0
  const int kmax = pos0 + t1;                                // keys 0 .. kmax - 1 are seen
  const int nsteps = (kmax + kStep - 1) / kStep;
  const int nblk = (kmax + BS - 1) / BS;                     // <= MB

  // block-table window 0 .. nblk - 1, in chunks of 1024 entries (refilled per 1024 blocks).
  // Entries past the last block with a seen key repeat that block, so the last step's
  // loads past kmax need no clamp (in bounds; those keys are masked, their V zeroed).
  const int* bt = a.block_table + (size_t)s * a.MB;
  auto load_table = [&](int first) {
    const int end = min(1024, nblk + kStep / BS + 1 - first);
    for (int i = threadIdx.x; i < end; i += kThreads) {
      const unsigned b = static_cast<unsigned>(bt[min(first + i, nblk - 1)]);
      tbl_lds[i] = static_cast<int>(min(b, static_cast<unsigned>(a.NB - 1)));
    }
  };

  // ---- this wave's query rows: operand, position, output row -------------------------
  // column block cb (0, 1) of this wave: row = 32 * wave + 16 * cb + n
  u32x4 qop[kPrefillBlocks][kNc];
  int pos[kPrefillBlocks];                                   // row's position (-1: no row)
  size_t orow[kPrefillBlocks];
  const T* qbase = static_cast<const T*>(a.q);
#pragma unroll
  for (int cb = 0; cb < kPrefillBlocks; ++cb) {
    const int row = 32 * wave + 16 * cb + n;
    const int tok = t0 + row / g;
    const int head = kvh * g + row % g;
    const bool live = tok < t1;
    pos[cb] = live ? pos0 + tok : -1;
    orow[cb] = ((size_t)(r0 + (live ? tok : 0)) * a.Hq + head) * D;
#pragma unroll
    for (int c = 0; c < kNc; ++c) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      qop[cb][c] = live ? load16(qbase + orow[cb] + kX * (4 * c + j)) : z;
    }
  }

  // ---- cooperative K/V tile loads (global -> registers -> LDS) -------------------------
  const T* kc = static_cast<const T*>(a.k_cache);
  const T* vc = static_cast<const T*>(a.v_cache);
  const size_t head_elems = (size_t)D * BS;
  u32x4 kreg[kLoadsK], vreg[kLoadsV];

  // LDS row of a key within the step: the MFMA row that reads it (bf16: tile t = (key/4)%2,
  // row (key%4) + 4 * (key/8)), so the 16 lanes of a read pass take consecutive rows and
  // the 17-chunk row stride spreads them over distinct banks
  auto krow = [](int key) -> int {
    return kBf16 ? ((key >> 2) & 1) * 16 + (key & 3) + 4 * ((key >> 3) & 3) : key;
  };

  // chunk ids: K id = key * (D / kX) + q (q = 16-byte chunk of the key's row in the
  // token-major K pool), V id = group * D + channel (a V chunk is one channel's group of
  // kX tokens, and the groups of a block are channel-major); consecutive threads read
  // consecutive addresses within a block.
  // A step is kStep keys starting at a multiple of kStep.  When BS divides kStep, each
  // chunk's block within the step and its offset inside the block are fixed per thread
  // and a step only adds its first block; when kStep divides BS (f32, BS 32) the step
  // also adds its own offset inside the block.  Blocks past the last one with a seen key
  // are clamped to it (in bounds; those keys are masked, their V zeroed).
  static_assert(kStep % BS == 0 || BS % kStep == 0, "steps and blocks must nest");
  static_assert(v_group<T>(BS) == kX, "a V chunk is one token group");
  static_assert(Sh::kKChunks % kThreads == 0 && Sh::kVChunks % kThreads == 0,
                "every thread stages whole chunks of K and V");
  int k_blk[kLoadsK], v_blk[kLoadsV];                       // block offset within the step
  int k_off[kLoadsK], v_off[kLoadsV];                       // element offset in the tile
#pragma unroll
  for (int i = 0; i < kLoadsK; ++i) {
    const int cid = threadIdx.x + i * kThreads;
    const int q = cid % (D / kX), kk = cid / (D / kX);
    k_blk[i] = kk / BS;
    k_off[i] = (kk % BS) * D + q * kX;
  }
#pragma unroll
  for (int i = 0; i < kLoadsV; ++i) {
    const int cid = threadIdx.x + i * kThreads;
    const int ch = cid % D, grp = cid / D;
    v_blk[i] = grp * kX / BS;
    v_off[i] = (int)v_offset(grp * kX % BS, ch, D, kX);
  }
  // bytes per physical block (all kv heads), < 2^32: Hkv * D * BS * elt
  const uint32_t blk_bytes = static_cast<uint32_t>((size_t)a.Hkv * head_elems * sizeof(T));
  // each chunk's address is its fixed place within (block, kv head) plus block * blk_bytes
  const unsigned char* kp[kLoadsK];
  const unsigned char* vp[kLoadsV];
#pragma unroll
  for (int i = 0; i < kLoadsK; ++i)
    kp[i] = reinterpret_cast<const unsigned char*>(kc + (size_t)kvh * head_elems + k_off[i]);
#pragma unroll
  for (int i = 0; i < kLoadsV; ++i)
    vp[i] = reinterpret_cast<const unsigned char*>(vc + (size_t)kvh * head_elems + v_off[i]);
  auto at = [&](const unsigned char* p, int phys) {
    return p + (uint64_t)static_cast<uint32_t>(phys) * blk_bytes;
  };
  auto fetch = [&](int st) {
    const int b0 = st * kStep / BS;                          // first block of the step
    const int tb0 = b0 / 1024 * 1024;                        // its table window
    // kStep < BS (f32, BS 32): the step's offset inside its block, D * elt bytes per token
    // in both pools (a V group of kX tokens spans D chunks)
    const size_t boff = kStep < BS ? (size_t)(st * kStep % BS) * sizeof(T) : 0;
#pragma unroll
    for (int i = 0; i < kLoadsK; ++i)
      kreg[i] = load16(at(kp[i], tbl_lds[b0 - tb0 + k_blk[i]]) + boff * D);
#pragma unroll
    for (int i = 0; i < kLoadsV; ++i)
      vreg[i] = load16(at(vp[i], tbl_lds[b0 - tb0 + v_blk[i]]) + boff * D);
  };
  auto stage = [&](int st, int buf) {
    const int base = st * kStep;
    unsigned char* kb = kt + buf * Sh::kKBytes;
    unsigned char* vb = vt + buf * Sh::kVBytes;
#pragma unroll
    for (int i = 0; i < kLoadsK; ++i) {
      const int cid = threadIdx.x + i * kThreads;
      const int q = cid % (D / kX), key = cid / (D / kX);
      *reinterpret_cast<u32x4*>(kb + (krow(key) * Sh::kKRow + q) * 16) = kreg[i];
    }
    if (__builtin_expect(base + kStep > kmax, 0)) {          // the step ends past kmax
      // zero positions >= L (kmax <= L): weight 0 must not meet NaN
#pragma unroll
      for (int i = 0; i < kLoadsV; ++i) {
        const int grp = (threadIdx.x + i * kThreads) / D;
        const int nv = min(max(kmax - (base + grp * kX), 0), kX);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t mask;
          if (kBf16)
            mask = (2 * w + 1 < nv) ? 0xFFFFFFFFu : ((2 * w < nv) ? 0x0000FFFFu : 0u);
          else
            mask = (w < nv) ? 0xFFFFFFFFu : 0u;
          vreg[i][w] &= mask;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kLoadsV; ++i) {
      const int cid = threadIdx.x + i * kThreads;
      const int ch = cid % D, grp = cid / D;
      *reinterpret_cast<u32x4*>(vb + (ch * Sh::kVRow + grp) * 16) = vreg[i];
    }
  };

  float m_run[kPrefillBlocks], l_run[kPrefillBlocks];
  f32x4 acc[kPrefillBlocks][kNs];
#pragma unroll
  for (int cb = 0; cb < kPrefillBlocks; ++cb) {
    m_run[cb] = kNegInf;
    l_run[cb] = 0.f;
#pragma unroll
    for (int i = 0; i < kNs; ++i) acc[cb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // table window of a step (a window of 1024 blocks spans >= 8192 keys, many steps)
  auto window = [&](int st) { return (st * kStep / BS) / 1024; };
  load_table(0);
  __syncthreads();
  if (nsteps > 0) {
    fetch(0);
    stage(0, 0);
  }
  __syncthreads();
  if (nsteps > 1) fetch(1);                                  // same window as step 0
  auto run_step = [&](const int st, auto masked) {
    constexpr bool kMasked = decltype(masked)::value;
    const int base = st * kStep;
    const unsigned char* ktc = kt + (st & 1) * Sh::kKBytes;
    const unsigned char* vtc = vt + (st & 1) * Sh::kVBytes;

    // scores of both column blocks; each K fragment is read from LDS once and used by
    // both blocks' MFMAs (K tile rows are the A operand, query rows the B operand)
    float y[kPrefillBlocks][kTpl];
    if constexpr (kBf16) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        // row n of tile t holds key 8 * (n / 4) + 4 * t + n % 4 (stored at LDS row 16 t + n)
        f32x4 sc[kPrefillBlocks];
#pragma unroll
        for (int cb = 0; cb < kPrefillBlocks; ++cb) sc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < kNc; ++c) {
          const u32x4 kk =
              *reinterpret_cast<const u32x4*>(ktc + ((16 * t + n) * Sh::kKRow + 4 * c + j) * 16);
#pragma unroll
          for (int cb = 0; cb < kPrefillBlocks; ++cb)
            sc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kk),
                                                             __builtin_bit_cast(bf16x8, qop[cb][c]),
                                                             sc[cb], 0, 0, 0);
        }
#pragma unroll
        for (int cb = 0; cb < kPrefillBlocks; ++cb)
#pragma unroll
          for (int e = 0; e < 4; ++e) y[cb][4 * t + e] = sc[cb][e];
      }
    } else {
      f32x4 sc[kPrefillBlocks];
#pragma unroll
      for (int cb = 0; cb < kPrefillBlocks; ++cb) sc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < kNc; ++c) {
        const u32x4 kk = *reinterpret_cast<const u32x4*>(ktc + (n * Sh::kKRow + 4 * c + j) * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int cb = 0; cb < kPrefillBlocks; ++cb)
            sc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kk[e]),
                                                          __uint_as_float(qop[cb][c][e]), sc[cb],
                                                          0, 0, 0);
      }
#pragma unroll
      for (int cb = 0; cb < kPrefillBlocks; ++cb)
#pragma unroll
        for (int e = 0; e < 4; ++e) y[cb][e] = sc[cb][e];
    }

    // online softmax (base 2).  Masked steps: key base + kTpl*j + v counts if <= the
    // row's position.  The scale (> 0) enters in the exponent, exp2(y * s - m), and the
    // row max is taken on the raw scores (max(y * s) = s * max(y) for s > 0).  A row's
    // running max moves only when a step raises it by more than kLazy (its weights then
    // stay below 2^kLazy), so the accumulators are rescaled on few steps; the result is
    // the same sum with another common factor.
    float pw[kPrefillBlocks][kTpl];
    float alpha[kPrefillBlocks];
    bool moved = false;
#pragma unroll
    for (int cb = 0; cb < kPrefillBlocks; ++cb) {
      float mx = kNegInf;
#pragma unroll
      for (int v = 0; v < kTpl; ++v) {
        if constexpr (kMasked) {
          const bool live = base + kTpl * j + v <= pos[cb];
          y[cb][v] = live ? y[cb][v] : kNegInf;
        }
        mx = fmaxf(mx, y[cb][v]);
      }
      mx = max_xor16(mx);
      mx = max_xor32(mx);
      mx *= a.scale_log2;                                    // -inf stays -inf
      const float m_old = m_run[cb];
      const float m_new = (mx > m_old + kLazy) ? mx : m_old;    // -inf + kLazy = -inf
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      alpha[cb] = exp2_fast(m_old - m_use);                    // 1 unless the max moved
      float psum = 0.f;
#pragma unroll
      for (int v = 0; v < kTpl; ++v) {
        pw[cb][v] = exp2_fast(fmaf(y[cb][v], a.scale_log2, -m_use));
        psum += pw[cb][v];
      }
      l_run[cb] = l_run[cb] * alpha[cb] + psum;
      m_run[cb] = m_new;
      // while a row's max is -inf its weights were all 0 and its accumulators are 0
      moved = moved || (m_new != m_old && m_old != kNegInf);
    }
    if (__builtin_amdgcn_ballot_w64(moved) != 0) {
#pragma unroll
      for (int cb = 0; cb < kPrefillBlocks; ++cb)
#pragma unroll
        for (int sl = 0; sl < kNs; ++sl) acc[cb][sl] *= alpha[cb];
    }

    // P.V: each V fragment (A operand) is read once and used by both blocks' weights (B)
    if constexpr (kBf16) {
      // p = hi + lo: hi is p with its low 16 bits cleared (exact), lo = bf16(p - hi), so
      // the pair carries p to ~2^-16; two weights per packing instruction
      bf16x8 phi[kPrefillBlocks], plo[kPrefillBlocks];
#pragma unroll
      for (int cb = 0; cb < kPrefillBlocks; ++cb) {
        u32x4 hw, lw;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t u0 = __float_as_uint(pw[cb][2 * k]);
          const uint32_t u1 = __float_as_uint(pw[cb][2 * k + 1]);
          hw[k] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);    // upper halves of u0, u1
          const f32x2 r = {pw[cb][2 * k] - __uint_as_float(u0 & 0xFFFF0000u),
                           pw[cb][2 * k + 1] - __uint_as_float(u1 & 0xFFFF0000u)};
          lw[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
        }
        phi[cb] = __builtin_bit_cast(bf16x8, hw);
        plo[cb] = __builtin_bit_cast(bf16x8, lw);
      }
#pragma unroll
      for (int sl = 0; sl < kNs; ++sl) {
        const bf16x8 vv = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(vtc + ((16 * sl + n) * Sh::kVRow + j) * 16));
#pragma unroll
        for (int cb = 0; cb < kPrefillBlocks; ++cb)
          acc[cb][sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, phi[cb], acc[cb][sl], 0, 0, 0);
#pragma unroll
        for (int cb = 0; cb < kPrefillBlocks; ++cb)
          acc[cb][sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, plo[cb], acc[cb][sl], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int sl = 0; sl < kNs; ++sl) {
        const u32x4 vv =
            *reinterpret_cast<const u32x4*>(vtc + ((16 * sl + n) * Sh::kVRow + j) * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int cb = 0; cb < kPrefillBlocks; ++cb)
            acc[cb][sl] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vv[e]), pw[cb][e],
                                                               acc[cb][sl], 0, 0, 0);
      }
    }
    // stage the next step into the other buffer, then one barrier for both
    if (st + 1 < nsteps) stage(st + 1, (st + 1) & 1);
    if (st + 2 < nsteps && window(st + 2) != window(st + 1)) {
      __syncthreads();                                       // every fetch of step st+1 done
      load_table(window(st + 2) * 1024);
    }
    __syncthreads();
    if (st + 2 < nsteps) fetch(st + 2);
  };
  // steps below the tile's first position need no causal mask
  const int nfull = min(nsteps, (pos0 + t0 + 1) / kStep);
  for (int st = 0; st < nfull; ++st) run_step(st, std::false_type{});
  for (int st = nfull; st < nsteps; ++st) run_step(st, std::true_type{});

  // ---- normalise and write the rows -----------------------------------------------------
#pragma unroll
  for (int cb = 0; cb < kPrefillBlocks; ++cb) {
    float lsum = sum_xor16(l_run[cb]);
    lsum = sum_xor32(lsum);
    if (pos[cb] < 0) continue;
    const float inv = (m_run[cb] == kNegInf || lsum == 0.f) ? 0.f : 1.f / lsum;
#pragma unroll
    for (int sl = 0; sl < kNs; ++sl) {
      const size_t o = orow[cb] + 16 * sl + 4 * j;
      if constexpr (kBf16) {
        uint16_t* op = static_cast<uint16_t*>(a.out) + o;
#pragma unroll
        for (int e = 0; e < 4; ++e) op[e] = bf16_bits(acc[cb][sl][e] * inv);
      } else {
        float* op = static_cast<float*>(a.out) + o;
#pragma unroll
        for (int e = 0; e < 4; ++e) op[e] = acc[cb][sl][e] * inv;
      }
    }
  }
}

template <typename T, int D, int BS>
hipError_t launch_prefill(const PrefillParams& a, hipStream_t stream) {
  const long grid = (long)a.Hkv * a.S * a.tiles;
  hipLaunchKernelGGL((paged_prefill_kernel<T, D, BS>), dim3((unsigned)grid),
                     dim3(kPrefillWaves * 64), 0, stream, a);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_prefill(const PrefillParams& a, int D, int BS, hipStream_t stream) {
#define PA_CASE(DD, BB) \
  if (D == DD && BS == BB) return launch_prefill<T, DD, BB>(a, stream);
  PA_CASE(64, 8) PA_CASE(64, 16) PA_CASE(64, 32)
  PA_CASE(128, 8) PA_CASE(128, 16) PA_CASE(128, 32)
#undef PA_CASE
  return hipErrorInvalidValue;
}

}  // namespace pa

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" pa_status pa_paged_prefill(void* out, const void* query, const int32_t* query_start_loc,
                                      const int32_t* block_table, const int32_t* context_lens,
                                      const void* k_cache, const void* v_cache, int num_seqs,
                                      int num_heads, int num_kv_heads, int head_dim,
                                      int block_size, int max_blocks_per_seq, int num_blocks,
                                      int num_query_tokens, int max_query_len, float scale,
                                      pa_dtype dtype, void* stream) {
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads) return PA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != 8 && block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
  const int g = num_heads / num_kv_heads;
  if (g > 16 || pa::kPrefillRows % g != 0) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || num_query_tokens < 0 ||
      max_query_len < 0)
    return PA_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !(scale <= 3.4028234663852886e38f)) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0 || num_query_tokens == 0 || max_query_len == 0) return PA_OK;
  if (!out || !query || !query_start_loc || !block_table || !context_lens || !k_cache ||
      !v_cache)
    return PA_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(block_table, 4) || !aligned(context_lens, 4) ||
      !aligned(query_start_loc, 4))
    return PA_ERR_INVALID_ARG;
  const int tile_tokens = pa::kPrefillRows / g;
  const long tiles = ((long)max_query_len + tile_tokens - 1) / tile_tokens;
  const long grid = (long)num_kv_heads * num_seqs * tiles;
  if (grid > 0x7FFFFFFFL) return PA_ERR_INVALID_ARG;

  pa::PrefillParams a;
  a.out = out;
  a.q = query;
  a.qsl = query_start_loc;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.S = num_seqs;
  a.Hq = num_heads;
  a.Hkv = num_kv_heads;
  a.g = g;
  a.MB = max_blocks_per_seq;
  a.NB = num_blocks;
  a.T = num_query_tokens;
  a.tiles = (int)tiles;
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = dtype == PA_DTYPE_BF16
                       ? pa::dispatch_prefill<uint16_t>(a, head_dim, block_size, s)
                       : pa::dispatch_prefill<float>(a, head_dim, block_size, s);
  return err == hipSuccess ? PA_OK : PA_ERR_HIP;
}
