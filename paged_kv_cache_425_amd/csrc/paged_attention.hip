// Paged decode attention for gfx950 (MI355X).
//
// What is computed: each sequence's single query token attends over the K/V
// reassembled through its block table (page "vLLM core architecture",
// section 2.2.2: attention over the KV sequence put back together from the
// block table).  The per-block loop there is made exact with a running max
// and running sum (online softmax): every partial result is rescaled to the
// largest logit seen so far, so the block-by-block accumulation equals the
// softmax over the whole sequence.
//
// Work decomposition
//   workgroup = (kv head, sequence, partition of P tokens); the kv head is the
//     fastest-varying index, so consecutive workgroups -- which the dispatcher
//     spreads round-robin over the 8 XCDs -- carry equal work, and the
//     partition index is the slowest, so the workgroups of partitions past a
//     sequence's end (which exit at once) come last.
//   NW waves per workgroup take the partition's 32-token steps round-robin;
//     each wave keeps the loads of its next step in flight while it computes
//     the current one (two register buffers; the prefetch is issued on every
//     iteration -- past the last step it re-reads the current, cached step --
//     so the compiler's wait counts never fall back to "wait for everything").
//   One step is 32 tokens (bf16) or 16 tokens (f32) of one KV head, shared by
//     the whole query-head group (GQA): each K/V byte is fetched once per group.
//   When partitions are short and plentiful, a workgroup instead takes NW
//     consecutive partitions of one sequence, one per wave: one table window and
//     prologue serve them all, and each wave writes its own partition's result.
//   When every sequence is one partition, a workgroup takes two (sequence, kv
//     head) units, the r-th longest and the r-th shortest sequence (the paired
//     mode below); the order comes from the host when it has the lengths.
//   Sequences that fit in one partition write their output directly.  Longer
//     ones write (max, sum, unnormalised output) per partition to the
//     workspace and a second kernel merges the partitions with a log-sum-exp
//     reduce.  When the batch has enough (sequence, kv head) pairs to fill the
//     GPU the default partition covers the longest sequence, so no merge is
//     needed; a merge inside the first kernel would need an agent-scope
//     release per workgroup, which on this multi-XCD part writes back and
//     invalidates the L2 and costs far more than a second launch.
//
// Matrix cores
//   Q.K^T for a step is [tokens x D] . [D x head-rows] and P.V is
//   [D x tokens] . [tokens x head-rows]: dense contractions, run on
//   v_mfma_f32_16x16x32_bf16 (bf16) or v_mfma_f32_16x16x4_f32 (f32).
//   With the cache layout of pagedattn.h every MFMA operand is one 16-byte
//   load per lane straight from HBM: K rows of 8 channels for Q.K^T, one V token
//   group -- 8 (bf16) or 4 (f32) consecutive tokens of one channel -- for P.V.
//   For bf16 the softmax weights must enter the P.V product in bf16.  To keep
//   float32 accuracy each weight is split p = hi + lo (both bf16, the error of
//   the pair is ~2^-17 p) and the head group occupies 2g of the 16 MFMA rows:
//   rows [0, g) carry hi, rows [g, 2g) carry lo, and the two are added at the
//   end.  The rows are there anyway (g <= 8 < 16), so this costs no extra MFMA.
//   A vector-ALU form of both products (VG > 0: bf16, g = 1, 2, 4; selected with
//   pa_set_decode_math) uses the same loads: bf16 dot products per lane, summed across
//   the lanes that hold a K row, and float32 FMAs for P.V with unsplit weights.  It is
//   kept for measurement: on the Llama-3-8B batch, with the same loads, the two tie at
//   g = 1 and the matrix cores are twice as fast at g = 4.
//
// FP8 pools (cache element C = uint8_t, E4M3 codes; queries bf16)
//   The cache element type is a template parameter.  With 1-byte codes a 16-byte
//   load holds 16 channels of a K row or a 16-token V group, so a step is 64
//   tokens (four 16-row K tiles) at the register cost of a 32-token bf16 step.
//   Codes are widened to bf16 in registers (v_cvt_scalef32_pk_bf16_fp8 at scale 1,
//   exact: every E4M3 value is a bf16 value) and go through the same bf16 MFMAs;
//   k_scale is folded into the softmax scale on the host and v_scale multiplies
//   the output.  The fused step quantises the new token with the write kernel's
//   encoder (e4m3_code) before patching it in.
//
// Lane mapping of a 16x16 MFMA output: lane l holds rows 4*(l/16)..+3 of
// column l%16.  Below, n = l%16 and j = l/16.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.h"

#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 4
#endif
#ifndef PA_DECODE_PIPE
#define PA_DECODE_PIPE 2
#endif
#ifndef PA_DECODE_OCC
#define PA_DECODE_OCC 2
#endif

namespace pa {

struct DecodeParams {
  void* out;
  float* part_ml;          // [S][Hq][Pmax][2]  (max in log2 units, weight sum)
  float* part_acc;         // [S][Hq][Pmax][D]  unnormalised output
  const void* q;
  const int32_t* block_table;
  const int32_t* context_lens;
  const void* k_cache;
  const void* v_cache;
  // fused decode step (all null for plain decode): the step's new token of each
  // sequence, [S][Hkv][D], and its slot, written into the caches before the reads
  const void* new_k;
  const void* new_v;
  const int64_t* new_slot;
  int S, Hq, Hkv, g, MB, NB, P, Pmax;
  int max_len;             // the caller's max_context_len (host-side launch choices only)
  int wave_parts;          // partition mode: 1 = each wave owns one partition of NW in a row
  float scale_log2;        // scale * log2(e) (* k_scale for FP8 K): base-2 logits
  float v_scale;           // output multiplier: 1, or the FP8 V scale
  float k_quant, v_quant;  // FP8 fused step: the scales the new token is quantised with
  // Shared-prefix mode (pa_decode_step_shared_prefix): every sequence's first pfx_len
  // positions are the same blocks; a workgroup takes `grp` consecutive sequences.
  int pfx_len;
  int grp;
};

// A context length clamped to what the launch can address.
__device__ __forceinline__ int clamp_len(const DecodeParams& a, int L, int BS) {
  const long cap = min((long)a.MB * BS, (long)a.P * a.Pmax);
  L = L < 0 ? 0 : L;
  return L > cap ? (int)cap : L;
}

__device__ __forceinline__ int clamped_len(const DecodeParams& a, int s, int BS) {
  return clamp_len(a, a.context_lens[s], BS);
}

// Final output of one channel of a row whose tokens gave the running max M (log2 units),
// weight sum den and unnormalised value num; nothing seen (M = -inf) gives 0.
__device__ __forceinline__ float finish_row(float M, float den, float num) {
  return (M == kNegInf || den == 0.f) ? 0.f : num / den;
}

// Per-step shape constants for a query/output type T and a cache element type C (C = T,
// or uint8_t for FP8 E4M3 codes, which need bf16 queries).
template <typename T, typename C, int D>
struct StepShape {
  static constexpr bool kBf16 = ElemTraits<T>::kBf16;
  static constexpr bool kFp8 = sizeof(C) == 1;
  static constexpr int kX = ElemTraits<C>::kX;      // cache elements per 16-byte chunk
  static constexpr int kStep = kFp8 ? 64 : (kBf16 ? 32 : 16);   // tokens per step
  static constexpr int kTpl = kStep / 4;            // logits per lane per step
  static constexpr int kTiles = kStep / 16;         // 16-row K tiles per step
  // 16-byte K chunks per lane per tile, and Q operands (MFMAs per tile)
  static constexpr int kNc = kFp8 ? D / 64 : D / (kBf16 ? 32 : 16);
  static constexpr int kNq = kFp8 ? D / 32 : kNc;
  static constexpr int kNs = D / 16;                // 16-channel slices of the output
  static_assert(!kFp8 || kBf16, "an FP8 cache is read with bf16 queries");
};

// The K and V operands of one step, as loaded.
template <typename T, typename C, int D>
struct StepData {
  using Sh = StepShape<T, C, D>;
  u32x4 k[Sh::kTiles][Sh::kNc];
  u32x4 v[Sh::kNs];
};

// LDS words per wave for the cross-wave merge: m[16], l[16], g rows of D (+4 pad).
__host__ __device__ constexpr int merge_stride(int D) { return D + 4; }
__host__ __device__ constexpr int merge_words(int D, int g) { return 32 + g * merge_stride(D); }

// Sequences the paired mode orders (the in-kernel ordering is O(S^2 / threads)).
constexpr int kMaxPairedSeqs = 512;
// Longest partition (tokens); a workgroup's table windows hold at most this many tokens
// per unit.
constexpr int kMaxPartition = 8192;
static_assert(kMaxPairedSeqs <= 1024, "a sort key holds 10 bits of sequence index");

// Paired mode: waves of the first unit, so that the busier unit's waves finish together.
// With a second sequence each unit keeps at least one wave (even an empty one), so that
// a split made from the host lengths never leaves a sequence without waves.
// Paired mode: waves are ranked 0, NW/2, 1, NW/2 + 1, ... (rank r = wave w gives w =
// r / 2 + (r % 2) * NW / 2).  With 8 waves, two share each SIMD and progress at different
// rates (the first half of the workgroup's waves ~1.5x faster than the second on gfx950), so
// a wave of the first half (even rank) takes 3 steps for every 2 of a wave of the second half
// (odd rank).  With 4 waves (one per SIMD of the workgroup) every wave takes 1.
__host__ __device__ constexpr int rank_weight(int rank, int nw) {
  return nw == 8 ? (rank % 2 == 0 ? 3 : 2) : 1;
}
__host__ __device__ inline int rank_capacity(int r0, int r1, int nw) {
  int c = 0;
  for (int r = r0; r < r1; ++r) c += rank_weight(r, nw);
  return c;
}

// Paired mode: waves (ranks [0, nA)) of the first unit, chosen so that the two units' steps per
// unit of capacity are as even as possible (exact integer comparisons, so that the host and the
// kernel choose alike).  With a second sequence each unit keeps at least one wave (even an empty
// one), so that a split made from the host lengths never leaves a sequence without waves.
__host__ __device__ inline int split_waves(int nw, int stA, int stB, bool two) {
  if (!two) return nw;
  int nA = 1;
  long long bn = -1, bd = 1;                                 // best max(stA/capA, stB/capB)
  for (int c = 1; c < nw; ++c) {
    const long long capA = rank_capacity(0, c, nw), capB = rank_capacity(c, nw, nw);
    const bool a_max = (long long)stA * capB >= (long long)stB * capA;
    const long long tn = a_max ? stA : stB, td = a_max ? capA : capB;
    if (bn < 0 || tn * bd < bn * td) {
      bn = tn;
      bd = td;
      nA = c;
    }
  }
  return nA;
}

// The pairs of the paired mode, made on the host from the scheduler's copy of the
// lengths and passed with the launch.  Pair r holds the r-th longest and the r-th
// shortest sequence (ties: lower index first):
//   pair[r].x = sA | sB << 16 (sB = 0xFFFF: none, the middle sequence of an odd count)
//   pair[r].y = blocks of sA | blocks of sB << 12 | waves of sA << 24, from the host
//               lengths (the table entries to stage at once -- the device lengths
//               decide the rest -- and the split of the waves between the two)
// pair[r].x = 0xFFFFFFFF: no plan, the kernel ranks the lengths itself.  The flag
// sits in the entry so that one scalar load, issued with the parameters', brings both.
struct PairOrder {
  uint2 pair[kMaxPairedSeqs / 2];
};
constexpr uint32_t kNoPlan = 0xFFFFFFFFu;
struct NoOrder {};
template <bool PAIRED>
using OrderArg = typename std::conditional<PAIRED, PairOrder, NoOrder>::type;

// Pair-balanced mode (PAIRED): a workgroup of NW waves (8, or 4 for short pairs that
// outnumber the compute units) takes two
// (sequence, kv head) units -- the r-th longest and the r-th shortest
// sequence -- and splits its waves between them in proportion to their steps,
// so that every workgroup carries about the same number of tokens.  The order
// of the sequences by length comes with the launch when the host has the
// lengths; otherwise every workgroup computes it from context_lens
// (identically), by counting for each sequence the sequences that are longer
// (ties broken by index).  Used when each sequence is one partition;
// otherwise a workgroup is one (kv head, sequence, partition).
//
// Shared-prefix mode (PREFIX, NW = 8): a workgroup takes one group of a.grp (1, 2 or 4)
// consecutive sequences that share their first a.pfx_len positions (the same physical
// blocks).  The first waves stream the shared prefix once for the whole group: the group's
// g-head query rows fill the columns of the MFMA operand (grp * g <= 16), so each prefix
// K/V byte is read once per group instead of once per sequence.  The other waves stream
// the sequences' private suffixes; the split follows the units' steps.  Each unit's waves
// are merged lane by lane in registers, and the prefix and suffix results of each row are
// combined with a log-sum-exp merge before the output is written.
template <typename T, typename C, int D, int BS, int NW, int PIPE, bool PAIRED,
          bool PREFIX = false, int VG = 0>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(PA_DECODE_OCC)))
paged_decode_kernel(const DecodeParams a, const OrderArg<PAIRED> ord) {
  static_assert(!(PAIRED && PREFIX), "the prefix pass is not paired");
  static_assert(VG == 0 || (ElemTraits<T>::kBf16 && sizeof(C) == 2 && !PREFIX),
                "the VALU math serves bf16 pools outside the shared-prefix mode");
  using Sh = StepShape<T, C, D>;
  constexpr bool kBf16 = Sh::kBf16;
  constexpr bool kFp8 = Sh::kFp8;
  constexpr int kX = Sh::kX;
  constexpr int kStep = Sh::kStep;
  constexpr int kTpl = Sh::kTpl;
  constexpr int kNc = Sh::kNc;
  constexpr int kNq = Sh::kNq;
  constexpr int kNs = Sh::kNs;
  constexpr int kThreads = NW * 64;
  constexpr int kXv = v_group<C>(BS);                      // tokens per V group
  static_assert(kXv == kTpl || (kFp8 && BS == 8), "a lane's V tokens are one group");

  // LDS: [ctrl: 16 ints][new K/V: 2 units x 2 x D elements][sort keys: S ints, PAIRED only]
  //      [tables: 1 or 2 windows of P/BS][merge]
  // paired mode: this pair's plan entry, requested before anything else so that its
  // scalar load goes out with the parameters' (the barrier keeps it first)
  uint64_t plan_entry = 0;
  if constexpr (PAIRED) {
    plan_entry = reinterpret_cast<const uint64_t*>(ord.pair)[blockIdx.y];
    __builtin_amdgcn_sched_barrier(0);
  }

  static_assert(!PREFIX || NW == 8, "the shared-prefix mode splits 8 waves 4 + 4");
  constexpr int kNewUnits = PREFIX ? 4 : 2;                 // new tokens staged in LDS
  extern __shared__ __align__(16) unsigned char smem[];
  int* ctrl = reinterpret_cast<int*>(smem);
  T* newkv = reinterpret_cast<T*>(smem + 64);                // [unit][K, V][D]
  const int win = a.P / BS;                                 // table entries per window
  const int lens_words = PAIRED ? (a.S + 3) / 4 * 4 : 0;
  int* lens = reinterpret_cast<int*>(smem + 64 + 2 * kNewUnits * D * sizeof(T));
  int* tbl = lens + lens_words;
  const int tbl_words =
      ((PAIRED ? 2 : (PREFIX ? 1 + a.grp : (a.wave_parts ? NW : 1))) * win + 3) / 4 * 4;
  float* red = reinterpret_cast<float*>(tbl + tbl_words);

  const int lane = threadIdx.x & 63;
  // wave index in a scalar register: the step loop below is then uniform per wave
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int j = lane >> 4;
  // position that row n of K tile t holds, in the step starting at position `base`
  auto step_row = [&](int base, int t) {
    return Sh::kTiles == 1 ? base + n : base + kTpl * (n >> 2) + 4 * t + (n & 3);
  };

  // paired mode: a 2-D grid (kv head, pair), so that the pair's plan entry can be
  // read together with the parameters; otherwise kv head fastest in a 1-D grid
  int id = PAIRED ? (int)blockIdx.y : (int)blockIdx.x;
  const int kvh = PAIRED ? (int)blockIdx.x : id % a.Hkv;
  if constexpr (!PAIRED) id /= a.Hkv;

  // ---- this wave's unit: sequence s, tokens [tok0, tok1), table window, wave slot ----
  int s, tok0 = 0, tok1 = 0, lw, nw, p = 0, nparts = 1, uidx = 0;
  int p0 = 0, seqL = 0;      // partition mode: the workgroup's first partition, the length
  int sA = 0, sB = -1, nA = NW;                             // PAIRED: the two sequences
  int gseq = 1, s0 = 0;                                     // PREFIX: the group's sequences
  bool pfx_wave = false;                                    // PREFIX: a wave of the prefix
  int part0 = 0;                                            // PREFIX: first wave of the unit
  int LA = 0, LB = 0;                                       // PAIRED: their lengths
  int blkA = 0, blkB = 0;                                   // PAIRED: their blocks
  bool planned = false;                                     // PAIRED: pairs from the host
  bool onA = true;
  const int* tblw = tbl;
  if constexpr (PAIRED) {
    const int r = id;                                       // pair index
    const int rB = a.S - 1 - r;
    const uint32_t ex = static_cast<uint32_t>(plan_entry);
    const uint32_t ey = static_cast<uint32_t>(plan_entry >> 32);
    planned = ex != kNoPlan;
    if (planned) {
      // the host's pair and wave split: the wave's sequence is known before any load
      sA = (int)(ex & 0xFFFFu);
      sB = (ex >> 16) == 0xFFFFu ? -1 : (int)(ex >> 16);
      nA = sB < 0 ? NW : min(max((int)(ey >> 24), 1), NW - 1);
      // the device lengths: both loads go out now and are first used after the
      // prologue's other loads (sA stands in for a missing second sequence)
      LA = a.context_lens[sA];
      LB = a.context_lens[sB >= 0 ? sB : sA];
      blkA = (int)(ey & 0xFFFu);                            // the host's block counts
      blkB = (int)((ey >> 12) & 0xFFFu);
    } else {
      // Sort keys: key_t = (L_t << 10) | (1023 - t), unique per sequence and ordered by
      // length, then by index for equal lengths (L_t <= P <= 8192 here, and S <= 512, so the
      // key fits in 24 bits; L_t = key >> 10).  Padded to a multiple of 4 with 0, below
      // every real key.
      for (int t = threadIdx.x; t < lens_words; t += kThreads)
        lens[t] = t < a.S ? (clamped_len(a, t, BS) << 10) | (1023 - t) : 0;
      __syncthreads();
      // rank of sequence t = how many keys are larger: one comparison per pair.  The S x S
      // comparisons are spread over every thread: thread x compares t = x % S with the
      // nparts-th slice (x / S) of the keys and leaves a partial count in the merge area
      // (free until the end), and thread t then adds its partial counts.
      int* part_rank = reinterpret_cast<int*>(red);           // [nparts][S]
      const int nparts = max(1, kThreads / a.S);              // 1 when S >= kThreads
      const int nq = lens_words / 4;                          // int4 groups of keys
      const int per = (nq + nparts - 1) / nparts;
      for (int x = threadIdx.x; x < nparts * a.S; x += kThreads) {
        const int t = x % a.S, pt = x / a.S;
        const int Kt = lens[t];
        int rank = 0;
        const int q1 = min(nq, (pt + 1) * per);
#pragma unroll 4
        for (int u4 = pt * per; u4 < q1; ++u4) {
          const int4 v = reinterpret_cast<const int4*>(lens)[u4];
          rank += (v.x > Kt) + (v.y > Kt) + (v.z > Kt) + (v.w > Kt);
        }
        part_rank[x] = rank;
      }
      __syncthreads();
      for (int t = threadIdx.x; t < a.S; t += kThreads) {
        int rank = 0;
        for (int pt = 0; pt < nparts; ++pt) rank += part_rank[pt * a.S + t];
        if (rank == r) ctrl[0] = t;
        if (rank == rB) ctrl[1] = t;
      }
      __syncthreads();
      sA = __builtin_amdgcn_readfirstlane(ctrl[0]);
      sB = r == rB ? -1 : __builtin_amdgcn_readfirstlane(ctrl[1]);
      LA = lens[sA] >> 10;
      LB = sB >= 0 ? lens[sB] >> 10 : 0;
      nA = split_waves(NW, (LA + kStep - 1) / kStep, (LB + kStep - 1) / kStep, sB >= 0);
      blkA = (LA + BS - 1) / BS;
      blkB = (LB + BS - 1) / BS;
    }
    nA = __builtin_amdgcn_readfirstlane(nA);
    // The two halves of the workgroup's waves share the SIMDs (wave w and w + NW / 2 on one)
    // and progress at different rates, so the units take waves alternately from the two
    // halves: unit A the first nA of waves 0, NW/2, 1, NW/2 + 1, ...
    const int rank = (wave % (NW / 2)) * 2 + wave / (NW / 2);
    onA = rank < nA;
    uidx = onA ? 0 : 1;
    s = onA ? sA : sB;
    lw = onA ? rank : rank - nA;
    nw = onA ? nA : NW - nA;
    tblw = tbl + (onA ? 0 : win);
  } else if constexpr (PREFIX) {
    // group id: sequences [s0, s0 + gseq); the first one's table row holds the prefix.
    // The waves are split between the prefix (unit 0) and the group's private suffixes
    // (units 1 .. gseq) in proportion to their steps -- the prefix's counted at 3/4, as
    // its blocks come from the L2 once the first group has read them (prefix-sharing batch:
    // 44.9 us at 3/4, 45.5 at 1/2, 47.6 at 1, 54.6 at 1/4) -- with at least one
    // and at most NW / 2 waves per unit (greedy: one more wave at a time to the unit with
    // the most steps per wave).  Every wave computes the same split.
    s0 = id * a.grp;
    gseq = min(a.grp, a.S - s0);
    const int cap = min(a.P / BS, a.MB - a.pfx_len / BS) * BS;   // suffix positions staged
    int ust[5], uwv[5];
    ust[0] = ((a.pfx_len + kStep - 1) / kStep * 3 + 3) / 4;
#pragma unroll
    for (int u = 1; u < 5; ++u) {
      const int Lu = u <= gseq ? min(max(a.context_lens[s0 + u - 1] - a.pfx_len, 0), cap) : 0;
      ust[u] = (Lu + kStep - 1) / kStep;
    }
    const int nunit = 1 + gseq;
#pragma unroll
    for (int u = 0; u < 5; ++u) uwv[u] = u < nunit ? 1 : 0;
    for (int k = nunit; k < NW; ++k) {
      int best = 0;
#pragma unroll
      for (int u = 1; u < 5; ++u)
        if (u < nunit && uwv[u] < NW / 2 &&
            (uwv[best] >= NW / 2 || ust[u] * uwv[best] > ust[best] * uwv[u]))
          best = u;
      uwv[best] += 1;
    }
    int u = 0, b = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (u < nunit - 1 && wave >= b + uwv[u]) {
        b += uwv[u];
        u += 1;
      }
    pfx_wave = u == 0;
    uidx = pfx_wave ? kNewUnits : u - 1;                    // the prefix has no new token
    lw = __builtin_amdgcn_readfirstlane(wave - b);
    nw = __builtin_amdgcn_readfirstlane(uwv[u]);
    part0 = __builtin_amdgcn_readfirstlane(b);
    s = pfx_wave ? s0 : s0 + uidx;
    // prefix positions [0, pfx_len), or suffix positions [0, L - pfx_len)
    tok1 = pfx_wave ? a.pfx_len : min(max(a.context_lens[s] - a.pfx_len, 0), cap);
  } else if (a.wave_parts) {
    // NW consecutive partitions, one per wave: the workgroup stages one table window
    // for all of them and each wave streams its partition alone and writes its own
    // partial result (no merge across waves)
    s = id % a.S;
    p0 = (id / a.S) * NW;
    seqL = clamped_len(a, s, BS);
    nparts = max(1, (seqL + a.P - 1) / a.P);
    if (p0 >= nparts) return;
    p = p0 + wave;
    tok0 = min(p * a.P, seqL);
    tok1 = min(seqL, tok0 + a.P);
    lw = 0;
    nw = 1;
    tblw = tbl + (tok0 - p0 * a.P) / BS;
  } else {
    s = id % a.S;
    p = id / a.S;
    const int L = clamped_len(a, s, BS);
    nparts = max(1, (L + a.P - 1) / a.P);
    if (p >= nparts) return;
    tok0 = p * a.P;
    tok1 = min(L, tok0 + a.P);
    lw = wave;
    nw = NW;
    p0 = p;
    seqL = L;
  }

  const int g = a.g;
  // MFMA columns in use: the g heads (bf16: plus their lo copies), or for the prefix's
  // waves the g heads of each of the group's sequences
  const int rows = pfx_wave ? gseq * g : (kBf16 ? 2 * g : g);
  const int head = kvh * g + (n % g);
  const bool row_live = n < rows;
  const int row_seq = pfx_wave ? s + (row_live ? n / g : 0) : s;   // sequence of column n

  const C* kc = static_cast<const C*>(a.k_cache);
  const C* vc = static_cast<const C*>(a.v_cache);
  const size_t head_elems = (size_t)D * BS;          // elements of one (block, kv head)

  // ---- loads of one step ------------------------------------------------------
  // Load policy.  Each K load instruction reads 64 bytes of each of 16 rows, half of each
  // 128-byte line, and the next instruction reads the other half: K keeps the default
  // policy, so that half comes from the cache.  V instructions read whole lines (16
  // channel rows of a block, contiguous) and stream with the nt policy, which gathers
  // scattered 4 KB tiles ~15% faster on gfx950 -- except in the waves of a shared prefix,
  // whose blocks every group of the launch reads again from L2.
  const bool v_stream = !(PREFIX && pfx_wave);
  auto v_load = [&](const C* p) { return v_stream ? load16_nt(p) : load16(p); };
  // Loads of step st, with positions clamped below `end` and the block of a position
  // given by phys_k(t, pos) (K tile t) and phys_v(h, pos) (V group h).
  auto load_step_from = [&](int st, StepData<T, C, D>& b, int end, auto&& phys_k,
                            auto&& phys_v) {
    const int base = tok0 + st * kStep;
#pragma unroll
    for (int t = 0; t < Sh::kTiles; ++t) {
      // K-tile row n: bf16/FP8 rows interleave the step as kTpl*(n/4) + 4*t + n%4 so
      // that the score of lane (n, j), register 4t + e is token kTpl*j + 4*t + e; f32
      // rows are tokens n.  Rows past the partition's end read the last live token
      // instead (in bounds; their logits are masked to -inf).
      const int tok = min(step_row(base, t), end - 1);
      const int phys = phys_k(t, tok);
      // token-major K: the row of token `tok` is D contiguous elements; lane j takes its
      // 16-byte chunks j, j + 4, ...
      const C* kp = kc + (((size_t)phys * a.Hkv + kvh) * BS + tok % BS) * D + (size_t)j * kX;
#pragma unroll
      for (int c = 0; c < kNc; ++c) b.k[t][c] = load16(kp + 4 * c * kX);
    }
    // V operand of slice sl: channel 16*sl + n, tokens base + kTpl*j .. + kTpl - 1 -- one
    // 16-byte token group of the channel, so the 16 lanes of a row read 256 contiguous
    // bytes.  A group wholly past the end reads the group of the last live token (in
    // bounds; it is zeroed before use).
    const int tokv = min(base + kTpl * j, (end - 1) / kTpl * kTpl);
    const int physv = phys_v(0, tokv);
    const C* vp = vc + ((size_t)physv * a.Hkv + kvh) * head_elems + v_offset(tokv % BS, n, D, kXv);
    if constexpr (kFp8 && BS < 16) {
      // 16 tokens span two blocks of 8: two 8-byte groups (the second clamped like tokv)
      const int tokv2 = min(tokv + 8, (end - 1) / 8 * 8);
      const int physv2 = phys_v(1, tokv2);
      const C* vp2 = vc + ((size_t)physv2 * a.Hkv + kvh) * head_elems + v_offset(0, n, D, kXv);
#pragma unroll
      for (int sl = 0; sl < kNs; ++sl) {
        const uint2 lo = load8_nt(vp + (size_t)16 * sl * kXv);
        const uint2 hi = load8_nt(vp2 + (size_t)16 * sl * kXv);
        b.v[sl] = u32x4{lo.x, lo.y, hi.x, hi.y};
      }
    } else {
#pragma unroll
      for (int sl = 0; sl < kNs; ++sl) b.v[sl] = v_load(vp + (size_t)16 * sl * kXv);
    }
  };
  auto window = [&](int, int pos) { return tblw[(pos - tok0) / BS]; };
  auto load_step = [&](int st, StepData<T, C, D>& b) {
    load_step_from(st, b, tok1, window, window);
  };

  // Paired mode over FP8 pools: each wave's first step is loaded before the table windows
  // reach LDS, from table entries its lanes read themselves, so that its K/V loads wait
  // for neither the windows nor the barrier and run while the prologue encodes the new
  // tokens to E4M3 (bf16 pools have no such work there, and gained nothing from it).  The
  // entries are read before the prologue's other loads, so that waiting for them waits for
  // no other load: the columns of the step's own positions and the column of the unit's
  // last block (by the host's block count for a planned launch).  By the time they land,
  // so has the length: positions past the end are clamped to its last position, as in
  // every other step, and read the last block's entry -- or, if the host's count was
  // stale, their own column's, which is in bounds (the column clamped to the row, the
  // block id to the pool) and masked.
  constexpr bool kEarly = PAIRED && PIPE == 2 && kFp8;
  int first_st = 0, first_last = 0;
  unsigned first_k[Sh::kTiles], first_v[2], first_lb = 0;
  StepData<T, C, D> first_b;
  if constexpr (kEarly) {
    first_st = __builtin_amdgcn_readfirstlane(rank_capacity(onA ? 0 : nA, (onA ? 0 : nA) + lw, NW));
    const int base = tok0 + first_st * kStep;
    const int32_t* row = a.block_table + (size_t)s * a.MB;
#pragma unroll
    for (int t = 0; t < Sh::kTiles; ++t) first_k[t] = row[min(step_row(base, t) / BS, a.MB - 1)];
    first_v[0] = row[min((base + kTpl * j) / BS, a.MB - 1)];
    if constexpr (kFp8 && BS < 16) first_v[1] = row[min((base + kTpl * j + 8) / BS, a.MB - 1)];
    first_last = max(min(onA ? blkA : blkB, a.MB) - 1, 0);
    first_lb = row[first_last];
    __builtin_amdgcn_sched_barrier(0);
  }

  // Every load of the prologue is issued before the first wait on any of them: the
  // query operand, the new tokens and the block-table windows land in one round trip.
  //
  // Query operand: lane (n, j) holds head-row n's channels of the chunks it multiplies.
  // FP8: K chunk j + 4c' (16 channels) feeds MFMAs 2c' and 2c' + 1 (8 channels each).
  const T* qrow = static_cast<const T*>(a.q) + ((size_t)row_seq * a.Hq + head) * D;
  u32x4 qop[kNq];
  // VALU math: lane (n, j) holds the same channels of every head of the group
  u32x4 qv[VG > 0 ? VG : 1][kNc];
  if constexpr (VG > 0) {
    const T* qg = static_cast<const T*>(a.q) + ((size_t)s * a.Hq + kvh * VG) * D;
#pragma unroll
    for (int h = 0; h < VG; ++h)
#pragma unroll
      for (int c = 0; c < kNc; ++c) qv[h][c] = load16(qg + (size_t)h * D + kX * (4 * c + j));
  } else {
#pragma unroll
    for (int c = 0; c < kNq; ++c) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      const int off = kFp8 ? 16 * (j + 4 * (c >> 1)) + 8 * (c & 1) : kX * (4 * c + j);
      qop[c] = row_live ? load16(qrow + off) : z;
    }
  }

  // Block-table windows: entry i of `count` is column col(i) of row row(i), staged at
  // LDS word dst(i); ids are clamped so that every read stays inside the pool.  The
  // loads go to registers first (lanes past the end re-read the last entry, so no load
  // sits in a divergent branch) and are written to LDS once the new tokens' loads are
  // out as well.  kPer entries per thread cover two windows of the longest partition.
  constexpr int kPer =
      ((PAIRED ? 2 : (PREFIX ? 5 : 1)) * (kMaxPartition / BS) + kThreads - 1) / kThreads;
  auto stage_load = [&](int count, unsigned (&b)[kPer], auto&& where) {
    const int iters = min(kPer, (count + kThreads - 1) / kThreads);       // uniform
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      if (k < iters) {
        const int i = min(k * kThreads + (int)threadIdx.x, count - 1);
        int row = 0, col = 0, dst = 0;
        where(i, row, col, dst);
        b[k] = static_cast<unsigned>(a.block_table[(size_t)row * a.MB + col]);
      }
    }
  };
  auto stage_store = [&](int count, const unsigned (&b)[kPer], auto&& where) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = k * kThreads + (int)threadIdx.x;
      if (i < count) {
        int row = 0, col = 0, dst = 0;
        where(i, row, col, dst);
        tbl[dst] = static_cast<int>(min(b[k], static_cast<unsigned>(a.NB - 1)));
      }
    }
  };
  unsigned tb[kPer];
  int cA = 0, cB = 0, nblk = 0;
  auto where_pair = [&](int i, int& row, int& col, int& dst) {
    row = i < cA ? sA : sB;
    col = i < cA ? i : i - cA;
    dst = (i < cA ? 0 : win) + col;
  };
  auto where_part = [&](int i, int& row, int& col, int& dst) {
    row = s;
    col = p0 * win + i;
    dst = i;
  };
  // shared-prefix mode: window 0 = the prefix's blocks (row s0), window 1 + u = the
  // first cS suffix blocks of sequence s0 + u (whatever its length: entries past it are
  // in the row and never used)
  const int cP = PREFIX ? a.pfx_len / BS : 0;
  const int cS = PREFIX ? min(win, a.MB - cP) : 1;             // >= 1: the host keeps cP < MB
  auto where_grp = [&](int i, int& row, int& col, int& dst) {
    const int k = i - cP;
    const int u = k < 0 ? 0 : k / cS;
    row = s0 + (k < 0 ? 0 : u);
    col = k < 0 ? i : cP + k % cS;
    dst = k < 0 ? i : (1 + u) * win + k % cS;
  };
  if constexpr (PREFIX) {
    stage_load(cP + gseq * cS, tb, where_grp);
  } else if constexpr (PAIRED) {
    // the host's block counts for a planned launch, else the lengths ranked above
    cA = min(blkA, win);
    cB = sB < 0 ? 0 : min(blkB, win);
    if (cA + cB > 0) stage_load(cA + cB, tb, where_pair);
  } else {
    // the window of the workgroup's partitions (one, or NW with one per wave)
    const int wend = min(seqL, (p0 + (a.wave_parts ? NW : 1)) * a.P);
    nblk = (wend - p0 * a.P + BS - 1) / BS;
    if (nblk > 0) stage_load(nblk, tb, where_part);
  }

  // Fused step: this workgroup's units' new tokens (kv head kvh).  Only the workgroup
  // that reads a sequence's last position L - 1 handles its new token (the last
  // partition, or the pair holding the sequence).  Thread t below 2 * kCh * units holds
  // one 16-byte chunk of it and copies the chunk to LDS (FP8 pools: it quantises the
  // chunk's 8 elements to E4M3 codes first, exactly as the FP8 write kernel does, and
  // LDS holds the codes).  When the token's slot is where the decode reads position
  // L - 1 (the usual case), the step covering that position substitutes the LDS copy for
  // what the cache returned and writes the patched K row chunks and V token chunks back
  // -- after its own loads brought those lines in, so the stores do not miss.  Any other
  // valid slot (read by no sequence of the call) is stored after the barrier below.
  constexpr int kSx = ElemTraits<T>::kX;                    // new-token elements per 16 bytes
  constexpr int kCh = D / kSx;                              // 16-byte new-token chunks per head
  const bool fused = a.new_slot != nullptr;
  const bool last_part = nparts - 1 < p0 + (a.wave_parts ? NW : 1);    // holds the last
  const int nun_new =
      !fused ? 0 : (PAIRED ? (sB >= 0 ? 2 : 1) : (PREFIX ? gseq : (last_part ? 1 : 0)));
  u32x4 new_val = {0u, 0u, 0u, 0u};
  int64_t new_slot = -1;
  int new_u = 0;
  const bool new_is_v = (threadIdx.x % (2 * kCh)) >= kCh;
  const int new_cc = threadIdx.x % kCh;
  const bool has_new = (int)threadIdx.x < nun_new * 2 * kCh;
  if (has_new) {
    new_u = threadIdx.x / (2 * kCh);
    const int su = PAIRED ? (new_u ? sB : sA) : (PREFIX ? s0 + new_u : s);
    const size_t src = ((size_t)su * a.Hkv + kvh) * D + (size_t)new_cc * kSx;
    new_val = load16(static_cast<const T*>(new_is_v ? a.new_v : a.new_k) + src);
    new_slot = a.new_slot[su];
  }

  if constexpr (PAIRED) {
    if constexpr (kEarly) {
      // the unit's length (device lengths: loaded before the entries, so here by now)
      const int end = max(clamp_len(a, onA ? LA : LB, BS), 1);
      const int base = tok0 + first_st * kStep;
      const bool last_known = (end - 1) / BS == first_last;
      auto entry = [&](unsigned own, int own_pos, int pos) {
        const unsigned e = pos != own_pos && last_known && pos / BS == first_last ? first_lb : own;
        return (int)min(e, (unsigned)(a.NB - 1));
      };
      auto first_kb = [&](int t, int pos) { return entry(first_k[t], step_row(base, t), pos); };
      auto first_vb = [&](int h, int pos) {
        return entry(first_v[h], base + kTpl * j + 8 * h, pos);
      };
      load_step_from(first_st, first_b, end, first_kb, first_vb);
    }
    stage_store(cA + cB, tb, where_pair);
    if (planned) {
      LA = clamp_len(a, LA, BS);
      LB = sB >= 0 ? clamp_len(a, LB, BS) : 0;
      // device lengths past the host's: stage the missing entries as well
      const int nbA = (LA + BS - 1) / BS, nbB = (LB + BS - 1) / BS;
      if (nbA > cA || nbB > cB) {
        const int xA = max(nbA - cA, 0), xB = max(nbB - cB, 0);
        auto where_more = [&](int i, int& row, int& col, int& dst) {
          row = i < xA ? sA : sB;
          col = i < xA ? cA + i : cB + i - xA;
          dst = (i < xA ? 0 : win) + col;
        };
        unsigned more[kPer];
        stage_load(xA + xB, more, where_more);
        stage_store(xA + xB, more, where_more);
      }
    }
    tok1 = __builtin_amdgcn_readfirstlane(onA ? LA : LB);
  } else if constexpr (PREFIX) {
    stage_store(cP + gseq * cS, tb, where_grp);
    tok1 = __builtin_amdgcn_readfirstlane(tok1);
    if (!pfx_wave) tblw = tbl + (1 + uidx) * win;
  } else {
    stage_store(nblk, tb, where_part);
  }

  if (has_new) {
    if constexpr (kFp8) {
      // 8 bf16 elements -> 8 codes (words 0 and 1 of new_val); a NaN keeps its sign
      const float sc = new_is_v ? a.v_quant : a.k_quant;
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t h = new_val[k >> 1];
        const float x = __uint_as_float((k & 1) ? (h & 0xFFFF0000u) : (h << 16));
        const uint32_t code = x != x ? (((__float_as_uint(x) >> 24) & 0x80u) | 0x7Fu)
                                     : e4m3_code(__fdiv_rn(x, sc));
        w[k >> 2] |= code << (8 * (k & 3));
      }
      new_val = u32x4{w[0], w[1], 0u, 0u};
      *reinterpret_cast<uint2*>(smem + 64 + (2 * new_u + (new_is_v ? 1 : 0)) * D + new_cc * 8) =
          make_uint2(w[0], w[1]);
    } else {
      store16(newkv + (2 * new_u + (new_is_v ? 1 : 0)) * D + new_cc * kX, new_val);
    }
  }
  __syncthreads();

  // slot of token `pos` of a unit whose table window `w` starts at token t0
  auto slot_of = [&](const int* w, int t0, int pos) -> int64_t {
    return (int64_t)w[(pos - t0) / BS] * BS + pos % BS;
  };
  const int64_t nslots = (int64_t)a.NB * BS;

  // position this wave takes from LDS and writes back (-1: none)
  int lm1 = -1;
  if (fused && uidx < nun_new && tok1 > tok0 && (PAIRED || PREFIX || p == nparts - 1)) {
    const int64_t sl = a.new_slot[s];
    if (sl >= 0 && sl < nslots && sl == slot_of(tblw, tok0, tok1 - 1)) lm1 = tok1 - 1;
  }
  lm1 = __builtin_amdgcn_readfirstlane(lm1);

  // a new slot that is not where position L - 1 is read from: store it here
  if (new_slot >= 0 && new_slot < nslots) {
    int Lu = PAIRED ? (new_u ? LB : LA) : seqL;
    if constexpr (PREFIX) Lu = min(max(a.context_lens[s0 + new_u] - a.pfx_len, 0), cS * BS);
    const int64_t loc =
        Lu > 0 ? slot_of(PAIRED ? tbl + new_u * win : (PREFIX ? tbl + (1 + new_u) * win : tbl),
                         (PAIRED || PREFIX) ? 0 : p0 * a.P, Lu - 1)
               : -1;
    if (new_slot != loc && kFp8) {
      uint8_t* kcw = static_cast<uint8_t*>(const_cast<void*>(a.k_cache));
      uint8_t* vcw = static_cast<uint8_t*>(const_cast<void*>(a.v_cache));
      const size_t blk = (size_t)(new_slot / BS);
      const int off = (int)(new_slot % BS);
      const int d0 = new_cc * 8;                           // first channel of the 8 codes
      if (!new_is_v) {
        uint8_t* dst = kcw + ((blk * a.Hkv + kvh) * BS + off) * D + d0;
        *reinterpret_cast<uint2*>(dst) = make_uint2(new_val[0], new_val[1]);
      } else {
        uint8_t* dst = vcw + (blk * a.Hkv + kvh) * D * BS + v_offset(off, d0, D, kXv);
#pragma unroll
        for (int k = 0; k < 8; ++k)
          dst[(size_t)k * kXv] = static_cast<uint8_t>(new_val[k >> 2] >> (8 * (k & 3)));
      }
    } else if (new_slot != loc) {
      T* kcw = const_cast<T*>(static_cast<const T*>(a.k_cache));
      T* vcw = const_cast<T*>(static_cast<const T*>(a.v_cache));
      const size_t blk = (size_t)(new_slot / BS);
      const int off = (int)(new_slot % BS);
      if (!new_is_v) {
        store16(kcw + ((blk * a.Hkv + kvh) * BS + off) * D + (size_t)new_cc * kSx, new_val);
      } else {
        T* dst = vcw + (blk * a.Hkv + kvh) * D * BS + v_offset(off, new_cc * kX, D, kXv);
        const T* e = reinterpret_cast<const T*>(&new_val);
#pragma unroll
        for (int k = 0; k < kX; ++k) dst[(size_t)k * kXv] = e[k];
      }
    }
  }

  float m_run = kNegInf;
  float l_run = 0.f;
  f32x4 acc[kNs];
#pragma unroll
  for (int i = 0; i < kNs; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // VALU math: per head, the running max and the lane's partial sum and output (lane
  // (n, j): channel 16 sl + n over the tokens of row j)
  constexpr int kVG = VG > 0 ? VG : 1;
  float mv[kVG], lv[kVG], accv[kVG][kNs];
#pragma unroll
  for (int h = 0; h < kVG; ++h) {
    mv[h] = kNegInf;
    lv[h] = 0.f;
#pragma unroll
    for (int sl = 0; sl < kNs; ++sl) accv[h][sl] = 0.f;
  }

  // ---- math of one step ---------------------------------------------------------
  auto compute_step = [&](int st, StepData<T, C, D>& b) {
    const int base = tok0 + st * kStep;
    // fused step: position L - 1 takes the new token's K/V from LDS, and the patched
    // chunks go back to the cache (their lines were just loaded)
    if constexpr (kFp8) {
      if (lm1 >= base && lm1 < base + kStep) {
        const uint8_t* nk = smem + 64 + (2 * uidx) * D;
        const uint8_t* nv = smem + 64 + (2 * uidx + 1) * D;
        uint8_t* kcw = static_cast<uint8_t*>(const_cast<void*>(a.k_cache));
        uint8_t* vcw = static_cast<uint8_t*>(const_cast<void*>(a.v_cache));
#pragma unroll
        for (int t = 0; t < Sh::kTiles; ++t) {
          const int tok = base + kTpl * (n >> 2) + 4 * t + (n & 3);
          if (tok == lm1) {
            const int phys = tblw[(tok - tok0) / BS];
            uint8_t* kp = kcw + (((size_t)phys * a.Hkv + kvh) * BS + tok % BS) * D + j * kX;
#pragma unroll
            for (int c = 0; c < kNc; ++c) {
              b.k[t][c] = *reinterpret_cast<const u32x4*>(nk + 16 * (j + 4 * c));
              store16(kp + 4 * c * kX, b.k[t][c]);
            }
          }
        }
        const int tokv = base + kTpl * j;
        const int e = lm1 - tokv;
        if (e >= 0 && e < kTpl) {
          // 16 tokens per lane; at BS 8 they are two 8-byte halves in two blocks
          const int half_tok = BS < 16 ? tokv + (e & 8) : tokv;
          const int physv = tblw[(half_tok - tok0) / BS];
          uint8_t* vp = vcw + ((size_t)physv * a.Hkv + kvh) * head_elems +
                        v_offset(BS < 16 ? 0 : tokv % BS, n, D, kXv);
#pragma unroll
          for (int sl = 0; sl < kNs; ++sl) {
            const uint32_t code = nv[16 * sl + n];
            const int sh = 8 * (e & 3);
            b.v[sl][e >> 2] = (b.v[sl][e >> 2] & ~(0xFFu << sh)) | (code << sh);
            if constexpr (BS < 16) {
              const int h = e >> 3;
              *reinterpret_cast<uint2*>(vp + (size_t)16 * sl * kXv) =
                  make_uint2(b.v[sl][2 * h], b.v[sl][2 * h + 1]);
            } else {
              store16(vp + (size_t)16 * sl * kXv, b.v[sl]);
            }
          }
        }
      }
    } else
    if (lm1 >= base && lm1 < base + kStep) {
      const T* nk = newkv + (2 * uidx) * D;
      const T* nv = newkv + (2 * uidx + 1) * D;
      T* kcw = const_cast<T*>(kc);
      T* vcw = const_cast<T*>(vc);
#pragma unroll
      for (int t = 0; t < Sh::kTiles; ++t) {
        const int tok = kBf16 ? base + 8 * (n >> 2) + 4 * t + (n & 3) : base + n;
        if (tok == lm1) {
          const int phys = tblw[(tok - tok0) / BS];
          T* kp = kcw + (((size_t)phys * a.Hkv + kvh) * BS + tok % BS) * D + j * kX;
#pragma unroll
          for (int c = 0; c < kNc; ++c) {
            b.k[t][c] = *reinterpret_cast<const u32x4*>(nk + kX * (4 * c + j));
            store16(kp + 4 * c * kX, b.k[t][c]);
          }
        }
      }
      const int tokv = base + kTpl * j;
      const int e = lm1 - tokv;
      if (e >= 0 && e < kTpl) {
        const int physv = tblw[(tokv - tok0) / BS];
        T* vp = vcw + ((size_t)physv * a.Hkv + kvh) * head_elems + v_offset(tokv % BS, n, D, kXv);
#pragma unroll
        for (int sl = 0; sl < kNs; ++sl) {
          const T val = nv[16 * sl + n];
          if constexpr (kBf16) {
            const uint32_t bitsv = __builtin_bit_cast(uint16_t, val);
            const int w = e >> 1;
            uint32_t word = b.v[sl][w];
            word = (e & 1) ? ((word & 0x0000FFFFu) | (bitsv << 16)) : ((word & 0xFFFF0000u) | bitsv);
            b.v[sl][w] = word;
          } else {
            b.v[sl][e] = __builtin_bit_cast(uint32_t, val);
          }
          store16(vp + (size_t)16 * sl * kXv, b.v[sl]);
        }
      }
    }

    const bool tail = base + kStep > tok1;
    {
      // zero V elements of tokens past the end (their weight is 0, and 0 * NaN is NaN);
      // branch-free so the loads of the other buffer keep their wait counts
      const int nv = min(max(tok1 - (base + kTpl * j), 0), kTpl);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t mask;
        if (kFp8) {
          const int r = nv - 4 * w;                          // live bytes of word w
          mask = r >= 4 ? 0xFFFFFFFFu : (r <= 0 ? 0u : (0xFFFFFFFFu >> (32 - 8 * r)));
        } else if (kBf16) {
          mask = (2 * w + 1 < nv) ? 0xFFFFFFFFu : ((2 * w < nv) ? 0x0000FFFFu : 0u);
        } else {
          mask = (w < nv) ? 0xFFFFFFFFu : 0u;
        }
#pragma unroll
        for (int sl = 0; sl < kNs; ++sl) b.v[sl][w] &= mask;
      }
    }

    if constexpr (VG > 0) {
      // Q.K^T on the VALU: lane (n, j) dots its channel chunks j + 4c of K row n (token
      // 8 (n / 4) + 4t + n % 4 of the step) with the same channels of each head's query
      // (v_dot2_f32_bf16: exact products, float32 sums); the four rows' partial dots are
      // then summed, so every row holds the step's 32 scores.
      float yv[kVG][2], mx[kVG];
#pragma unroll
      for (int h = 0; h < VG; ++h) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float part[kNc];
#pragma unroll
          for (int c = 0; c < kNc; ++c) {
            float x = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w)
              x = __builtin_amdgcn_fdot2_f32_bf16(bf16_pair(b.k[t][c], w), bf16_pair(qv[h][c], w),
                                                  x, false);
            part[c] = x;
          }
          float x = part[0];
#pragma unroll
          for (int c = 1; c < kNc; ++c) x += part[c];
          x = sum_xor32(sum_xor16(x));
          const int tok = base + 8 * (n >> 2) + 4 * t + (n & 3);
          yv[h][t] = (!tail || tok < tok1) ? x * a.scale_log2 : kNegInf;
        }
        mx[h] = row_max16(fmaxf(yv[h][0], yv[h][1]));
      }
      // online softmax per head, then P.V in float32: lane (n, j) takes the weights of
      // its V tokens 8j + i from lane 4j + i % 4 of its row (tile i / 4) and accumulates
      // them against its channels with FMAs (the weights need no bf16 split)
#pragma unroll
      for (int h = 0; h < VG; ++h) {
        const float m_new = fmaxf(mv[h], mx[h]);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = exp2_fast(mv[h] - m_use);
        const float p0 = exp2_fast(yv[h][0] - m_use);
        const float p1 = exp2_fast(yv[h][1] - m_use);
        lv[h] = lv[h] * alpha + (p0 + p1);
        mv[h] = m_new;
        float pw[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) pw[i] = lane_read(i < 4 ? p0 : p1, 20 * j + (i & 3));
#pragma unroll
        for (int sl = 0; sl < kNs; ++sl) {
          float x = accv[h][sl] * alpha;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t w = b.v[sl][i >> 1];
            x = fmaf(pw[i], __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16)), x);
          }
          accv[h][sl] = x;
        }
      }
      return;
    }

    // scores
    float y[kTpl];
    if constexpr (kFp8) {
#pragma unroll
      for (int t = 0; t < Sh::kTiles; ++t) {
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < kNc; ++c) {
          const u32x4 kk = b.k[t][c];
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16x8(kk[0], kk[1]),
                                                       __builtin_bit_cast(bf16x8, qop[2 * c]), sc,
                                                       0, 0, 0);
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16x8(kk[2], kk[3]),
                                                       __builtin_bit_cast(bf16x8, qop[2 * c + 1]),
                                                       sc, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) y[4 * t + e] = sc[e];
      }
    } else if constexpr (kBf16) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < kNc; ++c)
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b.k[t][c]),
                                                       __builtin_bit_cast(bf16x8, qop[c]), sc,
                                                       0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) y[4 * t + e] = sc[e];
      }
    } else {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < kNc; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(b.k[0][c][e]),
                                                    __uint_as_float(qop[c][e]), sc, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = sc[e];
    }

    // online softmax (base 2)
    float mx = kNegInf;
#pragma unroll
    for (int v = 0; v < kTpl; ++v) {
      const bool live = !tail || (base + kTpl * j + v < tok1);
      y[v] = live ? y[v] * a.scale_log2 : kNegInf;
      mx = fmaxf(mx, y[v]);
    }
    mx = max_xor16(mx);
    mx = max_xor32(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    float pw[kTpl];
    float psum = 0.f;
#pragma unroll
    for (int v = 0; v < kTpl; ++v) {
      pw[v] = exp2_fast(y[v] - m_use);
      psum += pw[v];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int sl = 0; sl < kNs; ++sl) acc[sl] *= alpha;

    // P.V
    if constexpr (kFp8) {
      // V bytes 8h .. 8h + 7 of lane j are tokens kTpl*j + 8h + i, whose weights are
      // pw[8h + i]; hi/lo rows as for bf16
      const bool is_hi = n < g;
      const bool is_lo = !is_hi && n < rows;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 pop;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const __bf16 hi = f32_to_bf16(pw[8 * h + v]);
          const __bf16 lo = f32_to_bf16(pw[8 * h + v] - bf16_to_f32(hi));
          pop[v] = is_hi ? hi : (is_lo ? lo : f32_to_bf16(0.f));
        }
#pragma unroll
        for (int sl = 0; sl < kNs; ++sl)
          acc[sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              e4m3x8_to_bf16x8(b.v[sl][2 * h], b.v[sl][2 * h + 1]), pop, acc[sl], 0, 0, 0);
      }
    } else if constexpr (kBf16) {
      // Rows [0, g) carry the hi weights and rows [g, 2g) the lo weights in one MFMA; a
      // wave of the shared prefix uses every column for a real row, so its hi and lo
      // weights go through two MFMAs into one accumulator.
      const bool two = PREFIX && pfx_wave;
      const bool is_hi = two ? row_live : n < g;
      const bool is_lo = !two && !is_hi && n < rows;
      bf16x8 pop, plo;
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const __bf16 hi = f32_to_bf16(pw[v]);
        const __bf16 lo = f32_to_bf16(pw[v] - bf16_to_f32(hi));
        pop[v] = is_hi ? hi : (is_lo ? lo : f32_to_bf16(0.f));
        plo[v] = (two && row_live) ? lo : f32_to_bf16(0.f);
      }
#pragma unroll
      for (int sl = 0; sl < kNs; ++sl) {
        acc[sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b.v[sl]), pop,
                                                          acc[sl], 0, 0, 0);
        if (two)
          acc[sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b.v[sl]),
                                                            plo, acc[sl], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int sl = 0; sl < kNs; ++sl)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[sl] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(b.v[sl][e]), pw[e],
                                                         acc[sl], 0, 0, 0);
    }
  };

  // ---- the wave's steps ----------------------------------------------------------------
  // Paired mode: the unit's steps are dealt in rounds of its waves' total weight, each wave
  // taking a run of rank_weight(rank) consecutive steps per round.  Other modes: st = lw,
  // lw + nw, ...
  const int nsteps = (tok1 - tok0 + kStep - 1) / kStep;
  if constexpr (PAIRED && PIPE == 2) {
    const int r0 = onA ? 0 : nA;                             // the unit's first rank
    const int cw = rank_weight(r0 + lw, NW);                 // this wave's steps per round
    const int round = __builtin_amdgcn_readfirstlane(rank_capacity(r0, r0 + nw, NW));
    const int pre = __builtin_amdgcn_readfirstlane(rank_capacity(r0, r0 + lw, NW));
    auto step_of = [&](int k) { return (k / cw) * round + pre + k % cw; };
    StepData<T, C, D>& b0 = first_b;                         // FP8: the first step, loaded above
    StepData<T, C, D> b1;
    int k = 0;
    int cur = step_of(0);                                    // the step in b0
    if (cur < nsteps) {
      if constexpr (!kEarly) load_step(cur, b0);
      int nxt = step_of(1);                                  // the step prefetched next
      for (;;) {
        load_step(nxt < nsteps ? nxt : cur, b1);
        __builtin_amdgcn_sched_barrier(0);
        compute_step(cur, b0);
        if (nxt >= nsteps) break;
        cur = nxt;
        nxt = step_of(++k + 1);
        load_step(nxt < nsteps ? nxt : cur, b0);
        __builtin_amdgcn_sched_barrier(0);
        compute_step(cur, b1);
        if (nxt >= nsteps) break;
        cur = nxt;
        nxt = step_of(++k + 1);
      }
    }
  } else if constexpr (PIPE == 2) {
    StepData<T, C, D> b0, b1;
    int st = lw;
    if (st < nsteps) {
      load_step(st, b0);
      for (;;) {
        load_step(st + nw < nsteps ? st + nw : st, b1);
        // keep the prefetch above the math: the scheduler would otherwise sink it to its use
        __builtin_amdgcn_sched_barrier(0);
        compute_step(st, b0);
        st += nw;
        if (st >= nsteps) break;
        load_step(st + nw < nsteps ? st + nw : st, b0);
        __builtin_amdgcn_sched_barrier(0);
        compute_step(st, b1);
        st += nw;
        if (st >= nsteps) break;
      }
    }
  } else {
    for (int st = lw; st < nsteps; st += nw) {
      StepData<T, C, D> b0;
      load_step(st, b0);
      compute_step(st, b0);
    }
  }

  if constexpr (VG > 0) {
    // Back to the MFMA path's register layout, which the merges below read: lane (n, j)
    // with n < g holds head n's max, a share of its sum (the whole sum in row 0, so that
    // the sum over rows is the total) and its channels 16 sl + 4j .. + 3; the other lanes
    // hold nothing (zero outputs, so the lo-row fold below adds nothing).
#pragma unroll
    for (int h = 0; h < VG; ++h) {
#pragma unroll
      for (int sl = 0; sl < kNs; ++sl) accv[h][sl] = sum_xor32(sum_xor16(accv[h][sl]));
      lv[h] = row_sum16(lv[h]);
    }
#pragma unroll
    for (int h = 0; h < VG; ++h)
      if (n == h) {
        m_run = mv[h];
        l_run = j == 0 ? lv[h] : 0.f;
      }
#pragma unroll
    for (int sl = 0; sl < kNs; ++sl)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float v = 0.f;
#pragma unroll
        for (int h = 0; h < VG; ++h) {
          const float x = lane_read(accv[h][sl], 4 * j + e);
          v = n == h ? x : v;
        }
        acc[sl][e] = v;
      }
  }

  // ---- merge the waves of the workgroup --------------------------------------------
  if ((kBf16 || kFp8) && !pfx_wave) {
    // add the lo rows [g, 2g) into the hi rows [0, g)
#pragma unroll
    for (int sl = 0; sl < kNs; ++sl)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[sl][e] += __shfl_down(acc[sl][e], g, 16);
  }
  float lsum = sum_xor16(l_run);
  lsum = sum_xor32(lsum);
  if constexpr (PREFIX) {
    // Lane (n, j) of every wave holds column n's max and sum and its channels
    // 16 sl + 4 j .. + 3, so waves merge lane by lane.  Tree merge within each unit (the
    // prefix's waves, each suffix's): in round st the waves at odd multiples of st within
    // their unit hand their registers through LDS (slot wave / 2; never two at once) to the
    // wave st below.
    constexpr int kLane = D / 4 + 2;                         // floats per lane
    float* xb = red;                                         // [NW / 2][kLane][64]
    const int rel = wave - part0;
    auto put = [&](int slot) {
      float* dst = xb + (size_t)slot * kLane * 64 + lane;
      dst[0] = m_run;
      dst[64] = lsum;
#pragma unroll
      for (int sl = 0; sl < kNs; ++sl)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(2 + 4 * sl + e) * 64] = acc[sl][e];
    };
    // (max, sum, channels) of lane `from` in `slot`, merged with this lane's
    auto take = [&](int slot, int from, float& M, float& L, f32x4 (&A)[kNs]) {
      const float* src = xb + (size_t)slot * kLane * 64 + from;
      const float mb = src[0];
      const float Mx = fmaxf(M, mb);
      if (Mx == kNegInf) return;
      const float fa = exp2_fast(M - Mx), fb = exp2_fast(mb - Mx);
      L = L * fa + src[64] * fb;
#pragma unroll
      for (int sl = 0; sl < kNs; ++sl)
#pragma unroll
        for (int e = 0; e < 4; ++e) A[sl][e] = A[sl][e] * fa + src[(2 + 4 * sl + e) * 64] * fb;
      M = Mx;
    };
    for (int st = 1; st < NW / 2; st *= 2) {
      if (rel % (2 * st) == st) put(wave >> 1);
      __syncthreads();
      if (rel % (2 * st) == 0 && rel + st < nw) take((wave + st) >> 1, lane, m_run, lsum, acc);
      __syncthreads();
    }
    // wave 0 holds the prefix's result for every column of the group, the first wave of
    // each suffix its rows: combine them per (sequence, head) and write the output
    if (wave == 0) put(0);
    __syncthreads();
    if (!pfx_wave && lw == 0 && uidx < gseq && n < g) {
      take(0, 16 * j + uidx * g + n, m_run, lsum, acc);
      const size_t row = (size_t)s * a.Hq + kvh * g + n;
#pragma unroll
      for (int sl = 0; sl < kNs; ++sl)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d = 16 * sl + 4 * j + e;
          const float o = m_run == kNegInf ? 0.f : (acc[sl][e] * a.v_scale) / lsum;
          if constexpr (kBf16)
            static_cast<uint16_t*>(a.out)[row * D + d] = bf16_bits(o);
          else
            static_cast<float*>(a.out)[row * D + d] = o;
        }
    }
    return;
  }
  if (!PAIRED && a.wave_parts) {
    // one partition per wave: lane (n, j) holds row n's channels 16 sl + 4 j .. + 3;
    // the wave writes its partition's result itself (the output when the sequence has
    // one partition, else its (max, sum, partial output) for the merge)
    if (p < nparts && n < g) {
      const size_t row = (size_t)s * a.Hq + kvh * g + n;
      if (nparts == 1) {
#pragma unroll
        for (int sl = 0; sl < kNs; ++sl)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int d = 16 * sl + 4 * j + e;
            const float o = finish_row(m_run, lsum, acc[sl][e] * a.v_scale);
            const size_t at = row * D + d;
            if constexpr (kBf16)
              static_cast<uint16_t*>(a.out)[at] = bf16_bits(o);
            else
              static_cast<float*>(a.out)[at] = o;
          }
      } else {
        float* dst = a.part_acc + (row * a.Pmax + p) * D + 4 * j;
#pragma unroll
        for (int sl = 0; sl < kNs; ++sl) {
          f32x4 v = acc[sl];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= a.v_scale;
          *reinterpret_cast<f32x4*>(dst + 16 * sl) = v;
        }
        if (j == 0) {
          a.part_ml[(row * a.Pmax + p) * 2 + 0] = m_run;
          a.part_ml[(row * a.Pmax + p) * 2 + 1] = lsum;
        }
      }
    }
    return;
  }
  const int rows_out = g;
  const int wstride = merge_words(D, g);
  float* wr = red + wave * wstride;
  if (n < rows_out) {
    if (j == 0) {
      wr[n] = m_run;
      wr[16 + n] = lsum;
    }
#pragma unroll
    for (int sl = 0; sl < kNs; ++sl)
      *reinterpret_cast<f32x4*>(wr + 32 + n * merge_stride(D) + 16 * sl + 4 * j) = acc[sl];
  }
  __syncthreads();

  // unit 0 = waves [0, nA) (all waves outside the paired mode), unit 1 = waves [nA, NW)
  const int nunits = (PAIRED && sB >= 0) ? 2 : 1;
  const bool single = nparts == 1;
  for (int idx = threadIdx.x; idx < nunits * rows_out * D; idx += kThreads) {
    const int u = idx / (rows_out * D);
    const int h = (idx % (rows_out * D)) / D;
    const int d = idx % D;
    // the unit's waves (paired mode: ranks [0, nA) are unit A, as assigned above)
    auto in_unit = [&](int w) {
      return !PAIRED || (((w % (NW / 2)) * 2 + w / (NW / 2)) < nA) == (u == 0);
    };
    const int su = PAIRED ? (u ? sB : sA) : s;
    float M = kNegInf;
    for (int w = 0; w < NW; ++w)
      if (in_unit(w)) M = fmaxf(M, red[w * wstride + h]);
    float num = 0.f, den = 0.f;
    if (M != kNegInf) {
      for (int w = 0; w < NW; ++w) {
        if (!in_unit(w)) continue;
        const float* r = red + w * wstride;
        const float f = exp2_fast(r[h] - M);
        den += f * r[16 + h];
        num += f * r[32 + h * merge_stride(D) + d];
      }
    }
    const size_t row = (size_t)su * a.Hq + kvh * g + h;
    num *= a.v_scale;
    if (single) {
      const float o = finish_row(M, den, num);
      if constexpr (kBf16)
        static_cast<uint16_t*>(a.out)[row * D + d] = bf16_bits(o);
      else
        static_cast<float*>(a.out)[row * D + d] = o;
    } else {
      a.part_acc[(row * a.Pmax + p) * D + d] = num;
      if (d == 0) {
        a.part_ml[(row * a.Pmax + p) * 2 + 0] = M;
        a.part_ml[(row * a.Pmax + p) * 2 + 1] = den;
      }
    }
  }
}

// Log-sum-exp merge of the partitions of one (sequence, query head):
//   M = max_p m_p,  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
// One wave per row.  The lanes read the partitions' (m, l) pairs side by side for M
// and the denominator; for the numerator lane i handles channels i, i + 64, ..., and
// the partitions are taken 16 at a time so that their loads are in flight together
// (each partition's weight is a wave-uniform value).
template <typename T, int D, int BS>
__global__ void __launch_bounds__(64)
reduce_partitions_kernel(const DecodeParams a) {
  const int s = blockIdx.x / a.Hq;
  const int h = blockIdx.x % a.Hq;
  const int L = clamped_len(a, s, BS);
  const int nparts = max(1, (L + a.P - 1) / a.P);
  if (nparts <= 1) return;
  const size_t row = (size_t)s * a.Hq + h;
  const float* ml = a.part_ml + row * a.Pmax * 2;
  const float* acc = a.part_acc + row * a.Pmax * D;
  const int lane = threadIdx.x;
  float M = kNegInf;
  for (int q = lane; q < nparts; q += 64) M = fmaxf(M, ml[2 * q]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  constexpr int kPer = D / 64;
  float num[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) num[i] = 0.f;
  float den = 0.f;
  if (M != kNegInf) {
    for (int q = lane; q < nparts; q += 64) den += exp2_fast(ml[2 * q] - M) * ml[2 * q + 1];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o, 64);
    constexpr int kU = 16;
    for (int q0 = 0; q0 < nparts; q0 += kU) {
      float f[kU], v[kU][kPer];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int q = min(q0 + u, nparts - 1);               // past the end: re-read, weight 0
        f[u] = q0 + u < nparts ? exp2_fast(ml[2 * q] - M) : 0.f;
#pragma unroll
        for (int i = 0; i < kPer; ++i) v[u][i] = acc[(size_t)q * D + lane + 64 * i];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int i = 0; i < kPer; ++i) num[i] += f[u] * v[u][i];
    }
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const float o = finish_row(M, den, num[i]);
    const size_t idx = row * D + lane + 64 * i;
    if constexpr (ElemTraits<T>::kBf16)
      static_cast<uint16_t*>(a.out)[idx] = bf16_bits(o);
    else
      static_cast<float*>(a.out)[idx] = o;
  }
}

constexpr int kWaves = PA_DECODE_WAVES;     // waves per workgroup, partition mode
constexpr int kPairWaves = 8;               // waves per workgroup, paired mode (at most)
constexpr int kPipe = PA_DECODE_PIPE;
constexpr size_t kMaxLds = 64 * 1024;

// Dynamic LDS of one workgroup; mirrors the layout at the top of paged_decode_kernel.
inline size_t decode_lds_bytes(bool paired, int nw, int S, int D, int BS, int P, int g,
                               int elt, bool wave_parts = false) {
  const size_t lens_words = paired ? (size_t)(S + 3) / 4 * 4 : 0;
  const size_t tbl_words =
      ((size_t)(paired ? 2 : (wave_parts ? nw : 1)) * (P / BS) + 3) / 4 * 4;
  // the merge area also holds the paired ranking's partial counts, [max(1, threads / S)][S]
  // ints <= max(S, threads)
  const size_t merge = std::max((size_t)nw * merge_words(D, g),
                                paired ? (size_t)std::max(S, nw * 64) : (size_t)0);
  return 64 + 4 * (size_t)D * elt + 4 * (lens_words + tbl_words + merge);
}

// Paired mode when every sequence is one partition, there are at least two
// sequences, the ordering stays cheap and the workgroup's LDS fits.
inline bool use_paired(const DecodeParams& a, int D, int BS, int elt) {
  return a.Pmax == 1 && a.S >= 2 && a.S <= kMaxPairedSeqs &&
         decode_lds_bytes(true, kPairWaves, a.S, D, BS, a.P, a.g, elt) <= kMaxLds;
}

// The paired mode's order of the sequences from a host copy of the lengths: the same
// keys the kernel ranks (clamped length, then lower index first), sorted on the host.
// Lengths are clamped to [0, cap], as the kernel clamps them (clamp_len).
inline void plan_pairs(int S, long cap, int BS, int step, int nw, const int32_t* host_lens,
                       PairOrder& ord) {
  uint32_t key[kMaxPairedSeqs];
  for (int t = 0; t < S; ++t) {
    const long L = std::min(std::max(0L, (long)host_lens[t]), cap);
    key[t] = (static_cast<uint32_t>(L) << 10) | static_cast<uint32_t>(1023 - t);
  }
  std::sort(key, key + S, [](uint32_t x, uint32_t y) { return x > y; });
  const int npairs = (S + 1) / 2;
  for (int r = 0; r < npairs; ++r) {
    const uint32_t kA = key[r], kB = key[S - 1 - r];
    const uint32_t sA = 1023u - (kA & 1023u);
    const uint32_t sB = r == S - 1 - r ? 0xFFFFu : 1023u - (kB & 1023u);
    const int LA = (int)(kA >> 10), LB = sB == 0xFFFFu ? 0 : (int)(kB >> 10);
    const uint32_t bA = (LA + BS - 1) / BS, bB = (LB + BS - 1) / BS;
    const uint32_t nA = split_waves(nw, (LA + step - 1) / step, (LB + step - 1) / step,
                                    sB != 0xFFFFu);
    ord.pair[r] = make_uint2(sA | sB << 16, bA | bB << 12 | nA << 24);
  }
}

inline void order_on_host(const DecodeParams& a, int BS, int step, int nw,
                          const int32_t* host_lens, PairOrder& ord) {
  plan_pairs(a.S, std::min((long)a.MB * BS, (long)a.P * a.Pmax), BS, step, nw, host_lens, ord);
}

// Compute units of the current device (queried once per device; concurrent first calls
// may both query, and store the same value).
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Paired mode's waves per workgroup.  8 (two per SIMD) keep a compute unit's loads in
// flight from one workgroup.  When the pairs outnumber the compute units and are short --
// the two longest sequences together within 32 steps -- 4 waves do better: two workgroups
// share a compute unit, so one's prologue and merge run under the other's loads
// (parallel-sampling batch: 22.5 against 26.4 us; the others slower).  The choice uses only
// max_context_len, not the host lengths, so that a call with and without them runs alike.
inline int pair_waves(const DecodeParams& a, int step, int max_context_len) {
  const long wgs = (long)(a.S + 1) / 2 * a.Hkv;
  return wgs > device_cu_count() && 2L * max_context_len <= 32L * step ? 4 : kPairWaves;
}

template <typename T, typename C, int D, int BS, int VG, int NW>
hipError_t launch_paired(const DecodeParams& a, const int32_t* host_lens, hipStream_t stream) {
  constexpr int elt = sizeof(T);
  const size_t lds = decode_lds_bytes(true, NW, a.S, D, BS, a.P, a.g, elt);
  PairOrder ord;
  if (host_lens)
    order_on_host(a, BS, StepShape<T, C, D>::kStep, NW, host_lens, ord);
  else
    for (int r = 0; r < (a.S + 1) / 2; ++r) ord.pair[r] = make_uint2(kNoPlan, 0u);
  hipLaunchKernelGGL((paged_decode_kernel<T, C, D, BS, NW, kPipe, true, false, VG>),
                     dim3((unsigned)a.Hkv, (unsigned)((a.S + 1) / 2)), dim3(NW * 64), lds,
                     stream, a, ord);
  return hipGetLastError();
}

template <typename T, typename C, int D, int BS, int VG = 0>
hipError_t launch_decode(const DecodeParams& a, const int32_t* host_lens, hipStream_t stream) {
  constexpr int elt = sizeof(T);
  if (use_paired(a, D, BS, elt)) {
    if (pair_waves(a, StepShape<T, C, D>::kStep, a.max_len) == 4)
      return launch_paired<T, C, D, BS, VG, 4>(a, host_lens, stream);
    return launch_paired<T, C, D, BS, VG, kPairWaves>(a, host_lens, stream);
  }
  const size_t lds = decode_lds_bytes(false, kWaves, a.S, D, BS, a.P, a.g, elt, a.wave_parts);
  const long groups = a.wave_parts ? (a.Pmax + kWaves - 1) / kWaves : a.Pmax;
  const long grid = (long)a.Hkv * groups * a.S;
  hipLaunchKernelGGL((paged_decode_kernel<T, C, D, BS, kWaves, kPipe, false, false, VG>),
                     dim3((unsigned)grid), dim3(kWaves * 64), lds, stream, a, NoOrder{});
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.Pmax == 1) return err;
  hipLaunchKernelGGL((reduce_partitions_kernel<T, D, BS>), dim3((unsigned)((long)a.S * a.Hq)),
                     dim3(64), 0, stream, a);
  return hipGetLastError();
}

// The prefix pass: one workgroup per (kv head, group of a.grp sequences, chunk of the
// prefix), kv head fastest, chunk slowest.
constexpr int kPrefixWaves = 8;

// LDS of a shared-prefix workgroup: control, the new tokens of up to 4 sequences, the
// table windows (the prefix, then one per sequence of the group) of P / BS entries, and
// the exchange of NW / 2 waves' registers for the merges.
inline size_t prefix_lds_bytes(int D, int BS, int P, int grp, int elt) {
  const size_t tbl_words = ((size_t)(1 + grp) * (P / BS) + 3) / 4 * 4;
  return 64 + 2 * 4 * (size_t)D * elt +
         4 * (tbl_words + (kPrefixWaves / 2) * 64 * (size_t)(D / 4 + 2));
}

// One workgroup per (kv head, group of a.grp sequences), kv head fastest.
template <typename T, int D, int BS>
hipError_t launch_prefix(const DecodeParams& a, hipStream_t stream) {
  const size_t lds = prefix_lds_bytes(D, BS, a.P, a.grp, sizeof(T));
  const long groups = (a.S + a.grp - 1) / a.grp;
  hipLaunchKernelGGL((paged_decode_kernel<T, T, D, BS, kPrefixWaves, kPipe, false, true>),
                     dim3((unsigned)((long)a.Hkv * groups)), dim3(kPrefixWaves * 64), lds,
                     stream, a, NoOrder{});
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_prefix(const DecodeParams& a, int D, int BS, hipStream_t stream) {
#define PA_CASE(DD, BB) \
  if (D == DD && BS == BB) return launch_prefix<T, DD, BB>(a, stream);
  PA_CASE(64, 8) PA_CASE(64, 16) PA_CASE(64, 32)
  PA_CASE(128, 8) PA_CASE(128, 16) PA_CASE(128, 32)
#undef PA_CASE
  return hipErrorInvalidValue;
}

// Arithmetic of the bf16 decode kernels (pa_set_decode_math).
std::atomic<int> g_decode_math{PA_MATH_MFMA};

// Group sizes the VALU math is built for.
inline bool valu_group(int g) { return g == 1 || g == 2 || g == 4; }

template <typename T, typename C>
hipError_t dispatch_decode(const DecodeParams& a, int D, int BS, const int32_t* host_lens,
                           hipStream_t stream) {
  if constexpr (std::is_same<T, uint16_t>::value && std::is_same<C, uint16_t>::value) {
    if (g_decode_math.load(std::memory_order_relaxed) == PA_MATH_VALU && valu_group(a.g)) {
#define PA_VCASE(DD, BB)                                                                    \
  if (D == DD && BS == BB)                                                                  \
    return a.g == 1   ? launch_decode<T, C, DD, BB, 1>(a, host_lens, stream)                \
           : a.g == 2 ? launch_decode<T, C, DD, BB, 2>(a, host_lens, stream)                \
                      : launch_decode<T, C, DD, BB, 4>(a, host_lens, stream);
      PA_VCASE(64, 8) PA_VCASE(64, 16) PA_VCASE(64, 32)
      PA_VCASE(128, 8) PA_VCASE(128, 16) PA_VCASE(128, 32)
#undef PA_VCASE
      return hipErrorInvalidValue;
    }
  }
#define PA_CASE(DD, BB) \
  if (D == DD && BS == BB) return launch_decode<T, C, DD, BB>(a, host_lens, stream);
  PA_CASE(64, 8) PA_CASE(64, 16) PA_CASE(64, 32)
  PA_CASE(128, 8) PA_CASE(128, 16) PA_CASE(128, 32)
#undef PA_CASE
  return hipErrorInvalidValue;
}

}  // namespace pa

// ---------------------------------------------------------------------------
// host entry points
// ---------------------------------------------------------------------------
namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int group_limit(pa_dtype dt) { return dt == PA_DTYPE_BF16 ? 8 : 16; }

pa_status check_shapes(int num_heads, int num_kv_heads, int head_dim, int block_size,
                       pa_dtype dtype) {
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (num_heads <= 0 || num_kv_heads <= 0) return PA_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads) return PA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != 8 && block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
  if (num_heads / num_kv_heads > group_limit(dtype)) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace layout: part_ml [rows][2] f32 | part_acc [rows][D] f32, rows = S * Hq * Pmax,
// each region 256-byte aligned.
struct WorkspaceLayout {
  size_t ml, acc, total;
};

WorkspaceLayout workspace_layout(int S, int Hq, int D, int pmax) {
  WorkspaceLayout w{0, 0, 0};
  if (pmax <= 1) return w;
  const size_t rows = (size_t)S * Hq * pmax;
  w.ml = 0;
  w.acc = round_up(rows * 2 * sizeof(float), 256);
  w.total = w.acc + round_up(rows * D * sizeof(float), 256);
  return w;
}


using pa::kMaxPartition;
static_assert(kMaxPartition <= (1 << 20), "a paired-mode sort key holds the length in 21 bits");

}  // namespace

// Default partition: a single partition per sequence (no merge) when the
// (sequence, kv head) pairs alone give every compute unit two workgroups;
// otherwise split so that the grid holds about four workgroups per compute
// unit, with partitions of at least 512 tokens.
extern "C" int pa_default_partition_size(int num_seqs, int num_kv_heads, int max_context_len,
                                         pa_dtype dtype) {
  (void)dtype;
  const long units = std::max(1L, (long)num_seqs * std::max(1, num_kv_heads));
  const long whole = std::max(64L, ((long)std::max(0, max_context_len) + 63) / 64 * 64);
  const long cus = pa::device_cu_count();
  if (whole <= kMaxPartition && units >= 2 * cus) return (int)whole;
  const long want_parts = std::max(1L, (4 * cus + units - 1) / units);
  long P = ((long)std::max(0, max_context_len) + want_parts - 1) / want_parts;
  P = (P + 63) / 64 * 64;
  P = std::max(512L, std::min((long)kMaxPartition, P));
  return (int)std::min(P, std::min(whole, (long)kMaxPartition));
}

extern "C" size_t pa_paged_attention_workspace_size(int num_seqs, int num_heads, int num_kv_heads,
                                                    int head_dim, int max_context_len,
                                                    int partition_size, pa_dtype dtype) {
  if (num_seqs < 0 || max_context_len < 0) return 0;
  if (check_shapes(num_heads, num_kv_heads, head_dim, 16, dtype) != PA_OK) return 0;
  const int P = partition_size ? partition_size
                               : pa_default_partition_size(num_seqs, num_kv_heads,
                                                           max_context_len, dtype);
  if (P < 64 || P > kMaxPartition || P % 64) return 0;
  const int pmax = std::max(1, (max_context_len + P - 1) / P);
  return workspace_layout(num_seqs, num_heads, head_dim, pmax).total;
}

namespace {

// Checks shared by pa_paged_attention and pa_decode_step, then the launch.
bool good_scale(float s) { return s > 0.f && s <= 3.4028234663852886e38f; }

// fp8: the caches hold E4M3 codes read with k_scale / v_scale (query and out bf16).
pa_status run_decode(void* out, const void* query, const int32_t* block_table,
                     const int32_t* context_lens, const void* k_cache, const void* v_cache,
                     const void* new_k, const void* new_v, const int64_t* new_slot,
                     int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                     int max_blocks_per_seq, int num_blocks, int max_context_len, float scale,
                     pa_dtype dtype, int partition_size, void* workspace, size_t workspace_bytes,
                     void* stream, const int32_t* host_lens, bool fp8 = false,
                     float k_scale = 1.f, float v_scale = 1.f) {
  pa_status st = check_shapes(num_heads, num_kv_heads, head_dim, block_size, dtype);
  if (st != PA_OK) return st;
  if (fp8 && dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (fp8 && (!good_scale(k_scale) || !good_scale(v_scale))) return PA_ERR_INVALID_ARG;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || max_context_len < 0)
    return PA_ERR_INVALID_ARG;
  if ((long)max_context_len > (long)max_blocks_per_seq * block_size) return PA_ERR_INVALID_ARG;
  if (partition_size != 0 &&
      (partition_size < 64 || partition_size > kMaxPartition || partition_size % 64))
    return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!out || !query || !block_table || !context_lens || !k_cache || !v_cache)
    return PA_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_table, 4) || !aligned(context_lens, 4))
    return PA_ERR_INVALID_ARG;
  if (new_slot && (!new_k || !new_v || !aligned(new_k, 16) || !aligned(new_v, 16) ||
                   !aligned(new_slot, 8)))
    return PA_ERR_INVALID_ARG;

  const int P = partition_size ? partition_size
                               : pa_default_partition_size(num_seqs, num_kv_heads,
                                                           max_context_len, dtype);
  const int pmax = std::max(1, (max_context_len + P - 1) / P);
  const long grid = (long)num_kv_heads * pmax * num_seqs;
  if (grid > 0x7FFFFFFFL || (long)num_seqs * num_heads > 0x7FFFFFFFL) return PA_ERR_INVALID_ARG;

  const WorkspaceLayout wl = workspace_layout(num_seqs, num_heads, head_dim, pmax);
  if (wl.total > 0 && (!workspace || workspace_bytes < wl.total || !aligned(workspace, 16)))
    return PA_ERR_WORKSPACE;

  pa::DecodeParams a;
  a.out = out;
  a.q = query;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.new_k = new_k;
  a.new_v = new_v;
  a.new_slot = new_slot;
  a.S = num_seqs;
  a.Hq = num_heads;
  a.Hkv = num_kv_heads;
  a.g = num_heads / num_kv_heads;
  a.MB = max_blocks_per_seq;
  a.NB = num_blocks;
  a.P = P;
  a.Pmax = pmax;
  a.max_len = max_context_len;
  a.pfx_len = 0;
  a.grp = 0;
  // Short partitions: each wave of a workgroup owns one of kWaves consecutive
  // partitions, so one prologue serves them all and no cross-wave merge is needed --
  // when the workgroups still give every compute unit two.
  {
    const long groups = (pmax + pa::kWaves - 1) / pa::kWaves;
    a.wave_parts = pmax >= 2 && (long)P * pa::kWaves <= pa::kMaxPartition &&
                   (long)num_kv_heads * num_seqs * groups >= 2L * pa::device_cu_count();
  }
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * (fp8 ? k_scale : 1.0) *
                                    1.4426950408889634);
  a.v_scale = fp8 ? v_scale : 1.f;
  a.k_quant = fp8 ? k_scale : 1.f;
  a.v_quant = fp8 ? v_scale : 1.f;
  char* ws = static_cast<char*>(workspace);
  a.part_ml = wl.total ? reinterpret_cast<float*>(ws + wl.ml) : nullptr;
  a.part_acc = wl.total ? reinterpret_cast<float*>(ws + wl.acc) : nullptr;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err =
      fp8 ? pa::dispatch_decode<uint16_t, uint8_t>(a, head_dim, block_size, host_lens, s)
      : dtype == PA_DTYPE_BF16
          ? pa::dispatch_decode<uint16_t, uint16_t>(a, head_dim, block_size, host_lens, s)
          : pa::dispatch_decode<float, float>(a, head_dim, block_size, host_lens, s);
  return err == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

extern "C" pa_status pa_set_decode_math(pa_math math) {
  if (math != PA_MATH_MFMA && math != PA_MATH_VALU) return PA_ERR_INVALID_ARG;
  pa::g_decode_math.store(math, std::memory_order_relaxed);
  return PA_OK;
}

extern "C" pa_math pa_get_decode_math(void) {
  return static_cast<pa_math>(pa::g_decode_math.load(std::memory_order_relaxed));
}

extern "C" pa_status pa_paged_attention(void* out, const void* query, const int32_t* block_table,
                                        const int32_t* context_lens, const void* k_cache,
                                        const void* v_cache, int num_seqs, int num_heads,
                                        int num_kv_heads, int head_dim, int block_size,
                                        int max_blocks_per_seq, int num_blocks,
                                        int max_context_len, float scale, pa_dtype dtype,
                                        int partition_size, void* workspace,
                                        size_t workspace_bytes, void* stream,
                                        const int32_t* host_context_lens) {
  return run_decode(out, query, block_table, context_lens, k_cache, v_cache, nullptr, nullptr,
                    nullptr, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                    max_blocks_per_seq, num_blocks, max_context_len, scale, dtype,
                    partition_size, workspace, workspace_bytes, stream, host_context_lens);
}

extern "C" pa_status pa_decode_step(void* out, const void* query, const void* key,
                                    const void* value, const int64_t* slot_mapping,
                                    const int32_t* block_table, const int32_t* context_lens,
                                    void* k_cache, void* v_cache, int num_seqs, int num_heads,
                                    int num_kv_heads, int head_dim, int block_size,
                                    int max_blocks_per_seq, int num_blocks, int max_context_len,
                                    float scale, pa_dtype dtype, int partition_size,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    const int32_t* host_context_lens) {
  if (num_seqs > 0 && (!key || !value || !slot_mapping)) return PA_ERR_INVALID_ARG;
  return run_decode(out, query, block_table, context_lens, k_cache, v_cache, key, value,
                    num_seqs > 0 ? slot_mapping : nullptr, num_seqs, num_heads, num_kv_heads,
                    head_dim, block_size, max_blocks_per_seq, num_blocks, max_context_len, scale,
                    dtype, partition_size, workspace, workspace_bytes, stream, host_context_lens);
}

// ---------------------------------------------------------------------------
// the decode step over a prefix that every sequence shares
// ---------------------------------------------------------------------------
namespace {

// Sequences per workgroup: their g query heads fill at most the 16 columns of the MFMA,
// and the 4 suffix waves split evenly among them (1, 2 or 4 sequences).
int prefix_group(int g) {
  const int most = std::min(4, 16 / g);
  return most >= 4 ? 4 : (most >= 2 ? 2 : 1);
}

}  // namespace

extern "C" pa_status pa_decode_step_shared_prefix(
    void* out, const void* query, const void* key, const void* value,
    const int64_t* slot_mapping, const int32_t* block_table, const int32_t* context_lens,
    void* k_cache, void* v_cache, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
    int block_size, int max_blocks_per_seq, int num_blocks, int max_context_len,
    int prefix_blocks, float scale, pa_dtype dtype, void* stream,
    const int32_t* host_context_lens) {
  pa_status st = check_shapes(num_heads, num_kv_heads, head_dim, block_size, dtype);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || max_context_len < 0 ||
      prefix_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  const long pfx = (long)prefix_blocks * block_size;
  if (prefix_blocks >= max_blocks_per_seq || max_context_len < pfx ||
      (long)max_context_len > (long)max_blocks_per_seq * block_size)
    return PA_ERR_INVALID_ARG;
  // one table window holds the prefix, another each private suffix
  const long window = std::max(pfx, (long)max_context_len - pfx);
  if (window > kMaxPartition) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!out || !query || !block_table || !context_lens || !k_cache || !v_cache)
    return PA_ERR_INVALID_ARG;
  if (slot_mapping && (!key || !value)) return PA_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(block_table, 4) || !aligned(context_lens, 4) ||
      (slot_mapping && (!aligned(key, 16) || !aligned(value, 16) || !aligned(slot_mapping, 8))))
    return PA_ERR_INVALID_ARG;
  if (host_context_lens)
    for (int t = 0; t < num_seqs; ++t)
      if (host_context_lens[t] < pfx || host_context_lens[t] > max_context_len)
        return PA_ERR_INVALID_ARG;
  const int g = num_heads / num_kv_heads;
  const int grp = prefix_group(g);
  if ((long)num_kv_heads * ((num_seqs + grp - 1) / grp) > 0x7FFFFFFFL) return PA_ERR_INVALID_ARG;

  pa::DecodeParams a{};
  a.out = out;
  a.q = query;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.new_k = slot_mapping ? key : nullptr;
  a.new_v = slot_mapping ? value : nullptr;
  a.new_slot = slot_mapping;
  a.S = num_seqs;
  a.Hq = num_heads;
  a.Hkv = num_kv_heads;
  a.g = g;
  a.MB = max_blocks_per_seq;
  a.NB = num_blocks;
  a.P = (int)round_up((size_t)window, 64);
  a.Pmax = 1;
  a.wave_parts = 0;
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  a.v_scale = 1.f;
  a.k_quant = a.v_quant = 1.f;
  a.pfx_len = (int)pfx;
  a.grp = grp;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t err = dtype == PA_DTYPE_BF16
                             ? pa::dispatch_prefix<uint16_t>(a, head_dim, block_size, s)
                             : pa::dispatch_prefix<float>(a, head_dim, block_size, s);
  return err == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// ---------------------------------------------------------------------------
// the decode step without a caller's workspace
// ---------------------------------------------------------------------------
// Partition workspace of pa_decode_step_noalloc: one array per GPU, in the library's
// code object.  In host code `scratch` names a host-side stand-in, never the device
// memory: kernels and copies get its device address from scratch_address().
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current GPU, looked up once per GPU (with that GPU
// current) and kept; concurrent first calls look it up twice and keep the same address.
// nullptr when the lookup fails.
void* scratch_address() {
  static std::atomic<void*> addr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return nullptr;
    addr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" pa_status pa_decode_step_noalloc(void* out, const void* query, const void* key,
                                            const void* value, const int64_t* slot_mapping,
                                            const int32_t* block_table,
                                            const int32_t* context_lens, void* k_cache,
                                            void* v_cache, int num_seqs, int num_heads,
                                            int num_kv_heads, int head_dim, int block_size,
                                            int max_blocks_per_seq, int num_blocks,
                                            int max_context_len, float scale, pa_dtype dtype,
                                            int partition_size, void* stream,
                                            const int32_t* host_context_lens) {
  if (num_seqs > 0 && (!key || !value || !slot_mapping)) return PA_ERR_INVALID_ARG;
  // the workspace this call needs (0 when no sequence is split, or for arguments that the
  // checks in run_decode reject)
  const size_t need = num_seqs > 0
                          ? pa_paged_attention_workspace_size(num_seqs, num_heads, num_kv_heads,
                                                              head_dim, max_context_len,
                                                              partition_size, dtype)
                          : 0;
  if (need > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_address();
    if (ws == nullptr) return PA_ERR_HIP;
  }
  return run_decode(out, query, block_table, context_lens, k_cache, v_cache, key, value,
                    num_seqs > 0 ? slot_mapping : nullptr, num_seqs, num_heads, num_kv_heads,
                    head_dim, block_size, max_blocks_per_seq, num_blocks, max_context_len, scale,
                    dtype, partition_size, ws, need > 0 ? PA_NOALLOC_SCRATCH_BYTES : 0, stream,
                    host_context_lens);
}

extern "C" pa_status pa_paged_attention_fp8(void* out, const void* query,
                                            const int32_t* block_table,
                                            const int32_t* context_lens, const void* k_cache,
                                            const void* v_cache, int num_seqs, int num_heads,
                                            int num_kv_heads, int head_dim, int block_size,
                                            int max_blocks_per_seq, int num_blocks,
                                            int max_context_len, float scale, float k_scale,
                                            float v_scale, pa_dtype dtype, int partition_size,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream, const int32_t* host_context_lens) {
  return run_decode(out, query, block_table, context_lens, k_cache, v_cache, nullptr, nullptr,
                    nullptr, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                    max_blocks_per_seq, num_blocks, max_context_len, scale, dtype,
                    partition_size, workspace, workspace_bytes, stream, host_context_lens, true,
                    k_scale, v_scale);
}

extern "C" pa_status pa_decode_step_fp8(void* out, const void* query, const void* key,
                                        const void* value, const int64_t* slot_mapping,
                                        const int32_t* block_table, const int32_t* context_lens,
                                        void* k_cache, void* v_cache, int num_seqs,
                                        int num_heads, int num_kv_heads, int head_dim,
                                        int block_size, int max_blocks_per_seq, int num_blocks,
                                        int max_context_len, float scale, float k_scale,
                                        float v_scale, pa_dtype dtype, int partition_size,
                                        void* workspace, size_t workspace_bytes, void* stream,
                                        const int32_t* host_context_lens) {
  if (num_seqs > 0 && (!key || !value || !slot_mapping)) return PA_ERR_INVALID_ARG;
  return run_decode(out, query, block_table, context_lens, k_cache, v_cache, key, value,
                    num_seqs > 0 ? slot_mapping : nullptr, num_seqs, num_heads, num_kv_heads,
                    head_dim, block_size, max_blocks_per_seq, num_blocks, max_context_len, scale,
                    dtype, partition_size, workspace, workspace_bytes, stream, host_context_lens,
                    true, k_scale, v_scale);
}

// ---------------------------------------------------------------------------
// the paired mode's host plan, for inspection
// ---------------------------------------------------------------------------
extern "C" pa_status pa_plan_pairs(const int32_t* host_lens, int num_seqs, int block_size,
                                   int max_len, int step_tokens, int waves, uint32_t* pairs) {
  if (!host_lens || !pairs || num_seqs < 2 || num_seqs > pa::kMaxPairedSeqs ||
      (block_size != 8 && block_size != 16 && block_size != 32) || max_len < 0 ||
      max_len > pa::kMaxPartition || step_tokens <= 0 || (waves != 4 && waves != 8))
    return PA_ERR_INVALID_ARG;
  pa::PairOrder ord;
  pa::plan_pairs(num_seqs, max_len, block_size, step_tokens, waves, host_lens, ord);
  for (int r = 0; r < (num_seqs + 1) / 2; ++r) {
    pairs[2 * r] = ord.pair[r].x;
    pairs[2 * r + 1] = ord.pair[r].y;
  }
  return PA_OK;
}
