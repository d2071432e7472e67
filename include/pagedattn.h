/*
 * pagedattn.h -- C ABI of the MI355X (gfx950) paged-KV decode library.
 *
 * The operations follow the problem statement on the pages about vLLM's
 * paged KV cache:
 *   - the KV cache is cut into fixed-size blocks; a per-sequence block table
 *     maps logical blocks to physical blocks that may sit anywhere in the pool
 *     (page "vLLM core architecture: model loading, PagedAttention principle,
 *     KV Cache management", section 2.2.1 and its table);
 *   - decode attention reads each sequence's K/V back through its block table
 *     (same page, section 2.2.2, the pseudo-code paged_attention(query,
 *     block_table, physical_kv_cache));
 *   - a new token only adds one entry to its sequence's mapping (page
 *     "vLLM core features: PagedAttention, Continuous Batching, quantization,
 *     distributed inference", section 4.1) -- here reshape_and_cache writes
 *     that token's K and V into its slot.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All array arguments are DEVICE pointers owned by the caller (the one
 *   exception, host_context_lens of the decode calls, says so); the library
 *   allocates nothing and keeps no device state between calls.
 * - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *   NULL means the null stream) and never synchronises the host.
 * - Arguments are checked on the host before anything is launched; a failed
 *   check returns a status and launches nothing.  PA_ERR_HIP reports a failed
 *   launch (hipGetLastError after the launch).
 * - dtype names the element type of query, out, key, value and both caches:
 *   PA_DTYPE_F32 (IEEE float32) or PA_DTYPE_BF16 (bfloat16).
 * - Supported shapes: head_dim D in {64, 128}; block_size BS in {8, 16, 32};
 *   num_heads a multiple of num_kv_heads with group size
 *   g = num_heads / num_kv_heads <= 8 (bf16) or <= 16 (f32).
 *   Other values return PA_ERR_UNSUPPORTED.
 * - query/out/key/value/k_cache/v_cache must be 16-byte aligned; tables
 *   4-byte aligned; slot_mapping and seq_offsets 8-byte aligned.
 *
 * Cache layout (one K pool and one V pool):
 *   k_cache: [num_blocks][num_kv_heads][BS][D]   (token-major: a token's K row of
 *            one kv head is D contiguous elements)
 *   v_cache: [num_blocks][num_kv_heads][BS / X][D][X]   (token groups: X =
 *            min(16 / element bytes, BS) consecutive tokens of one channel are
 *            one contiguous 16-byte chunk, the groups channel-major)
 * X is 8 for bf16, 4 for f32 and 16 for FP8 codes (8 at BS 8).
 * Token t of a sequence with block-table row `bt` lives in physical block
 * b = bt[t / BS] at offset o = t % BS; its K channel d is k_cache[b][h][o][d] and
 * its V channel d is v_cache[b][h][o / X][d][o % X].  One (block, kv head) tile
 * of either pool is BS * D contiguous elements.  A slot is b * BS + o.
 *
 * Device-side preconditions (not checked by the library; violating them gives
 * wrong results but no access outside the buffers passed in):
 *   block ids in [0, num_blocks); context_lens[s] <= max_context_len;
 *   slots of one reshape_and_cache call distinct; out aliases no input.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 7

typedef enum {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1,   /* null pointer, negative size, misalignment, bad length */
    PA_ERR_UNSUPPORTED = 2,   /* well-formed but not built: D, BS, dtype, group size     */
    PA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required              */
    PA_ERR_HIP = 4            /* a HIP launch failed                                     */
} pa_status;

typedef enum {
    PA_DTYPE_F32 = 0,
    PA_DTYPE_BF16 = 1,
    PA_DTYPE_FP8_E4M3 = 2     /* FP8 pools (uint8 codes): pa_copy_blocks and pa_swap_blocks
                                 only; the FP8 calls below name their pool type themselves */
} pa_dtype;

typedef enum {
    PA_MATH_MFMA = 0,         /* matrix cores (the default)                             */
    PA_MATH_VALU = 1          /* vector ALU: v_dot2_f32_bf16 scores, float32 FMA P.V    */
} pa_math;

/* Version of this ABI (PA_ABI_VERSION of the build). */
int pa_abi_version(void);

/* Static, human-readable name of a status code. */
const char* pa_status_string(pa_status status);

/*
 * Partition length (tokens) pa_paged_attention uses for these sizes when the
 * caller passes partition_size = 0.  Always a multiple of 64 in [64, 8192].
 * When num_seqs * num_kv_heads gives every compute unit of the current
 * device two workgroups and max_context_len <= 8192, one partition covers the
 * longest sequence (no merge step); otherwise the context is split so that
 * the grid holds about four workgroups per compute unit, with partitions of
 * at least 512 tokens.  The value depends on the current device's compute
 * unit count, so size the workspace on the device that runs the call.
 */
int pa_default_partition_size(int num_seqs, int num_kv_heads, int max_context_len,
                              pa_dtype dtype);

/*
 * Bytes of workspace pa_paged_attention needs (0 when every sequence fits in
 * one partition).  partition_size = 0 selects pa_default_partition_size.
 * Returns 0 for arguments pa_paged_attention would reject.
 */
size_t pa_paged_attention_workspace_size(int num_seqs, int num_heads, int num_kv_heads,
                                         int head_dim, int max_context_len,
                                         int partition_size, pa_dtype dtype);

/*
 * Decode attention over a paged KV cache (one query token per sequence).
 *
 * For sequence s (length L = context_lens[s]) and query head h with KV head
 * kvh = h / g:
 *   z_t   = scale * sum_d query[s][h][d] * K_s[t][kvh][d],   t in [0, L)
 *   out[s][h] = sum_t softmax(z)_t * V_s[t][kvh]
 * where K_s/V_s is the sequence reassembled through block_table (the result
 * is the attention over the whole reassembled sequence; the library combines
 * block-wise partial results exactly with a running max and sum).  L = 0
 * gives out = 0.  out is rounded to dtype (round to nearest even for bf16).
 *
 *   out, query     [num_seqs][num_heads][head_dim], contiguous
 *   block_table    [num_seqs][max_blocks_per_seq] int32, row stride
 *                  max_blocks_per_seq; entries past ceil(L / BS) are never read
 *   context_lens   [num_seqs] int32
 *   k_cache/v_cache  layouts above, num_blocks blocks
 *   max_context_len  host-side upper bound of context_lens (sizes the grid;
 *                  must be <= max_blocks_per_seq * block_size)
 *   partition_size 0 = default, else a multiple of 64 in [64, 8192]: each
 *                  sequence is split into partitions of this many tokens that
 *                  run in parallel; sequences longer than one partition are
 *                  merged by a second, log-sum-exp reduce kernel on the same
 *                  stream
 *   workspace      device scratch of at least
 *                  pa_paged_attention_workspace_size(...) bytes, 16-byte
 *                  aligned, any contents; may be NULL when that size is 0.
 *                  It holds per-partition (max, sum, partial output) rows
 *                  between the two kernels.  Two calls in flight at once must
 *                  not share a workspace.
 *   host_context_lens  optional HOST copy of context_lens ([num_seqs] int32,
 *                  read during the call only), or NULL.  When every sequence
 *                  is one partition, the kernel gives each workgroup the r-th
 *                  longest and the r-th shortest sequence; with this copy the
 *                  library sorts the lengths on the host and passes the order
 *                  with the launch, so that the workgroups need not rank the
 *                  lengths themselves.  The device context_lens still decide
 *                  every length the kernel reads; a host copy that differs
 *                  from them changes only how the work is spread, not the
 *                  result's accuracy.  When it matches, the output is the same
 *                  bit for bit as with NULL.
 */
pa_status pa_paged_attention(void* out, const void* query, const int32_t* block_table,
                             const int32_t* context_lens, const void* k_cache,
                             const void* v_cache, int num_seqs, int num_heads,
                             int num_kv_heads, int head_dim, int block_size,
                             int max_blocks_per_seq, int num_blocks, int max_context_len,
                             float scale, pa_dtype dtype, int partition_size,
                             void* workspace, size_t workspace_bytes, void* stream,
                             const int32_t* host_context_lens);

/*
 * Write path: store each new token's K and V into its slot.
 *
 *   key, value     [num_tokens][num_kv_heads][head_dim], contiguous
 *   slot_mapping   [num_tokens] int64; slot = physical_block * BS + offset.
 *                  A negative slot skips that token (padding); a slot at or
 *                  past num_blocks * BS is skipped as well.
 *   k_cache, v_cache  pools in the layouts above (written in place)
 * The copy is bit-exact; nothing outside the written slots changes.
 */
pa_status pa_reshape_and_cache(const void* key, const void* value, const int64_t* slot_mapping,
                               void* k_cache, void* v_cache, int num_tokens, int num_kv_heads,
                               int head_dim, int block_size, int num_blocks, pa_dtype dtype,
                               void* stream);

/*
 * One decode step in a single launch: store each sequence's new token in its
 * slot, then decode attention over the caches that now hold it.  The result
 * (out and both caches) is the same as
 *   pa_reshape_and_cache(key, value, slot_mapping, k_cache, v_cache, num_seqs, ...)
 *   followed by pa_paged_attention(out, query, ...).
 *
 *   key, value     [num_seqs][num_kv_heads][head_dim], contiguous: the K and V
 *                  of the token each sequence appends in this step
 *   slot_mapping   [num_seqs] int64: slot of that token, which must be the
 *                  slot of position context_lens[s] - 1 of sequence s (the
 *                  block-table entry block_table[s][(L - 1) / BS] at offset
 *                  (L - 1) % BS), or negative to write nothing for s
 *   k_cache, v_cache  written in place (the new tokens' slots only)
 *   other arguments as in pa_paged_attention
 * Preconditions: a slot written for sequence s lies in a block that no other
 * sequence of the call reads or writes (after copy-on-write a sequence's last
 * block is its own); a slot other than position L - 1's is read by no sequence
 * of the call.  The workgroup that reads position L - 1 of s writes s's new
 * token: it uses the token for that position directly and stores it back
 * together with the neighbouring tokens of the same 16-byte chunks, unchanged.
 */
pa_status pa_decode_step(void* out, const void* query, const void* key, const void* value,
                         const int64_t* slot_mapping, const int32_t* block_table,
                         const int32_t* context_lens, void* k_cache, void* v_cache,
                         int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                         int block_size, int max_blocks_per_seq, int num_blocks,
                         int max_context_len, float scale, pa_dtype dtype, int partition_size,
                         void* workspace, size_t workspace_bytes, void* stream,
                         const int32_t* host_context_lens);

/*
 * The decode step when every sequence of the call starts with the same shared prefix:
 * the first prefix_blocks entries of every block-table row name the same physical
 * blocks (one system prompt stored once and shared by reference: page "vLLM core
 * inference engine", section 2.2; prefix caching, page "vLLM core features", section
 * 4.6).  The result (out and both caches) is that of pa_decode_step.  One launch; a
 * workgroup takes a group of 1, 2 or 4 consecutive sequences (their query heads side by
 * side fill at most the 16 columns of one matrix-core operand): half of its waves read
 * the shared positions [0, P), P = prefix_blocks * block_size, once for the whole group,
 * the other half the group's private positions [P, L), and the two parts of each row are
 * combined with a log-sum-exp merge.  Each prefix block is read once per group instead of
 * once per sequence.  Nothing is allocated and no workspace is needed.
 *
 *   prefix_blocks  shared leading blocks, >= 1 and < max_blocks_per_seq
 *   slot_mapping   as in pa_decode_step, or NULL for decode attention alone (no token
 *                  appended; key and value are then ignored)
 *   dtype          PA_DTYPE_BF16 or PA_DTYPE_F32
 *   other arguments as in pa_decode_step
 * P and the longest suffix, max_context_len - P, must each be at most 8192 tokens
 * (PA_ERR_UNSUPPORTED otherwise: use pa_decode_step).
 * Preconditions (device side): every context_lens[s] >= P, and > P when a token is
 * appended for s (a new token goes to a private block).  With host_context_lens, a
 * length below P or above max_context_len is rejected (PA_ERR_INVALID_ARG) before any
 * launch.
 */
pa_status pa_decode_step_shared_prefix(void* out, const void* query, const void* key,
                                       const void* value, const int64_t* slot_mapping,
                                       const int32_t* block_table, const int32_t* context_lens,
                                       void* k_cache, void* v_cache, int num_seqs,
                                       int num_heads, int num_kv_heads, int head_dim,
                                       int block_size, int max_blocks_per_seq, int num_blocks,
                                       int max_context_len, int prefix_blocks, float scale,
                                       pa_dtype dtype, void* stream,
                                       const int32_t* host_context_lens);

/*
 * pa_decode_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It takes no workspace: when the call needs one (sequences split into
 * partitions) it uses a fixed scratch array inside the library,
 * PA_NOALLOC_SCRATCH_BYTES on each GPU, held from the first call on that GPU
 * until the process ends.  The call itself allocates nothing.
 *   - Arguments, result, caches and preconditions as pa_decode_step (same
 *     kernels; out and the caches are the same bit for bit).
 *   - A call needing more than PA_NOALLOC_SCRATCH_BYTES
 *     (pa_paged_attention_workspace_size) returns PA_ERR_WORKSPACE and
 *     launches nothing; pass a larger partition_size or use pa_decode_step.
 *   - Every call on one GPU shares that GPU's scratch, and the array keeps
 *     what the last call left (nothing in it needs to start at zero: each
 *     call writes every partial result it reads).  Calls that overlap on one
 *     GPU (other streams, other host threads) race on it and give wrong
 *     results: order them, e.g. on one stream.
 *   - PA_ERR_HIP if the scratch array's address cannot be obtained.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
pa_status pa_decode_step_noalloc(void* out, const void* query, const void* key,
                                 const void* value, const int64_t* slot_mapping,
                                 const int32_t* block_table, const int32_t* context_lens,
                                 void* k_cache, void* v_cache, int num_seqs, int num_heads,
                                 int num_kv_heads, int head_dim, int block_size,
                                 int max_blocks_per_seq, int num_blocks, int max_context_len,
                                 float scale, pa_dtype dtype, int partition_size, void* stream,
                                 const int32_t* host_context_lens);

/*
 * Paged prefill: causal attention of a chunk of new query tokens per sequence
 * over the sequence's paged K/V (the chunk's own K/V already stored, e.g. by
 * pa_reshape_and_cache).  A request's earlier context -- a system prompt kept
 * in shared blocks, a cached prefix (page "vLLM core inference engine",
 * section 2.2; page "vLLM core features", sections 4.2 and 4.6) -- is read
 * through the block table and only the new tokens are computed.
 *
 * Sequence s owns query rows query_start_loc[s] .. query_start_loc[s+1] - 1
 * (n tokens, n <= L = context_lens[s]); row i is the token at position
 * p = L - n + i and
 *   out[row][h] = sum_{t <= p} softmax_t(scale * query[row][h] . K_s[t][kvh]) V_s[t][kvh]
 * with kvh = h / g.  n = 1 gives the decode result.
 *
 *   out, query       [num_query_tokens][num_heads][head_dim], contiguous
 *   query_start_loc  [num_seqs + 1] int32, non-decreasing, query_start_loc[0] = 0,
 *                    query_start_loc[num_seqs] = num_query_tokens
 *   max_query_len    host-side upper bound of the chunk lengths (sizes the grid)
 *   scale            softmax scale; must be positive and finite (else
 *                    PA_ERR_INVALID_ARG): the kernel takes the row maximum on the
 *                    raw scores and applies the scale in the exponent
 *   other arguments as in pa_paged_attention; group size g = num_heads /
 *   num_kv_heads must divide 128 (1, 2, 4, 8, 16)
 * Values outside these ranges are clamped on the device (rows that fall outside
 * [0, num_query_tokens) are not written).
 */
pa_status pa_paged_prefill(void* out, const void* query, const int32_t* query_start_loc,
                           const int32_t* block_table, const int32_t* context_lens,
                           const void* k_cache, const void* v_cache, int num_seqs, int num_heads,
                           int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                           int num_blocks, int num_query_tokens, int max_query_len, float scale,
                           pa_dtype dtype, void* stream);

/*
 * Copy-on-write: make physical block dst a copy of physical block src (every
 * kv head, K and V), for each pair of block_mapping.  A sequence that appends
 * into a block it shares with others (parallel samples, beams, a common prompt:
 * page "vLLM core features", section 4.1; page "vLLM core architecture",
 * section 2.2.1) first gets a private copy of it.
 *
 *   block_mapping  [num_pairs][2] int64: (src, dst).  Destinations must be
 *                  distinct and none may be a source of the same call (the
 *                  copies run in parallel).  A pair with a block outside
 *                  [0, num_blocks) is skipped.
 *   k_cache, v_cache  pools in the layouts above (written in place)
 *   dtype          the pools' element type; PA_DTYPE_FP8_E4M3 for FP8 pools
 * The copy is bit-exact; blocks that are not destinations do not change.
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping,
                         int num_pairs, int num_kv_heads, int head_dim, int block_size,
                         int num_blocks, pa_dtype dtype, void* stream);

/*
 * FP8 K/V cache.  The pages list FP8 E4M3 as an 8-bit float precision that
 * needs about half the memory of 16-bit formats (page "vLLM core features",
 * section 4.3, the table of quantisation formats); here it is the storage
 * format of the K/V pools, which halves the bytes a decode step reads.
 *
 * Format: OCP FP8 E4M3 codes, one byte per element (bias 7, subnormals
 * m * 2^-9, S.1111.111 = NaN, no infinities, largest finite 448).  One scale
 * per tensor: the stored code of a K element x is the E4M3 value nearest to
 * the float32 quotient x / k_scale (ties to the even code; magnitudes above
 * 448 and infinities saturate to +-448; a NaN x gives the NaN code with the
 * sign of x), and it reads back as
 * E4M3(code) * k_scale; likewise V with v_scale.  k_scale and v_scale must be
 * finite and > 0 (else PA_ERR_INVALID_ARG).
 *
 * Layout: the pools above with 1-byte elements:
 *   k_cache: [num_blocks][num_kv_heads][BS][D] uint8
 *   v_cache: [num_blocks][num_kv_heads][BS / X][D][X] uint8, X = min(16, BS)
 */

/*
 * Write path into FP8 pools: quantise each new token's K and V (given in
 * dtype, f32 or bf16) with k_scale / v_scale and store the codes in its slot.
 * Slots as in pa_reshape_and_cache (negative or past the pool: skipped).
 * The codes are bit-exact functions of the inputs and scales.
 */
pa_status pa_reshape_and_cache_fp8(const void* key, const void* value,
                                   const int64_t* slot_mapping, void* k_cache, void* v_cache,
                                   int num_tokens, int num_kv_heads, int head_dim,
                                   int block_size, int num_blocks, pa_dtype dtype,
                                   float k_scale, float v_scale, void* stream);

/*
 * Decode attention over FP8 pools: the result of pa_paged_attention over the
 * dequantised K and V.  query and out are bf16 (dtype must be PA_DTYPE_BF16;
 * f32 returns PA_ERR_UNSUPPORTED).  The codes are widened to bf16 exactly on
 * load; k_scale joins the softmax scale and v_scale multiplies the output.
 * partition_size, when not 0, must also be a multiple of 64; the workspace is
 * sized by pa_paged_attention_workspace_size with dtype PA_DTYPE_BF16.  Other
 * arguments as in pa_paged_attention.
 */
pa_status pa_paged_attention_fp8(void* out, const void* query, const int32_t* block_table,
                                 const int32_t* context_lens, const void* k_cache,
                                 const void* v_cache, int num_seqs, int num_heads,
                                 int num_kv_heads, int head_dim, int block_size,
                                 int max_blocks_per_seq, int num_blocks, int max_context_len,
                                 float scale, float k_scale, float v_scale, pa_dtype dtype,
                                 int partition_size, void* workspace, size_t workspace_bytes,
                                 void* stream, const int32_t* host_context_lens);

/*
 * One decode step over FP8 pools in a single launch: quantise each sequence's
 * new token (bf16 key/value, with k_scale / v_scale, codes identical to
 * pa_reshape_and_cache_fp8) into its slot, then decode attention as
 * pa_paged_attention_fp8 over the pools that now hold it.  The result is the
 * same as those two calls in a row.  Slot rules and preconditions as in
 * pa_decode_step; other arguments as in pa_paged_attention_fp8.
 */
pa_status pa_decode_step_fp8(void* out, const void* query, const void* key, const void* value,
                             const int64_t* slot_mapping, const int32_t* block_table,
                             const int32_t* context_lens, void* k_cache, void* v_cache,
                             int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                             int block_size, int max_blocks_per_seq, int num_blocks,
                             int max_context_len, float scale, float k_scale, float v_scale,
                             pa_dtype dtype, int partition_size, void* workspace,
                             size_t workspace_bytes, void* stream,
                             const int32_t* host_context_lens);

/*
 * Swapping: make block d of the destination pools a copy of block s of the
 * source pools, for each pair of block_mapping.  When GPU memory runs short
 * the scheduler moves a request's KV out block by block and can write it to
 * CPU memory, and brings it back later (page "vLLM core architecture",
 * section 2.3.2): swap-out is a call with the HBM pools as source and pools
 * in pinned host memory as destination, swap-in the reverse (into whatever
 * free blocks the allocator chose).  Both pairs of pools have the layout
 * above; they may hold different numbers of blocks.
 *
 *   src_k, src_v   source pools, src_num_blocks blocks
 *   dst_k, dst_v   destination pools, dst_num_blocks blocks (written in place)
 *   block_mapping  [num_pairs][2] int64 (source block, destination block);
 *                  destinations distinct; a pair naming a block outside its
 *                  pool is skipped
 *   dtype          element type of all four pools (PA_DTYPE_FP8_E4M3: codes)
 * Each of the four pools and block_mapping must be device memory or pinned
 * host memory mapped for the device (hipHostMalloc, a pinned torch tensor);
 * anything else -- pageable host memory in particular -- returns
 * PA_ERR_INVALID_ARG before any launch.  The GPU moves the data itself in
 * one launch, through the host memory's device mapping.  The copy is
 * bit-exact; nothing else in the destination changes.
 */
pa_status pa_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                         const int64_t* block_mapping, int num_pairs, int num_kv_heads,
                         int head_dim, int block_size, int src_num_blocks, int dst_num_blocks,
                         pa_dtype dtype, void* stream);

/*
 * Diagnostic read path: reassemble every sequence's K and V through its block
 * table into contiguous token-major arrays (bit-exact copies).
 *
 *   k_out, v_out   [sum_s context_lens[s]][num_kv_heads][head_dim]
 *   seq_offsets    [num_seqs] int64, row of k_out/v_out where sequence s
 *                  starts (the exclusive prefix sum of context_lens)
 *   other arguments as in pa_paged_attention
 */
pa_status pa_gather_kv(void* k_out, void* v_out, const int64_t* seq_offsets,
                       const int32_t* block_table, const int32_t* context_lens,
                       const void* k_cache, const void* v_cache, int num_seqs,
                       int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                       int num_blocks, int max_context_len, pa_dtype dtype, void* stream);

/*
 * Arithmetic of the bf16 decode (process-wide; for measurement and diagnostics).
 * The attention of "core architecture" section 2.2.2 needs two small products per
 * step of a (block, kv head): the g query rows of a group against the step's K rows,
 * and the softmax weights against its V rows.  With PA_MATH_MFMA (the default) both
 * run on the matrix cores; with PA_MATH_VALU they run on the vector ALU (bf16 dot
 * products for the scores, float32 FMAs with unsplit weights for P.V), with the same
 * loads, partitioning and merges.  The VALU form serves pa_paged_attention,
 * pa_decode_step and pa_decode_step_noalloc on bf16 pools with group size 1, 2 or 4;
 * every other call and shape runs on the matrix cores whatever is set.  Both forms
 * meet the same accuracy bound; their results differ in rounding only.  A call takes
 * the value set when it is made.  Returns PA_ERR_INVALID_ARG for another value.
 */
pa_status pa_set_decode_math(pa_math math);
pa_math pa_get_decode_math(void);

/*
 * Diagnostic read-bandwidth probe (not a step of the decode path).  A paged decode
 * streams K and V as whole (block, kv head) tiles scattered through the pool; this
 * call reads such pieces and keeps only a checksum, so its rate is the ceiling the
 * decode's loads can reach on the device (in order: a streaming read; shuffled:
 * the paged gather).
 *
 *   buf            device buffer read from
 *   piece_offsets  [num_pieces] int64, device: byte offset of piece i in buf
 *                  (16-byte aligned); every piece [off, off + piece_bytes) must
 *                  lie inside buf (not checked: the library does not know its size)
 *   piece_bytes    bytes per piece, a multiple of 4096
 *   workgroups     workgroups of 256 threads; workgroup b reads pieces
 *                  [in_flight * b, in_flight * (b + 1)), then the same group
 *                  workgroups * in_flight pieces further on, and so on
 *   in_flight      4, 8 or 16: pieces whose 16-byte loads each thread issues
 *                  before using any of them
 *   nontemporal    0: default-policy loads; 1: streaming (nt) loads, the policy of
 *                  the paged decode's V loads
 *   sink           [workgroups * 256] uint32, device: written with checksums
 * Returns PA_ERR_INVALID_ARG / PA_ERR_UNSUPPORTED for bad arguments (nothing
 * launched).
 */
pa_status pa_read_probe(const void* buf, const int64_t* piece_offsets, int num_pieces,
                        int piece_bytes, int workgroups, int in_flight, int nontemporal,
                        uint32_t* sink, void* stream);

/*
 * Diagnostic co-execution probe (not a step of any path).  A SIMD of gfx950 can run
 * matrix-core (MFMA) and vector-ALU work at once; this call measures how much of the
 * two overlaps, within a wave and between the waves of a SIMD.  Every wave
 * runs `iters` iterations of its work -- MFMA work: 8 independent chains of 16x16x32
 * bf16 MFMAs; VALU work: 32 fused multiply-adds over 8 independent chains -- and the
 * launch's time (events on `stream`) is the answer:
 *   mode 0  MFMA work only            mode 1  VALU work only
 *   mode 2  both in every wave, one MFMA then four FMAs
 *   mode 3  MFMA work in the first half of the workgroup's waves, VALU work in the
 *           second half (wave w runs on SIMD w % 4, so at 8 waves per workgroup every
 *           SIMD runs one wave of each kind)
 *   mode 4  placement check: no work; every thread writes the index (0..3) of the SIMD
 *           its wave runs on, so that the placement mode 3 relies on can be seen
 *   workgroups           >= 1
 *   waves_per_workgroup  4 (one wave per SIMD) or 8 (two)
 *   iters                1 .. 2^20
 *   out                  [workgroups * waves_per_workgroup * 64] float, device:
 *                        written with one value per thread
 * Returns PA_ERR_INVALID_ARG for bad arguments (nothing launched).
 */
pa_status pa_coexec_probe(int mode, int workgroups, int waves_per_workgroup, int iters,
                          float* out, void* stream);

/*
 * The paired mode's plan made on the host (diagnostic; no GPU work, callable without a
 * GPU).  When every sequence of a decode call is one partition, a workgroup takes the r-th
 * longest and the r-th shortest sequence of a kv head and splits its waves between the
 * two in proportion to their steps, so that every workgroup carries about the same tokens.
 * The pages define the attention (page "vLLM core architecture", section 2.2.2); this
 * pairing is the library's own schedule of it.  With host_context_lens the decode calls
 * make exactly this plan; without it the kernel derives the same pairs from context_lens.
 *   host_lens    [num_seqs] int32, host memory; each clamped to [0, max_len]
 *   num_seqs     2 .. 512
 *   block_size   8, 16 or 32
 *   max_len      the clamp, 0 .. 8192 (the decode uses the partition size)
 *   step_tokens  positions per step of the kernel (32 for bf16, 16 for f32, 64 for FP8)
 *   waves        4 or 8 per workgroup (rank r of a workgroup's waves takes 3 steps for
 *                every 2 of rank r + 1 at 8 waves when r is even, 1 each at 4)
 *   pairs        [2 * ((num_seqs + 1) / 2)] uint32, host memory, written: for pair r,
 *                pairs[2r] = sA | sB << 16 (sA the r-th longest sequence, sB the r-th
 *                shortest, ties to the lower index; sB = 0xFFFF for the middle sequence
 *                of an odd count) and pairs[2r + 1] = blocks of sA | blocks of sB << 12 |
 *                waves of sA << 24 (the split that evens the two units' steps per unit of
 *                wave weight; each unit of a pair keeps at least one wave)
 * Returns PA_ERR_INVALID_ARG for bad arguments (nothing written).
 */
pa_status pa_plan_pairs(const int32_t* host_lens, int num_seqs, int block_size, int max_len,
                        int step_tokens, int waves, uint32_t* pairs);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
