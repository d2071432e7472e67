"""Plain, slow CPU oracle for paged decode attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
calls it, shares no code with it, and must fail loudly rather than fall back
to it.

What is computed, and where the pages define it
-----------------------------------------------
* KV cache in blocks: every sequence's keys and values are cut into
  fixed-size blocks of ``block_size`` tokens; a logical block and a physical
  block hold the same number of tokens; a per-sequence block table maps
  logical block numbers to physical blocks, which may sit anywhere in the
  pool ("core architecture" page, section 2.2.1 and its table;
  "core features" page, section 4.1).
* Attention over a paged cache: the result is attention of the query over the
  complete K/V sequence put back together through the block table
  ("core architecture" page, section 2.2.2, the sentence before the
  pseudo-code).  The pages never write the formula out; this oracle takes the
  standard scaled dot-product softmax attention with the caller's ``scale``,
  and no mask other than the sequence length.  The pseudo-code's per-block
  ``+=`` is read as the exact softmax over the whole sequence, since the same
  section defines the result through the reassembled sequence.
* Appending a token writes one slot: a newly generated token costs one more
  entry in its sequence's mapping, nothing is moved ("core features" page,
  section 4.1).  The slot of a token is physical_block * block_size +
  offset_in_block, and reshape_and_cache scatters each new token's K and V
  into its slot.
* Grouped query heads: query head h reads KV head h // (Hq / Hkv).  The pages
  are silent on grouping; contiguous groups are the plainest reading.

Cache layout (the library's boundary format; the pages show only that a
physical block yields its k and v):
* k_cache: [num_blocks, Hkv, block_size, D] (token-major: one token's K row of
  one kv head is contiguous);
* v_cache: [num_blocks, Hkv, block_size / X, D, X] with X = min(16 bytes / element,
  block_size): the block's tokens in groups of X, each group channel-major (X
  consecutive tokens of one channel are one 16-byte chunk).
Element (token t, kv head h, channel d) of sequence s lives at
``k_cache[b, h, t % BS, d]`` and ``v_cache[b, h, (t % BS) // X, d, t % X]`` with
``b = block_table[s, t // BS]``.

Precision: inputs are float32 arrays or bfloat16 bit patterns (uint16);
everything is decoded exactly to float64 and computed in float64 with NumPy's
matmul, exp and sum as the only library steps.  Nothing is rounded back.

Pins: the checks that tie these functions to the pages and to independent
formulations live in the test suite (dense brute force over the never-paged
sequence, block-permutation, sharing and block-size invariance, closed forms,
a hand-worked fixture, and a per-element gather loop).  Every function below
is pinned by at least one of them.
"""
from __future__ import annotations

import math

import numpy as np

ELEMENT_BYTES = {"f32": 4, "bf16": 2}


# ---------------------------------------------------------------------------
# element decoding and cache layout
# ---------------------------------------------------------------------------
def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of each element.

    bfloat16 is the upper half of an IEEE float32: widening the 16-bit pattern
    to 32 bits with zeros below gives the same number as a float32.
    """
    if dtype == "bf16":
        bits = np.ascontiguousarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def chunk_elems(dtype: str) -> int:
    """Elements in one 16-byte chunk."""
    return 16 // ELEMENT_BYTES[dtype]


def k_cache_shape(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int,
                  dtype: str) -> tuple:
    return (num_blocks, num_kv_heads, block_size, head_dim)


def v_group(block_size: int, element_bytes: int) -> int:
    """Tokens per V group: one 16-byte chunk of a channel, at most the block."""
    return min(16 // element_bytes, block_size)


def v_cache_shape(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int,
                  dtype: str) -> tuple:
    X = v_group(block_size, ELEMENT_BYTES[dtype])
    return (num_blocks, num_kv_heads, block_size // X, head_dim, X)


# ---------------------------------------------------------------------------
# write path: reshape_and_cache
# ---------------------------------------------------------------------------
def reshape_and_cache(key: np.ndarray, value: np.ndarray, slot_mapping: np.ndarray,
                      k_cache: np.ndarray, v_cache: np.ndarray, inplace: bool = False):
    """Pools with token i's K/V stored at slot_mapping[i] (copies unless ``inplace``).

    key, value: [T, Hkv, D].  A negative slot means "no write" (padding).
    Slots of one call must be distinct and inside the pool.
    """
    k_new = k_cache if inplace else k_cache.copy()
    v_new = v_cache if inplace else v_cache.copy()
    NB, Hkv, BS, D = k_cache.shape
    slots = np.asarray(slot_mapping, dtype=np.int64)
    live = np.nonzero(slots >= 0)[0]
    assert len(np.unique(slots[live])) == len(live), "slots of one call must be distinct"
    assert (slots[live] < NB * BS).all(), "slot outside the pool"
    X = v_cache.shape[4]
    blk, off = slots[live] // BS, slots[live] % BS
    k_new[blk, :, off, :] = key[live]
    v_new[blk, :, off // X, :, off % X] = value[live]
    return k_new, v_new


# ---------------------------------------------------------------------------
# copy-on-write: whole physical blocks
# ---------------------------------------------------------------------------
def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, block_mapping: np.ndarray,
                inplace: bool = False):
    """Pools where physical block dst holds a copy of block src, for every (src, dst).

    Several sequences may point at one physical block (parallel samples of one
    prompt, beams, a shared system prompt: "core features" page, section 4.1;
    "core architecture" page, section 2.2.1).  A sharer that appends into such
    a block first gets a private copy of it; this is that copy, every kv head
    of K and V.  Destinations must be distinct and none may be a source, so the
    order of the copies does not matter.
    """
    pairs = np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2)
    src, dst = pairs[:, 0], pairs[:, 1]
    assert len(np.unique(dst)) == len(dst), "destinations must be distinct"
    assert not (set(dst.tolist()) & set(src.tolist())), "a destination is also a source"
    k_new = k_cache if inplace else k_cache.copy()
    v_new = v_cache if inplace else v_cache.copy()
    k_new[dst] = k_cache[src]
    v_new[dst] = v_cache[src]
    return k_new, v_new


# ---------------------------------------------------------------------------
# swapping: whole blocks between two pools (HBM and host memory)
# ---------------------------------------------------------------------------
def swap_blocks(src_k: np.ndarray, src_v: np.ndarray, dst_k: np.ndarray, dst_v: np.ndarray,
                block_mapping: np.ndarray, inplace: bool = False):
    """Destination pools where block d holds a copy of source block s, for every (s, d).

    When GPU memory runs short the scheduler moves a request's KV out block by
    block, not the request as a whole, and can write the blocks to CPU memory;
    they come back when there is room ("core architecture" page, section
    2.3.2).  Swap-out is this copy from the HBM pool into a host pool, swap-in
    the copy back (into whatever free blocks the allocator picks).  The two
    pools have the same layout and may hold different numbers of blocks.
    Destinations must be distinct and inside the destination pool; sources
    inside the source pool.
    """
    pairs = np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2)
    src, dst = pairs[:, 0], pairs[:, 1]
    assert len(np.unique(dst)) == len(dst), "destinations must be distinct"
    assert ((src >= 0) & (src < src_k.shape[0])).all(), "source block outside its pool"
    assert ((dst >= 0) & (dst < dst_k.shape[0])).all(), "destination block outside its pool"
    assert src_k.shape[1:] == dst_k.shape[1:] and src_v.shape[1:] == dst_v.shape[1:]
    k_new = dst_k if inplace else dst_k.copy()
    v_new = dst_v if inplace else dst_v.copy()
    k_new[dst] = src_k[src]
    v_new[dst] = src_v[src]
    return k_new, v_new


# ---------------------------------------------------------------------------
# read path: reassemble through the block table
# ---------------------------------------------------------------------------
def gather_sequence(block_table_row: np.ndarray, context_len: int,
                    k_cache: np.ndarray, v_cache: np.ndarray):
    """Contiguous K and V ([L, Hkv, D], pool dtype, bit-exact) of one sequence."""
    NB, Hkv, BS, D = k_cache.shape
    L = int(context_len)
    n = -(-L // BS)
    blocks = np.asarray(block_table_row[:n], dtype=np.int64)
    k = k_cache[blocks].transpose(0, 2, 1, 3).reshape(n * BS, Hkv, D)[:L]
    # [n, Hkv, BS / X, D, X] -> [n, BS / X, X, Hkv, D]: token (group, x) = group * X + x
    v = v_cache[blocks].transpose(0, 2, 4, 1, 3).reshape(n * BS, Hkv, D)[:L]
    return k, v


def gather_kv(block_table: np.ndarray, context_lens: np.ndarray,
              k_cache: np.ndarray, v_cache: np.ndarray):
    """All sequences' K/V concatenated along tokens: ([sum L, Hkv, D], same)."""
    ks, vs = [], []
    for s, L in enumerate(context_lens):
        k, v = gather_sequence(block_table[s], int(L), k_cache, v_cache)
        ks.append(k)
        vs.append(v)
    return np.concatenate(ks), np.concatenate(vs)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def attention_one(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of queries q [G, D] over keys/values k, v [L, D] (float64)."""
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]))
    z = scale * (k @ q.T)                     # [L, G] logits
    w = np.exp(z - z.max(axis=0))             # unnormalised weights
    return (w.T @ v) / w.sum(axis=0)[:, None]


def paged_attention(query: np.ndarray, block_table: np.ndarray, context_lens: np.ndarray,
                    k_cache: np.ndarray, v_cache: np.ndarray, scale: float,
                    dtype: str, seqs=None) -> np.ndarray:
    """Decode attention of each sequence's query over its paged K/V, in float64.

    query: [S, Hq, D].  Returns [S, Hq, D] float64 (rows of sequences not in
    ``seqs`` are left at zero).  A sequence of length 0 gives zeros.
    """
    S, Hq, D = query.shape
    Hkv = k_cache.shape[1]
    g = Hq // Hkv
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        k, v = gather_sequence(block_table[s], int(context_lens[s]), k_cache, v_cache)
        kf, vf, qf = decode(k, dtype), decode(v, dtype), decode(query[s], dtype)
        for kvh in range(Hkv):
            heads = slice(kvh * g, (kvh + 1) * g)
            out[s, heads] = attention_one(qf[heads], kf[:, kvh], vf[:, kvh], scale)
    return out


def paged_prefill(query: np.ndarray, query_start_loc: np.ndarray, block_table: np.ndarray,
                  context_lens: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                  scale: float, dtype: str, seqs=None) -> np.ndarray:
    """Causal attention of a chunk of new query tokens per sequence over its paged K/V.

    Sequence s owns query rows query_start_loc[s] .. query_start_loc[s+1] - 1; with
    n = that count and L = context_lens[s] (the chunk included), row i is the
    token at position p = L - n + i and attends to positions 0 .. p.  The chunk's
    own K/V are already in the pool.  This is what a request's prompt needs when
    an earlier part of its context is cached in blocks (a shared system prompt,
    "core inference engine" page, section 2.2; prefix caching, "core features"
    page, sections 4.2 and 4.6): only the new tokens are computed, attending to
    the cached prefix through the block table ("core architecture" page,
    section 2.2.2).  One new token (n = 1) is the decode step.

    query: [T, Hq, D]; returns [T, Hq, D] float64.
    """
    T, Hq, D = query.shape
    Hkv = k_cache.shape[1]
    g = Hq // Hkv
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for s in (range(len(qsl) - 1) if seqs is None else seqs):
        r0, r1 = int(qsl[s]), int(qsl[s + 1])
        L = int(context_lens[s])
        n = r1 - r0
        assert 0 <= n <= L, "a chunk cannot be longer than its context"
        if n == 0:
            continue
        k, v = gather_sequence(block_table[s], L, k_cache, v_cache)
        kf, vf, qf = decode(k, dtype), decode(v, dtype), decode(query[r0:r1], dtype)
        # query row (i, head) sits at position p_i = L - n + i and sees the keys t <= p_i
        pos = np.repeat(L - n + np.arange(n), g)                               # [n * g]
        seen = np.arange(L)[None, :] <= pos[:, None]                            # [n * g, L]
        for kvh in range(Hkv):
            heads = slice(kvh * g, (kvh + 1) * g)
            q = qf[:, heads].reshape(n * g, D)
            z = np.where(seen, scale * (q @ kf[:, kvh].T), -np.inf)             # logits
            w = np.exp(z - z.max(axis=1, keepdims=True))                        # 0 where unseen
            o = (w @ vf[:, kvh]) / w.sum(axis=1)[:, None]
            out[r0:r1, heads] = o.reshape(n, g, D)
    return out


# ---------------------------------------------------------------------------
# split context: per-partition statistics and their log-sum-exp combination
# ---------------------------------------------------------------------------
def partition_stats(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                    partition_size: int):
    """Per partition of ``partition_size`` tokens: running max m, weight sum l
    and unnormalised weighted value sum acc (natural-log domain, float64).

    q [G, D], k, v [L, D]; returns m [P, G], l [P, G], acc [P, G, D].
    """
    L = k.shape[0]
    P = -(-L // partition_size)
    m = np.empty((P, q.shape[0]))
    l = np.empty((P, q.shape[0]))
    acc = np.empty((P, q.shape[0], v.shape[1]))
    for p in range(P):
        kp = k[p * partition_size:(p + 1) * partition_size]
        vp = v[p * partition_size:(p + 1) * partition_size]
        z = scale * (kp @ q.T)
        m[p] = z.max(axis=0)
        w = np.exp(z - m[p])
        l[p] = w.sum(axis=0)
        acc[p] = w.T @ vp
    return m, l, acc


def combine_partitions(m: np.ndarray, l: np.ndarray, acc: np.ndarray) -> np.ndarray:
    """Log-sum-exp combination: with M = max_p m_p,
    out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p."""
    M = m.max(axis=0)
    w = np.exp(m - M)
    return (w[:, :, None] * acc).sum(axis=0) / (w * l).sum(axis=0)[:, None]


# ---------------------------------------------------------------------------
# helpers for building pools in tests
# ---------------------------------------------------------------------------
def empty_pools(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int,
                dtype: str, fill: str = "nan"):
    """Fresh pools filled with NaN (poison) or zeros."""
    ks = k_cache_shape(num_blocks, num_kv_heads, head_dim, block_size, dtype)
    vs = v_cache_shape(num_blocks, num_kv_heads, head_dim, block_size, dtype)
    if dtype == "bf16":
        val = np.uint16(0x7FC0) if fill == "nan" else np.uint16(0)
        return np.full(ks, val, dtype=np.uint16), np.full(vs, val, dtype=np.uint16)
    val = np.float32(math.nan) if fill == "nan" else np.float32(0)
    return np.full(ks, val, dtype=np.float32), np.full(vs, val, dtype=np.float32)
