"""FP8 (E4M3) K/V storage for the paged cache -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The GPU library shares no code with it and never calls it.

What the pages fix, and what is read into them
----------------------------------------------
The pages name FP8 E4M3 once, as one of the precisions a model can be served
in: an 8-bit float that needs about half the memory of 16-bit formats
("core features" page, section 4.3, the table of quantisation formats).  They
say nothing about storing the K/V cache in it.  This module takes the
plainest reading of an FP8 K/V cache:

* Format: E4M3 as the OCP 8-bit floating-point specification defines it (the
  variant gfx950 converts natively): 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits.  Exponent field 0 holds the subnormals m * 2^-9; the codes
  S.1111.111 are NaN; there are no infinities; the largest finite value is
  1.75 * 2^8 = 448.
* One scale per tensor: ``k_scale`` for every K element, ``v_scale`` for every
  V element.
* Writing (quantising) element x: q = x / scale rounded to float32 (the
  precision the write kernel divides in), then the E4M3 value nearest to q,
  ties to the code with the even last bit.  Magnitudes above 448 and
  infinities saturate to +-448; -0 keeps its sign.  A NaN element stays NaN
  with the sign of the element itself (code 0x7F or 0xFF): IEEE 754 leaves
  the sign of a NaN quotient open, so the code is fixed before the division.
* Reading (dequantising) code c: E4M3(c) * scale.  The product has at most
  4 + 24 significant bits, so float64 holds it exactly.
* Attention over an FP8 cache is attention over the dequantised K and V.

Cache layout: the boundary's layout with 1-byte elements, so a V group is
min(16, block_size) tokens: k_cache uint8 [num_blocks, Hkv, block_size, D],
v_cache uint8 [num_blocks, Hkv, block_size / X, D, X].

Pins (in the test suite): the code values the OCP specification lists
(0, min subnormal, min normal, 1, 448, NaN), the format's monotone order,
agreement with PyTorch's float8_e4m3fn conversion on every in-range input,
brute-force nearest-code search on random and tie inputs, saturation and
NaN cases, and attention invariants under the two scales.
"""
from __future__ import annotations

import numpy as np

from .paged_attention import attention_one, decode, gather_sequence, reshape_and_cache

FP8_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for S.1111.111), from the bit fields."""
    out = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            out[c] = np.nan
        elif e == 0:
            out[c] = sign * m * 2.0 ** -9            # subnormal: 0.m * 2^(1 - 7)
        else:
            out[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_VALUES = e4m3_values()
# the non-negative finite codes 0x00 .. 0x7E in increasing value order
_POS_VALUES = _VALUES[:0x7F]


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """float64 values of E4M3 codes (uint8 array)."""
    return _VALUES[np.asarray(codes, dtype=np.uint8).astype(np.int64)]


def e4m3_encode(q: np.ndarray) -> np.ndarray:
    """E4M3 codes (uint8) of float32 values: nearest, ties to even code, saturating."""
    q = np.asarray(q, dtype=np.float32).astype(np.float64)
    neg = np.signbit(q)
    nan = np.isnan(q)
    a = np.where(nan, 0.0, np.abs(q))
    # the two codes around a: lo with value <= a < value of lo + 1 (a < 448 here)
    lo = np.clip(np.searchsorted(_POS_VALUES, a, side="right") - 1, 0, 0x7D)
    hi = lo + 1
    dlo = a - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi] - a
    tie_code = np.where(lo % 2 == 0, lo, hi)               # tie: the even code
    code = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, tie_code))
    code = np.where(a >= FP8_MAX, 0x7E, code)              # saturate (and +-inf)
    code = np.where(nan, 0x7F, code)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


def quantize(x: np.ndarray, dtype: str, scale: float) -> np.ndarray:
    """Codes of elements x (float32 array or bfloat16 bits) stored with ``scale``."""
    xf = decode(x, dtype).astype(np.float32)           # exact: the inputs are float32 or bf16
    with np.errstate(invalid="ignore", over="ignore"):
        q = xf / np.float32(scale)                     # float32 division, correctly rounded
    codes = e4m3_encode(q)
    nan = np.isnan(xf)
    codes[nan] = np.where(np.signbit(xf[nan]), 0xFF, 0x7F)   # the element's own sign
    return codes


def quantize_bf16(x_bits: np.ndarray, scale: float) -> np.ndarray:
    """quantize() of bfloat16 elements, looked up in a table of quantize() over all 65536
    bit patterns: the code of an element depends only on its bits and the scale, so the
    result is the same array of codes (a pin in the test suite compares the two)."""
    table = quantize(np.arange(1 << 16, dtype=np.uint32).astype(np.uint16), "bf16", scale)
    return table[np.asarray(x_bits, dtype=np.uint16)]


def empty_fp8_pools(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int,
                    fill: int = 0x7F):
    """FP8 pools filled with one code (NaN by default, so stray reads show)."""
    X = min(16, block_size)
    ks = (num_blocks, num_kv_heads, block_size, head_dim)
    vs = (num_blocks, num_kv_heads, block_size // X, head_dim, X)
    return np.full(ks, fill, dtype=np.uint8), np.full(vs, fill, dtype=np.uint8)


def reshape_and_cache_fp8(key: np.ndarray, value: np.ndarray, slot_mapping: np.ndarray,
                          k_cache: np.ndarray, v_cache: np.ndarray, dtype: str,
                          k_scale: float, v_scale: float, inplace: bool = False):
    """FP8 pools with token i's quantised K/V at slot_mapping[i] (negative: no write)."""
    kq = quantize(key, dtype, k_scale)
    vq = quantize(value, dtype, v_scale)
    return reshape_and_cache(kq, vq, slot_mapping, k_cache, v_cache, inplace=inplace)


def paged_attention_fp8(query: np.ndarray, block_table: np.ndarray, context_lens: np.ndarray,
                        k_cache: np.ndarray, v_cache: np.ndarray, scale: float,
                        k_scale: float, v_scale: float, dtype: str, seqs=None) -> np.ndarray:
    """Decode attention over FP8 pools, in float64 (query of ``dtype``)."""
    S, Hq, D = query.shape
    Hkv = k_cache.shape[1]
    g = Hq // Hkv
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        k, v = gather_sequence(block_table[s], int(context_lens[s]), k_cache, v_cache)
        kf = e4m3_decode(k) * float(np.float32(k_scale))
        vf = e4m3_decode(v) * float(np.float32(v_scale))
        qf = decode(query[s], dtype)
        for kvh in range(Hkv):
            heads = slice(kvh * g, (kvh + 1) * g)
            out[s, heads] = attention_one(qf[heads], kf[:, kvh], vf[:, kvh], scale)
    return out
