"""Pins of the FP8 (E4M3) K/V oracle against the format's definition and independent routes.

The format facts come from the OCP 8-bit floating-point specification (E4M3:
bias 7, subnormals m * 2^-9, S.1111.111 = NaN, no infinities, max 448).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import make_workload

# code -> value, as the OCP specification lists them for E4M3
SPEC_VALUES = {
    0x00: 0.0,
    0x01: 2.0 ** -9,               # smallest subnormal
    0x07: 0.875 * 2.0 ** -6,       # largest subnormal
    0x08: 2.0 ** -6,               # smallest normal
    0x38: 1.0,
    0x3F: 1.875,
    0x40: 2.0,
    0x7E: 448.0,                   # largest normal
    0xB8: -1.0,
    0xFE: -448.0,
}


def test_spec_values():
    v = oracle.e4m3_values()
    for code, want in SPEC_VALUES.items():
        assert v[code] == want, hex(code)
    assert math.isnan(v[0x7F]) and math.isnan(v[0xFF])
    assert v[0x80] == 0.0 and math.copysign(1.0, v[0x80]) < 0
    assert np.isnan(v).sum() == 2


def test_order_and_sign_symmetry():
    v = oracle.e4m3_values()
    pos = v[:0x7F]
    assert (np.diff(pos) > 0).all()
    for c in range(0x7F):
        assert v[c | 0x80] == -v[c]


def test_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = oracle.e4m3_encode(oracle.e4m3_decode(codes).astype(np.float32))
    assert np.array_equal(back, codes)


def _midpoints() -> np.ndarray:
    pos = oracle.e4m3_values()[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2            # exact in float32 (<= 5 significant bits)
    return np.concatenate([mids, -mids]).astype(np.float32)


def test_matches_torch_float8_e4m3fn_in_range():
    rng = np.random.default_rng(5)
    mag = 2.0 ** rng.uniform(-13, np.log2(448.0), 200_000)
    x = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    x = np.concatenate([x, _midpoints(), np.float32([0.0, -0.0, 448.0, -448.0])])
    ours = oracle.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_nearest_code_by_brute_force_and_ties_to_even():
    v = oracle.e4m3_values()
    finite = np.array([c for c in range(256) if not math.isnan(v[c])])
    rng = np.random.default_rng(6)
    x = np.concatenate([rng.normal(0, 30, 3000), rng.normal(0, 0.01, 1000)]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    codes = oracle.e4m3_encode(x)
    for xi, c in zip(x.astype(np.float64), codes):
        d = np.abs(v[finite] - xi)
        assert abs(v[c] - xi) == d.min()
    mids = _midpoints()
    codes = oracle.e4m3_encode(mids)
    assert ((codes & 1) == 0).all()
    # just above / below a midpoint go up / down
    up = oracle.e4m3_encode(np.nextafter(mids[mids > 0], np.float32(np.inf)))
    down = oracle.e4m3_encode(np.nextafter(mids[mids > 0], np.float32(0)))
    lo_codes = np.arange(0x7E)
    assert np.array_equal(up, (lo_codes + 1).astype(np.uint8))
    assert np.array_equal(down, lo_codes.astype(np.uint8))


def test_saturation_nan_and_signed_zero():
    x = np.float32([448.0, 449.0, 464.0, 480.0, 1e6, np.inf, -500.0, -np.inf, np.nan, -np.nan,
                    -0.0, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -11])
    got = oracle.e4m3_encode(x)
    want = [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0xFF, 0x80, 0x00, 0x02, 0x00]
    assert got.tolist() == want


def test_quantize_divides_in_float32():
    """x / scale is rounded to float32 before the E4M3 rounding: same codes as PyTorch's
    float32 division followed by its float8_e4m3fn conversion."""
    rng = np.random.default_rng(7)
    x = rng.normal(0, 3, 50_000).astype(np.float32)
    for scale in (0.1, 0.037, 1.0, 3.3):
        q = oracle.quantize(x, "f32", scale)
        t = (torch.from_numpy(x) / torch.tensor(scale, dtype=torch.float32))
        ref = t.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(q, ref), scale


def test_quantize_keeps_the_sign_of_a_nan_element():
    """IEEE 754 leaves the sign of a NaN quotient open: the code takes the element's sign."""
    x = np.float32([np.nan, -np.nan, -np.inf, 448.0 * 0.3 * 2])
    assert oracle.quantize(x, "f32", 0.3).tolist() == [0x7F, 0xFF, 0xFE, 0x7E]
    bf = np.array([0x7FC0, 0xFFC0, 0xFF80], dtype=np.uint16)       # +NaN, -NaN, -inf
    assert oracle.quantize(bf, "bf16", 0.3).tolist() == [0x7F, 0xFF, 0xFE]


def _fp8_workload(seed=11):
    return make_workload(name="fp8", context_lens=[1, 17, 40, 95], num_heads=8, num_kv_heads=2,
                         head_dim=64, block_size=16, dtype="bf16", seed=seed)


def _fp8_pools(w, k_scale, v_scale):
    kc, vc = oracle.empty_fp8_pools(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size)
    oracle.reshape_and_cache_fp8(w.rec_key, w.rec_value, w.rec_slot, kc, vc, "bf16",
                                 k_scale, v_scale, inplace=True)
    return kc, vc


def test_fp8_attention_equals_bf16_attention_on_the_decoded_values():
    """k_scale = v_scale = 1: every E4M3 value is a bf16 value, so the FP8 attention must equal
    the bf16 attention over pools holding the decoded values."""
    w = _fp8_workload()
    kc, vc = _fp8_pools(w, 1.0, 1.0)
    from workloads.configs import f32_to_bf16_bits
    vb = f32_to_bf16_bits(oracle.e4m3_decode(vc).astype(np.float32))
    # both pools have the token-major K layout [NB, H, BS, D]
    kb = f32_to_bf16_bits(oracle.e4m3_decode(kc).astype(np.float32))
    got = oracle.paged_attention_fp8(w.query, w.block_table, w.context_lens, kc, vc, w.scale,
                                     1.0, 1.0, "bf16")
    ref = oracle.paged_attention(w.query, w.block_table, w.context_lens,
                                 np.ascontiguousarray(kb), vb, w.scale, "bf16")
    assert np.array_equal(got, ref)


def test_fp8_attention_scale_invariants():
    """Doubling k_scale while halving the softmax scale leaves the logits unchanged; doubling
    v_scale doubles the output.  A dropped or misplaced scale fails one of them."""
    w = _fp8_workload(12)
    kc, vc = _fp8_pools(w, 0.05, 0.02)
    base = oracle.paged_attention_fp8(w.query, w.block_table, w.context_lens, kc, vc, w.scale,
                                      0.05, 0.02, "bf16")
    k2 = oracle.paged_attention_fp8(w.query, w.block_table, w.context_lens, kc, vc, w.scale / 2,
                                    0.1, 0.02, "bf16")
    v2 = oracle.paged_attention_fp8(w.query, w.block_table, w.context_lens, kc, vc, w.scale,
                                    0.05, 0.04, "bf16")
    np.testing.assert_allclose(k2, base, rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(v2, 2 * base)
    # a changed k_scale alone does change the result
    k3 = oracle.paged_attention_fp8(w.query, w.block_table, w.context_lens, kc, vc, w.scale,
                                    0.1, 0.02, "bf16")
    assert np.abs(k3 - base).max() > 1e-3


def test_fp8_attention_equals_dense_attention_over_quantised_sequences():
    """Brute force: quantise each sequence's contiguous K/V directly, decode, and run dense
    softmax attention; the paged FP8 path must give the same numbers."""
    w = _fp8_workload(13)
    ks, vs = 0.03, 0.07
    kc, vc = _fp8_pools(w, ks, vs)
    got = oracle.paged_attention_fp8(w.query, w.block_table, w.context_lens, kc, vc, w.scale,
                                     ks, vs, "bf16")
    g = w.num_heads // w.num_kv_heads
    for s, recs in enumerate(w.seq_records):
        k = oracle.e4m3_decode(oracle.quantize(w.rec_key[recs], "bf16", ks)) * float(np.float32(ks))
        v = oracle.e4m3_decode(oracle.quantize(w.rec_value[recs], "bf16", vs)) * float(np.float32(vs))
        q = oracle.decode(w.query[s], "bf16")
        for h in range(w.num_heads):
            kvh = h // g
            z = w.scale * (k[:, kvh] @ q[h])
            p = np.exp(z - z.max())
            want = (p @ v[:, kvh]) / p.sum()
            np.testing.assert_allclose(got[s, h], want, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("bad", [0x7F, 0xFF])
def test_nan_codes_poison_only_their_reader(bad):
    w = _fp8_workload(14)
    kc, vc = _fp8_pools(w, 1.0, 1.0)
    s = 3                                        # longest sequence
    b = int(w.block_table[s, 0])
    vc[b, 0, 0, 5, 0] = bad                      # token 0 of the block, kv head 0, channel 5
    out = oracle.paged_attention_fp8(w.query, w.block_table, w.context_lens, kc, vc, w.scale,
                                     1.0, 1.0, "bf16")
    g = w.num_heads // w.num_kv_heads
    assert np.isnan(out[s, :g, 5]).all()
    assert not np.isnan(out[s, g:]).any()
    assert not np.isnan(out[:s]).any()


@pytest.mark.parametrize("scale", [0.0135, 1.0, 3.7e-3, 250.0])
def test_quantize_bf16_table_equals_quantize(scale):
    """The table form gives the codes quantize() gives, element for element: random bf16
    patterns of every magnitude, both NaNs, both infinities, zeros and subnormals."""
    rng = np.random.default_rng(77)
    x = rng.integers(0, 1 << 16, size=300_000).astype(np.uint16)
    x[:8] = [0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x0001, 0x8001]
    assert np.array_equal(oracle.quantize_bf16(x, scale), oracle.quantize(x, "bf16", scale))
