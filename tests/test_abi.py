"""The C ABI: every declared symbol is exported, and host-side checks reject bad
arguments before anything is launched (these calls never reach the GPU)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import paged_kv_cache_425_amd as pk

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "pagedattn.h")


def declared_functions() -> list:
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pk.LIB_PATH):
        from paged_kv_cache_425_amd.build import build
        build()
    return pk.load_library()


def test_coexec_probe_rejects_before_launch(lib):
    f = lib.pa_coexec_probe
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 2
    assert f(5, 256, 8, 16, FAKE, None) == 1         # no such mode
    assert f(-1, 256, 8, 16, FAKE, None) == 1
    assert f(0, 0, 8, 16, FAKE, None) == 1           # no workgroups
    assert f(0, 256, 6, 16, FAKE, None) == 1         # 4 or 8 waves only
    assert f(0, 256, 8, 0, FAKE, None) == 1          # no iterations
    assert f(0, 256, 8, (1 << 20) + 1, FAKE, None) == 1
    assert f(0, 256, 8, 16, None, None) == 1         # no output
    assert f(0, 256, 8, 16, FAKE + 2, None) == 1     # output misaligned


def test_plan_pairs_rejects_before_writing(lib):
    f = lib.pa_plan_pairs
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] + [ctypes.c_int] * 5 + [ctypes.c_void_p]
    lens = (ctypes.c_int32 * 4)(1, 2, 3, 4)
    out = (ctypes.c_uint32 * 4)(*([7] * 4))
    assert f(None, 4, 16, 8192, 32, 8, out) == 1             # no lengths
    assert f(lens, 4, 16, 8192, 32, 8, None) == 1            # no output
    assert f(lens, 1, 16, 8192, 32, 8, out) == 1             # fewer than two sequences
    assert f(lens, 4, 24, 8192, 32, 8, out) == 1             # block size
    assert f(lens, 4, 16, 9000, 32, 8, out) == 1             # clamp past 8192
    assert f(lens, 4, 16, 8192, 32, 5, out) == 1             # 4 or 8 waves only
    assert list(out) == [7] * 4                                # nothing written
    assert f(lens, 4, 16, 8192, 32, 8, out) == 0


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "pa_abi_version", "pa_status_string", "pa_default_partition_size",
        "pa_paged_attention_workspace_size", "pa_paged_attention", "pa_reshape_and_cache",
        "pa_gather_kv", "pa_decode_step", "pa_copy_blocks", "pa_paged_prefill",
        "pa_reshape_and_cache_fp8", "pa_paged_attention_fp8", "pa_decode_step_fp8",
        "pa_swap_blocks", "pa_decode_step_noalloc", "pa_read_probe", "pa_coexec_probe",
        "pa_decode_step_shared_prefix", "pa_set_decode_math", "pa_get_decode_math",
        "pa_plan_pairs"])


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.pa_abi_version() == 7
    for code in range(5):
        assert lib.pa_status_string(code).decode().startswith("PA_")
    assert b"unknown" in lib.pa_status_string(99)


def test_default_partition_is_a_multiple_of_64(lib):
    for S, L in ((1, 10), (64, 2048), (16, 32768), (256, 8192)):
        P = lib.pa_default_partition_size(S, 8, L, 1)
        assert P >= 64 and P % 64 == 0


def test_default_partition_policy(lib):
    """Without a visible device the policy assumes 256 compute units."""
    # 64 x 8 (sequence, kv head) pairs fill 256 units twice: one partition covers the longest
    assert lib.pa_default_partition_size(64, 8, 2011, 1) == 2048
    # 16 x 8 pairs do not: split into ~4 workgroups per unit, partitions >= 512 tokens
    assert lib.pa_default_partition_size(16, 8, 32768, 1) == 4096
    assert lib.pa_default_partition_size(16, 8, 3000, 1) == 512
    # never longer than the longest sequence (rounded to 64), never past 8192
    assert lib.pa_default_partition_size(1, 1, 10, 1) == 64
    assert lib.pa_default_partition_size(4096, 8, 100000, 1) == 8192


def test_workspace_size(lib):
    # one partition -> nothing needed
    assert lib.pa_paged_attention_workspace_size(64, 32, 8, 128, 256, 256, 1) == 0
    ws = lib.pa_paged_attention_workspace_size(16, 64, 8, 128, 32768, 512, 1)
    rows = 16 * 64 * 64
    assert ws >= rows * 2 * 4 + rows * 128 * 4
    # rejected arguments give 0
    assert lib.pa_paged_attention_workspace_size(16, 64, 8, 96, 32768, 512, 1) == 0
    assert lib.pa_paged_attention_workspace_size(16, 64, 8, 128, 32768, 100, 1) == 0


P = ctypes.c_void_p
FAKE = 0x1000          # a 16-byte aligned, never dereferenced address


def call_attention(lib, **over):
    args = dict(out=FAKE, q=FAKE, bt=FAKE, cl=FAKE, kc=FAKE, vc=FAKE, S=4, Hq=32, Hkv=8, D=128,
                BS=16, MB=8, NB=64, maxlen=128, scale=0.1, dtype=1, part=0, ws=None, wsb=0,
                stream=None, host_lens=None)
    args.update(over)
    return lib.pa_paged_attention(args["out"], args["q"], args["bt"], args["cl"], args["kc"],
                                  args["vc"], args["S"], args["Hq"], args["Hkv"], args["D"],
                                  args["BS"], args["MB"], args["NB"], args["maxlen"],
                                  args["scale"], args["dtype"], args["part"], args["ws"],
                                  args["wsb"], args["stream"], args["host_lens"])


@pytest.mark.parametrize("over,code", [
    (dict(D=96), 2), (dict(BS=64), 2), (dict(dtype=7), 2),
    (dict(Hq=36), 1), (dict(Hq=80, Hkv=8), 2),          # group of 10 > 8 for bf16
    (dict(q=None), 1), (dict(out=FAKE + 4), 1), (dict(kc=FAKE + 8), 1),
    (dict(maxlen=129), 1), (dict(MB=0), 1), (dict(part=100), 1), (dict(part=32), 1),
    (dict(S=-1), 1),
    (dict(maxlen=128, part=64), 3),                     # two partitions, no workspace
])
def test_paged_attention_rejects_before_launch(lib, over, code):
    assert call_attention(lib, **over) == code


def test_paged_attention_empty_batch_is_ok(lib):
    assert call_attention(lib, S=0, out=None, q=None) == 0


def test_f32_allows_larger_groups(lib):
    # group 16 is allowed for f32; with a null query it still fails as invalid argument,
    # i.e. the group check passed
    assert call_attention(lib, Hq=128, Hkv=8, dtype=0, q=None) == 1
    assert call_attention(lib, Hq=136, Hkv=8, dtype=0) == 2


def test_decode_step_rejects_before_launch(lib):
    f = lib.pa_decode_step
    base = [FAKE] * 9 + [4, 32, 8, 128, 16, 8, 64, 128, 0.1, 1, 0, None, 0, None, None]

    def call(over):
        a = list(base)
        for k, v in over.items():
            a[k] = v
        return f(*a)
    assert call({2: None}) == 1                 # key missing
    assert call({4: FAKE + 4}) == 1             # slot_mapping misaligned
    assert call({3: FAKE + 8}) == 1             # value misaligned
    assert call({12: 96}) == 2                  # head size
    assert call({16: 129}) == 1                 # max_context_len past the table
    assert call({9: 0, 2: None, 3: None, 4: None}) == 0   # empty batch
    assert call({16: 128, 19: 64}) == 3         # two partitions, no workspace


def test_decode_step_noalloc_rejects_before_launch(lib):
    """The allocation-free step takes the arguments of pa_decode_step minus the workspace;
    a call whose partitions need more than the fixed scratch is refused."""
    f = lib.pa_decode_step_noalloc
    base = [FAKE] * 9 + [4, 32, 8, 128, 16, 8, 64, 128, 0.1, 1, 0, None, None]

    def call(over):
        a = list(base)
        for k, v in over.items():
            a[k] = v
        return f(*a)
    assert call({2: None}) == 1                 # key missing
    assert call({12: 96}) == 2                  # head size
    assert call({16: 129}) == 1                 # max_context_len past the table
    assert call({9: 0, 2: None, 3: None, 4: None}) == 0   # empty batch
    # 4096 sequences x 64 heads in 64-token partitions of 32768 tokens: 4.4 GB of partials
    big = {9: 4096, 10: 64, 14: 2048, 16: 32768, 19: 64}
    need = lib.pa_paged_attention_workspace_size(4096, 64, 8, 128, 32768, 64, 1)
    assert need > 64 << 20
    assert call(big) == 3


def test_shared_prefix_step_rejects_before_launch(lib):
    f = lib.pa_decode_step_shared_prefix
    #       out..v_cache  S  Hq Hkv  D  BS MB  NB  maxL pfx scale dt strm hl
    base = [FAKE] * 9 + [4, 32, 8, 128, 16, 8, 64, 128, 2, 0.1, 1, None, None]

    def call(over):
        a = list(base)
        for k, v in over.items():
            a[k] = v
        return f(*a)
    assert call({12: 96}) == 2                  # head size
    assert call({17: 513, 14: 600, 16: 9000}) == 2    # prefix past 8192 tokens
    assert call({17: 2, 14: 600, 16: 8300}) == 2      # a suffix past 8192 tokens
    assert call({17: 8}) == 1                   # prefix takes every table column
    assert call({17: 0}) == 1                   # no prefix
    assert call({16: 20}) == 1                  # longest context shorter than the prefix
    assert call({4: None, 2: None, 3: None, 9: 0}) == 0   # empty batch
    assert call({2: None}) == 1                 # slot_mapping without key
    lens = (ctypes.c_int32 * 4)(40, 40, 31, 40)          # a host length below the prefix
    assert call({21: ctypes.cast(lens, ctypes.c_void_p)}) == 1


def test_decode_math_selector(lib):
    """The selector is process-wide state with no device work: MFMA by default, VALU on
    request, anything else refused and the setting kept."""
    assert lib.pa_get_decode_math() == 0
    try:
        assert lib.pa_set_decode_math(1) == 0
        assert lib.pa_get_decode_math() == 1
        assert lib.pa_set_decode_math(2) == 1 and lib.pa_set_decode_math(-1) == 1
        assert lib.pa_get_decode_math() == 1
        with pk.decode_math("mfma"):
            assert pk.get_decode_math() == "mfma"
        assert pk.get_decode_math() == "valu"
        with pytest.raises(ValueError):
            pk.set_decode_math("dot")
    finally:
        assert lib.pa_set_decode_math(0) == 0


def test_read_probe_rejects_before_launch(lib):
    f = lib.pa_read_probe
    base = [FAKE, FAKE, 16, 4096, 64, 8, 0, FAKE, None]

    def call(over):
        a = list(base)
        for k, v in over.items():
            a[k] = v
        return f(*a)
    assert call({3: 4000}) == 1                 # piece not a multiple of 4 KB
    assert call({5: 6}) == 2                    # in-flight count not built
    assert call({4: 0}) == 1                    # no workgroups
    assert call({0: FAKE + 4}) == 1             # buffer misaligned
    assert call({6: 2}) == 1                    # load policy is 0 or 1
    assert call({2: 0}) == 0                    # nothing to read
    assert call({2: 0, 6: 1}) == 0


def test_reshape_and_cache_rejects_before_launch(lib):
    f = lib.pa_reshape_and_cache
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 96, 16, 64, 1, None) == 2
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 12, 64, 1, None) == 2
    assert f(None, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 16, 64, 1, None) == 1
    assert f(FAKE, FAKE, FAKE + 4, FAKE, FAKE, 4, 8, 128, 16, 64, 1, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 8, 128, 16, 64, 1, None) == 1
    assert f(None, None, None, None, None, 0, 8, 128, 16, 64, 1, None) == 0


def test_prefill_rejects_before_launch(lib):
    f = lib.pa_paged_prefill
    base = [FAKE] * 7 + [4, 32, 8, 128, 16, 8, 64, 100, 40, 0.1, 1, None]

    def call(over):
        a = list(base)
        for k, v in over.items():
            a[k] = v
        return f(*a)
    assert call({1: None}) == 1                  # query missing
    assert call({2: FAKE + 2}) == 1              # query_start_loc misaligned
    for bad in (0.0, -0.5, float("nan"), float("inf")):
        assert call({16: bad}) == 1              # scale must be positive and finite
    assert call({10: 96}) == 2                   # head size
    assert call({11: 24}) == 2                   # block size
    assert call({8: 24, 9: 8}) == 2              # group of 3 does not divide 128
    assert call({8: 36}) == 1                    # heads not a multiple of kv heads
    assert call({14: 0}) == 0                    # no query tokens: nothing to do
    assert call({7: 0}) == 0                     # no sequences


def test_copy_blocks_rejects_before_launch(lib):
    f = lib.pa_copy_blocks
    assert f(None, FAKE, FAKE, 4, 8, 128, 16, 64, 1, None) == 1
    assert f(FAKE, FAKE, FAKE + 4, 4, 8, 128, 16, 64, 1, None) == 1
    assert f(FAKE, FAKE, FAKE, -1, 8, 128, 16, 64, 1, None) == 1
    assert f(FAKE, FAKE, FAKE, 4, 8, 96, 16, 64, 1, None) == 2
    assert f(None, None, None, 0, 8, 128, 16, 64, 1, None) == 0


def test_gather_rejects_before_launch(lib):
    f = lib.pa_gather_kv
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 128, 16, 4, 64, 65, 1, None) == 1
    assert f(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 2, 8, 128, 16, 4, 64, 64, 1, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 64, 24, 4, 64, 64, 1, None) == 2


def test_reshape_and_cache_fp8_rejects_before_launch(lib):
    f = lib.pa_reshape_and_cache_fp8
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 16, 64, 1, 0.5, 0.25, None]

    def call(over):
        a = list(ok)
        for k, v in over.items():
            a[k] = v
        return f(*a)

    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert call({11: bad}) == 1                 # k_scale
        assert call({12: bad}) == 1                 # v_scale
    assert call({7: 96}) == 2                       # head_dim
    assert call({8: 12}) == 2                       # block_size
    assert call({10: 7}) == 2                       # dtype
    assert call({0: None}) == 1
    assert call({3: FAKE + 8}) == 1                 # k_cache misaligned
    assert call({2: FAKE + 4}) == 1                 # slot_mapping misaligned
    assert call({5: -1}) == 1
    assert call({5: 0}) == 0                        # nothing to write: no launch


def test_paged_attention_fp8_rejects_before_launch(lib):
    f = lib.pa_paged_attention_fp8
    ok = [FAKE] * 6 + [4, 32, 8, 128, 16, 8, 64, 128, 0.1, 0.5, 0.25, 1, 0, None, 0, None, None]

    def call(over):
        a = list(ok)
        for k, v in over.items():
            a[k] = v
        return f(*a)

    assert call({17: 0}) == 2                       # f32 queries: not built for FP8 pools
    for bad in (0.0, -2.0, float("nan"), float("inf")):
        assert call({15: bad}) == 1                 # k_scale
        assert call({16: bad}) == 1                 # v_scale
    assert call({9: 96}) == 2
    assert call({7: 72}) == 2                       # group of 9 > 8
    assert call({18: 96}) == 1                      # partition not a multiple of 64
    assert call({4: FAKE + 8}) == 1                 # k_cache misaligned
    assert call({13: 129}) == 1                     # max_context_len past the table
    assert call({6: 0}) == 0                        # empty batch: no launch


def test_decode_step_fp8_rejects_before_launch(lib):
    f = lib.pa_decode_step_fp8
    ok = [FAKE] * 9 + [4, 32, 8, 128, 16, 8, 64, 128, 0.1, 0.5, 0.25, 1, 0, None, 0, None, None]

    def call(over):
        a = list(ok)
        for k, v in over.items():
            a[k] = v
        return f(*a)

    assert call({20: 0}) == 2                       # f32: not built for FP8 pools
    assert call({18: 0.0}) == 1                     # k_scale
    assert call({19: float("nan")}) == 1            # v_scale
    assert call({2: None}) == 1                     # key missing
    assert call({4: FAKE + 4}) == 1                 # slot_mapping misaligned
    assert call({3: FAKE + 8}) == 1                 # value misaligned
    assert call({9: 0}) == 0                        # empty batch: no launch


def test_swap_blocks_rejects_before_launch(lib):
    f = lib.pa_swap_blocks
    ok = [FAKE] * 5 + [4, 8, 128, 16, 64, 32, 1, None]

    def call(over):
        a = list(ok)
        for k, v in over.items():
            a[k] = v
        return f(*a)

    assert call({11: 3}) == 2                       # unknown dtype
    assert call({7: 96}) == 2                       # head_dim
    assert call({8: 12}) == 2                       # block_size
    assert call({5: -1}) == 1                       # num_pairs
    assert call({5: 0}) == 0                        # nothing to move: no launch
    assert call({9: 0}) == 1                        # empty source pool
    assert call({0: None}) == 1
    assert call({2: FAKE + 8}) == 1                 # destination misaligned
    assert call({4: FAKE + 4}) == 1                 # block_mapping misaligned


def test_copy_blocks_accepts_fp8_pools_and_checks_them(lib):
    f = lib.pa_copy_blocks
    assert f(FAKE, FAKE, FAKE, 4, 8, 96, 16, 64, 2, None) == 2   # FP8 pools, bad head_dim
    assert f(FAKE, FAKE, FAKE, 0, 8, 128, 16, 64, 2, None) == 0  # FP8 pools, nothing to copy
    assert f(FAKE, FAKE, FAKE, 4, 8, 128, 16, 64, 3, None) == 2  # unknown dtype


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from paged_kv_cache_425_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        binding.load_library()


def test_binding_host_lengths_are_checked_and_converted():
    """host_context_lens: a host int32 copy of the lengths (numpy or CPU tensor), or None."""
    import numpy as np
    import torch

    from paged_kv_cache_425_amd.binding import _host_lens
    assert _host_lens(None, 3) == (None, None)
    ptr, hold = _host_lens(np.array([5, 17, 33]), 3)
    assert hold.dtype == np.int32 and ptr == hold.ctypes.data and hold.tolist() == [5, 17, 33]
    ptr, hold = _host_lens(torch.tensor([4, 0, 9], dtype=torch.int64), 3)
    assert hold.dtype == torch.int32 and ptr == hold.data_ptr() and hold.tolist() == [4, 0, 9]
    with pytest.raises(ValueError):
        _host_lens(np.array([1, 2]), 3)
    with pytest.raises(ValueError):
        _host_lens(np.zeros((3, 1), dtype=np.int32), 3)
