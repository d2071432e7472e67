"""ctypes binding of libpagedattn.so: argument marshalling only.

Every operation runs in the HIP kernels of the library; this module checks
tensor devices, dtypes and shapes, passes raw device pointers and torch's
current stream, and turns status codes into exceptions.  If the library is
not built it raises -- there is no other implementation to fall back on.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")

PA_OK = 0
_DTYPE_CODES = {torch.float32: 0, torch.bfloat16: 1}
_POOL_CODES = {torch.float32: 0, torch.bfloat16: 1, torch.uint8: 2}   # uint8: FP8 E4M3 codes
_ERRORS = {1: ValueError, 2: NotImplementedError, 3: ValueError, 4: RuntimeError}

_lib = None


def load_library() -> ctypes.CDLL:
    """Load the HIP library (once); raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m paged_kv_cache_425_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    i32, vp, sz, f32 = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
    lib.pa_abi_version.restype = i32
    lib.pa_abi_version.argtypes = []
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_status_string.argtypes = [i32]
    lib.pa_default_partition_size.restype = i32
    lib.pa_default_partition_size.argtypes = [i32, i32, i32, i32]
    lib.pa_paged_attention_workspace_size.restype = sz
    lib.pa_paged_attention_workspace_size.argtypes = [i32] * 7
    lib.pa_paged_attention.restype = i32
    lib.pa_paged_attention.argtypes = [vp] * 6 + [i32] * 8 + [f32, i32, i32, vp, sz, vp, vp]
    lib.pa_reshape_and_cache.restype = i32
    lib.pa_reshape_and_cache.argtypes = [vp] * 5 + [i32] * 6 + [vp]
    lib.pa_decode_step.restype = i32
    lib.pa_decode_step.argtypes = [vp] * 9 + [i32] * 8 + [f32, i32, i32, vp, sz, vp, vp]
    lib.pa_paged_prefill.restype = i32
    lib.pa_paged_prefill.argtypes = [vp] * 7 + [i32] * 9 + [f32, i32, vp]
    lib.pa_copy_blocks.restype = i32
    lib.pa_copy_blocks.argtypes = [vp] * 3 + [i32] * 6 + [vp]
    lib.pa_gather_kv.restype = i32
    lib.pa_gather_kv.argtypes = [vp] * 7 + [i32] * 8 + [vp]
    lib.pa_reshape_and_cache_fp8.restype = i32
    lib.pa_reshape_and_cache_fp8.argtypes = [vp] * 5 + [i32] * 6 + [f32, f32, vp]
    lib.pa_swap_blocks.restype = i32
    lib.pa_swap_blocks.argtypes = [vp] * 5 + [i32] * 6 + [i32, vp]
    lib.pa_decode_step_fp8.restype = i32
    lib.pa_decode_step_fp8.argtypes = [vp] * 9 + [i32] * 8 + [f32] * 3 + [i32, i32, vp, sz, vp,
                                                                          vp]
    lib.pa_decode_step_shared_prefix.restype = i32
    lib.pa_decode_step_shared_prefix.argtypes = [vp] * 9 + [i32] * 9 + [f32, i32, vp, vp]
    lib.pa_read_probe.restype = i32
    lib.pa_read_probe.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp]
    lib.pa_coexec_probe.restype = i32
    lib.pa_coexec_probe.argtypes = [i32, i32, i32, i32, vp, vp]
    lib.pa_plan_pairs.restype = i32
    lib.pa_plan_pairs.argtypes = [vp, i32, i32, i32, i32, i32, vp]
    lib.pa_decode_step_noalloc.restype = i32
    lib.pa_decode_step_noalloc.argtypes = [vp] * 9 + [i32] * 8 + [f32, i32, i32, vp, vp]
    lib.pa_paged_attention_fp8.restype = i32
    lib.pa_paged_attention_fp8.argtypes = [vp] * 6 + [i32] * 8 + [f32] * 3 + [i32, i32, vp, sz,
                                                                              vp, vp]
    lib.pa_set_decode_math.restype = i32
    lib.pa_set_decode_math.argtypes = [i32]
    lib.pa_get_decode_math.restype = i32
    lib.pa_get_decode_math.argtypes = []
    _lib = lib
    return lib


def _check(status: int, what: str) -> None:
    if status != PA_OK:
        msg = load_library().pa_status_string(status).decode()
        raise _ERRORS.get(status, RuntimeError)(f"{what}: {msg}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPE_CODES:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")
    return _DTYPE_CODES[t.dtype]


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device, stream) -> int:
    s = torch.cuda.current_stream(device) if stream is None else stream
    return s.cuda_stream


def _record(stream, made) -> None:
    """Tensors this module allocated (on torch's current stream) that a kernel on the
    caller's `stream` still uses after the call returns: the caching allocator must not
    hand their memory to another tensor before that stream's work is done."""
    if stream is None:
        return
    for t in made:
        if t is not None:
            t.record_stream(stream)


def _host_lens(host_context_lens, num_seqs: int):
    """(pointer, holder) of an optional host int32 copy of context_lens [num_seqs]."""
    if host_context_lens is None:
        return None, None
    if isinstance(host_context_lens, torch.Tensor):
        if host_context_lens.is_cuda:
            raise ValueError("host_context_lens must be in host memory")
        arr = host_context_lens.detach().to(torch.int32).contiguous()
        ptr = arr.data_ptr()
    else:
        import numpy as np
        arr = np.ascontiguousarray(host_context_lens, dtype=np.int32)
        ptr = arr.ctypes.data
    if arr.shape != (num_seqs,):
        raise ValueError(f"host_context_lens must be [{num_seqs}], got {tuple(arr.shape)}")
    return ptr, arr


def _require(t: torch.Tensor, name: str, device: torch.device, dtype=None) -> None:
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def chunk_elems(dtype: torch.dtype) -> int:
    """Elements of one 16-byte chunk (8 for bfloat16, 4 for float32, 16 for FP8 codes)."""
    return 16 // torch.empty((), dtype=dtype).element_size()


def k_cache_shape(num_blocks, num_kv_heads, head_dim, block_size, dtype=None) -> tuple:
    """K pool shape: token-major [NB, Hkv, BS, D]."""
    return (num_blocks, num_kv_heads, block_size, head_dim)


def v_group(block_size: int, dtype: torch.dtype) -> int:
    """Tokens per V group: one 16-byte chunk of a channel, at most the block."""
    return min(chunk_elems(dtype), block_size)


def v_cache_shape(num_blocks, num_kv_heads, head_dim, block_size, dtype) -> tuple:
    """V pool shape: token groups of X = v_group(block_size, dtype) tokens, channel-major
    within a group: [NB, Hkv, BS / X, D, X]."""
    X = v_group(block_size, dtype)
    return (num_blocks, num_kv_heads, block_size // X, head_dim, X)


def _cache_dims(k_cache: torch.Tensor, v_cache: torch.Tensor):
    if k_cache.dim() != 4 or v_cache.dim() != 5:
        raise ValueError("k_cache must be [NB, Hkv, BS, D] and v_cache [NB, Hkv, BS / X, D, X]")
    NB, Hkv, BS, D = k_cache.shape
    want = v_cache_shape(NB, Hkv, D, BS, k_cache.dtype)
    if tuple(v_cache.shape) != want or v_cache.dtype != k_cache.dtype:
        raise ValueError(f"v_cache must be {want} of {k_cache.dtype}, got "
                         f"{tuple(v_cache.shape)} of {v_cache.dtype}")
    return NB, Hkv, D, BS


# ---------------------------------------------------------------------------
def default_partition_size(num_seqs: int, num_kv_heads: int, max_context_len: int,
                           dtype: torch.dtype) -> int:
    return load_library().pa_default_partition_size(num_seqs, num_kv_heads, max_context_len,
                                                    _DTYPE_CODES[dtype])


def workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                   max_context_len: int, partition_size: int = 0,
                   dtype: torch.dtype = torch.bfloat16) -> int:
    return int(load_library().pa_paged_attention_workspace_size(
        num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, partition_size,
        _DTYPE_CODES[dtype]))


def paged_attention(query: torch.Tensor, block_table: torch.Tensor, context_lens: torch.Tensor,
                    k_cache: torch.Tensor, v_cache: torch.Tensor, scale: float, *,
                    max_context_len: int, out: torch.Tensor | None = None,
                    partition_size: int = 0, workspace: torch.Tensor | None = None,
                    stream=None, host_context_lens=None) -> torch.Tensor:
    """Decode attention of query [S, Hq, D] over the paged caches (see pagedattn.h).
    host_context_lens: optional host copy of context_lens (numpy or CPU tensor)."""
    lib = load_library()
    dev = query.device
    _require(query, "query", dev)
    NB, Hkv, D, BS = _cache_dims(k_cache, v_cache)
    _require(k_cache, "k_cache", dev, query.dtype)
    _require(v_cache, "v_cache", dev, query.dtype)
    _require(block_table, "block_table", dev, torch.int32)
    _require(context_lens, "context_lens", dev, torch.int32)
    if query.dim() != 3 or query.shape[2] != D:
        raise ValueError(f"query must be [S, Hq, {D}], got {tuple(query.shape)}")
    S, Hq, _ = query.shape
    if block_table.dim() != 2 or block_table.shape[0] != S or tuple(context_lens.shape) != (S,):
        raise ValueError("block_table must be [S, MB] and context_lens [S]")
    MB = block_table.shape[1]
    made = []
    if out is None:
        out = torch.empty_like(query)
        made.append(out)
    _require(out, "out", dev, query.dtype)
    if tuple(out.shape) != tuple(query.shape):
        raise ValueError("out must have the shape of query")
    code = _dtype_code(query)
    need = workspace_size(S, Hq, Hkv, D, max_context_len, partition_size, query.dtype)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        made.append(workspace)
    if workspace is not None:
        _require(workspace, "workspace", dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    hl, _hold = _host_lens(host_context_lens, S)
    st = lib.pa_paged_attention(_ptr(out), _ptr(query), _ptr(block_table), _ptr(context_lens),
                                _ptr(k_cache), _ptr(v_cache), S, Hq, Hkv, D, BS, MB, NB,
                                int(max_context_len), float(scale), code, int(partition_size),
                                _ptr(workspace), ws_bytes, _stream(dev, stream), hl)
    _check(st, "pa_paged_attention")
    _record(stream, made)
    return out


def _decode_step_args(query, key, value, slot_mapping, block_table, context_lens, k_cache,
                      v_cache, scale, max_context_len, out, partition_size, workspace, stream,
                      host_context_lens=None, need_workspace=True):
    """Checked argument tuple of pa_decode_step (allocates out/workspace when None)."""
    dev = query.device
    _require(query, "query", dev)
    NB, Hkv, D, BS = _cache_dims(k_cache, v_cache)
    for t, name in ((k_cache, "k_cache"), (v_cache, "v_cache"), (key, "key"), (value, "value")):
        _require(t, name, dev, query.dtype)
    _require(slot_mapping, "slot_mapping", dev, torch.int64)
    _require(block_table, "block_table", dev, torch.int32)
    _require(context_lens, "context_lens", dev, torch.int32)
    if query.dim() != 3 or query.shape[2] != D:
        raise ValueError(f"query must be [S, Hq, {D}], got {tuple(query.shape)}")
    S, Hq, _ = query.shape
    if tuple(key.shape) != (S, Hkv, D) or tuple(value.shape) != (S, Hkv, D) or \
            tuple(slot_mapping.shape) != (S,):
        raise ValueError(f"key/value must be [{S}, {Hkv}, {D}] and slot_mapping [{S}]")
    if block_table.dim() != 2 or block_table.shape[0] != S or tuple(context_lens.shape) != (S,):
        raise ValueError("block_table must be [S, MB] and context_lens [S]")
    made = []
    if out is None:
        out = torch.empty_like(query)
        made.append(out)
    _require(out, "out", dev, query.dtype)
    if tuple(out.shape) != tuple(query.shape):
        raise ValueError("out must have the shape of query")
    need = workspace_size(S, Hq, Hkv, D, max_context_len, partition_size, query.dtype) \
        if need_workspace else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        made.append(workspace)
    if workspace is not None:
        _require(workspace, "workspace", dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    hl, hold = _host_lens(host_context_lens, S)
    args = (_ptr(out), _ptr(query), _ptr(key), _ptr(value), _ptr(slot_mapping), _ptr(block_table),
            _ptr(context_lens), _ptr(k_cache), _ptr(v_cache), S, Hq, Hkv, D, BS,
            block_table.shape[1], NB, int(max_context_len), float(scale), _dtype_code(query),
            int(partition_size), _ptr(workspace), ws_bytes, _stream(dev, stream), hl)
    keep = (query, key, value, slot_mapping, block_table, context_lens, k_cache, v_cache, out,
            workspace, hold)
    return args, out, keep, made


def decode_step(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                slot_mapping: torch.Tensor, block_table: torch.Tensor, context_lens: torch.Tensor,
                k_cache: torch.Tensor, v_cache: torch.Tensor, scale: float, *,
                max_context_len: int, out: torch.Tensor | None = None, partition_size: int = 0,
                workspace: torch.Tensor | None = None, stream=None,
                host_context_lens=None) -> torch.Tensor:
    """One fused step: store key/value [S, Hkv, D] at slot_mapping [S], then decode
    attention of query [S, Hq, D] (see pa_decode_step in pagedattn.h)."""
    lib = load_library()
    args, out, _, made = _decode_step_args(query, key, value, slot_mapping, block_table,
                                           context_lens, k_cache, v_cache, scale,
                                           max_context_len, out, partition_size, workspace,
                                           stream, host_context_lens)
    _check(lib.pa_decode_step(*args), "pa_decode_step")
    _record(stream, made)
    return out


def decode_step_noalloc(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                        slot_mapping: torch.Tensor, block_table: torch.Tensor,
                        context_lens: torch.Tensor, k_cache: torch.Tensor,
                        v_cache: torch.Tensor, scale: float, *, max_context_len: int,
                        out: torch.Tensor, partition_size: int = 0, stream=None,
                        host_context_lens=None) -> torch.Tensor:
    """decode_step without a workspace and without allocating: the library's fixed
    per-GPU scratch holds the partitions' partial results (pa_decode_step_noalloc).
    `out` must be given; calls that overlap on one GPU race on the scratch."""
    if out is None:
        raise ValueError("decode_step_noalloc allocates nothing: pass out")
    lib = load_library()
    args, out, _, made = _decode_step_args(query, key, value, slot_mapping, block_table,
                                           context_lens, k_cache, v_cache, scale,
                                           max_context_len, out, partition_size, None, stream,
                                           host_context_lens, need_workspace=False)
    assert not made
    # pa_decode_step_noalloc takes pa_decode_step's arguments minus workspace and its size
    _check(lib.pa_decode_step_noalloc(*(args[:20] + args[22:])), "pa_decode_step_noalloc")
    return out


def _shared_prefix_args(query, key, value, slot_mapping, block_table, context_lens, k_cache,
                        v_cache, scale, prefix_blocks, max_context_len, out, stream,
                        host_context_lens):
    dev = query.device
    _require(query, "query", dev)
    NB, Hkv, D, BS = _cache_dims(k_cache, v_cache)
    _require(k_cache, "k_cache", dev, query.dtype)
    _require(v_cache, "v_cache", dev, query.dtype)
    _require(block_table, "block_table", dev, torch.int32)
    _require(context_lens, "context_lens", dev, torch.int32)
    if query.dim() != 3 or query.shape[2] != D:
        raise ValueError(f"query must be [S, Hq, {D}], got {tuple(query.shape)}")
    S, Hq, _ = query.shape
    if block_table.dim() != 2 or block_table.shape[0] != S or tuple(context_lens.shape) != (S,):
        raise ValueError("block_table must be [S, MB] and context_lens [S]")
    if (slot_mapping is None) != (key is None) or (key is None) != (value is None):
        raise ValueError("key, value and slot_mapping come together")
    if slot_mapping is not None:
        for t, name in ((key, "key"), (value, "value")):
            _require(t, name, dev, query.dtype)
        _require(slot_mapping, "slot_mapping", dev, torch.int64)
        if tuple(key.shape) != (S, Hkv, D) or tuple(value.shape) != (S, Hkv, D) or \
                tuple(slot_mapping.shape) != (S,):
            raise ValueError(f"key/value must be [{S}, {Hkv}, {D}] and slot_mapping [{S}]")
    made = []
    if out is None:
        out = torch.empty_like(query)
        made.append(out)
    _require(out, "out", dev, query.dtype)
    if tuple(out.shape) != tuple(query.shape):
        raise ValueError("out must have the shape of query")
    hl, hold = _host_lens(host_context_lens, S)
    args = (_ptr(out), _ptr(query), _ptr(key), _ptr(value), _ptr(slot_mapping),
            _ptr(block_table), _ptr(context_lens), _ptr(k_cache), _ptr(v_cache), S, Hq, Hkv, D,
            BS, block_table.shape[1], NB, int(max_context_len), int(prefix_blocks),
            float(scale), _dtype_code(query), _stream(dev, stream), hl)
    keep = (query, key, value, slot_mapping, block_table, context_lens, k_cache, v_cache, out,
            hold)
    return args, out, keep, made


def decode_step_shared_prefix(query: torch.Tensor, key, value, slot_mapping,
                              block_table: torch.Tensor, context_lens: torch.Tensor,
                              k_cache: torch.Tensor, v_cache: torch.Tensor, scale: float, *,
                              prefix_blocks: int, max_context_len: int,
                              out: torch.Tensor | None = None, stream=None,
                              host_context_lens=None) -> torch.Tensor:
    """The fused decode step when every sequence's first `prefix_blocks` table entries
    name the same shared blocks (pa_decode_step_shared_prefix).  key, value and
    slot_mapping may all be None: decode attention alone."""
    args, out, _, made = _shared_prefix_args(query, key, value, slot_mapping, block_table,
                                             context_lens, k_cache, v_cache, scale,
                                             prefix_blocks, max_context_len, out, stream,
                                             host_context_lens)
    _check(load_library().pa_decode_step_shared_prefix(*args), "pa_decode_step_shared_prefix")
    _record(stream, made)
    return out


def prepare_decode_step_shared_prefix(query, key, value, slot_mapping, block_table,
                                      context_lens, k_cache, v_cache, scale, *,
                                      prefix_blocks: int, max_context_len: int, out,
                                      stream=None, host_context_lens=None) -> PreparedCall:
    """Check the arguments of decode_step_shared_prefix once and return a re-launchable
    call (it runs once)."""
    args, out, keep, _ = _shared_prefix_args(query, key, value, slot_mapping, block_table,
                                             context_lens, k_cache, v_cache, scale,
                                             prefix_blocks, max_context_len, out, stream,
                                             host_context_lens)
    call = PreparedCall(load_library().pa_decode_step_shared_prefix, args,
                        "pa_decode_step_shared_prefix", keep)
    call()
    return call


def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, slot_mapping: torch.Tensor,
                      k_cache: torch.Tensor, v_cache: torch.Tensor, stream=None) -> None:
    """Store key/value [T, Hkv, D] at slot_mapping [T] (int64) in the caches, in place."""
    lib = load_library()
    dev = key.device
    NB, Hkv, D, BS = _cache_dims(k_cache, v_cache)
    for t, name in ((key, "key"), (value, "value"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _require(t, name, dev, k_cache.dtype)
    _require(slot_mapping, "slot_mapping", dev, torch.int64)
    T = key.shape[0]
    if tuple(key.shape) != (T, Hkv, D) or tuple(value.shape) != (T, Hkv, D) or \
            tuple(slot_mapping.shape) != (T,):
        raise ValueError(f"key/value must be [T, {Hkv}, {D}] and slot_mapping [T]")
    st = lib.pa_reshape_and_cache(_ptr(key), _ptr(value), _ptr(slot_mapping), _ptr(k_cache),
                                  _ptr(v_cache), T, Hkv, D, BS, NB, _dtype_code(key),
                                  _stream(dev, stream))
    _check(st, "pa_reshape_and_cache")


# ---------------------------------------------------------------------------
# FP8 (E4M3) pools: uint8 tensors of codes, one scale per tensor (see pagedattn.h)
# ---------------------------------------------------------------------------
def _fp8_cache_dims(k_cache: torch.Tensor, v_cache: torch.Tensor):
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise TypeError("FP8 pools are uint8 tensors of E4M3 codes")
    return _cache_dims(k_cache, v_cache)


def _reshape_fp8_args(key, value, slot_mapping, k_cache, v_cache, k_scale, v_scale, stream):
    dev = key.device
    NB, Hkv, D, BS = _fp8_cache_dims(k_cache, v_cache)
    _require(key, "key", dev)
    _require(value, "value", dev, key.dtype)
    _require(k_cache, "k_cache", dev)
    _require(v_cache, "v_cache", dev)
    _require(slot_mapping, "slot_mapping", dev, torch.int64)
    T = key.shape[0]
    if tuple(key.shape) != (T, Hkv, D) or tuple(value.shape) != (T, Hkv, D) or \
            tuple(slot_mapping.shape) != (T,):
        raise ValueError(f"key/value must be [T, {Hkv}, {D}] and slot_mapping [T]")
    return (_ptr(key), _ptr(value), _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache), T, Hkv,
            D, BS, NB, _dtype_code(key), float(k_scale), float(v_scale), _stream(dev, stream))


def reshape_and_cache_fp8(key: torch.Tensor, value: torch.Tensor, slot_mapping: torch.Tensor,
                          k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: float,
                          v_scale: float, stream=None) -> None:
    """Quantise key/value [T, Hkv, D] (f32 or bf16) into the FP8 pools at slot_mapping [T]."""
    args = _reshape_fp8_args(key, value, slot_mapping, k_cache, v_cache, k_scale, v_scale,
                             stream)
    _check(load_library().pa_reshape_and_cache_fp8(*args), "pa_reshape_and_cache_fp8")


def _attention_fp8_args(query, block_table, context_lens, k_cache, v_cache, scale, k_scale,
                        v_scale, max_context_len, out, partition_size, workspace, stream,
                        host_context_lens=None):
    dev = query.device
    NB, Hkv, D, BS = _fp8_cache_dims(k_cache, v_cache)
    _require(query, "query", dev)
    _require(k_cache, "k_cache", dev)
    _require(v_cache, "v_cache", dev)
    _require(block_table, "block_table", dev, torch.int32)
    _require(context_lens, "context_lens", dev, torch.int32)
    if query.dim() != 3 or query.shape[2] != D:
        raise ValueError(f"query must be [S, Hq, {D}], got {tuple(query.shape)}")
    S, Hq, _ = query.shape
    if block_table.dim() != 2 or block_table.shape[0] != S or tuple(context_lens.shape) != (S,):
        raise ValueError("block_table must be [S, MB] and context_lens [S]")
    made = []
    if out is None:
        out = torch.empty_like(query)
        made.append(out)
    _require(out, "out", dev, query.dtype)
    if tuple(out.shape) != tuple(query.shape):
        raise ValueError("out must have the shape of query")
    need = workspace_size(S, Hq, Hkv, D, max_context_len, partition_size, torch.bfloat16)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        made.append(workspace)
    if workspace is not None:
        _require(workspace, "workspace", dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(out), _ptr(query), _ptr(block_table), _ptr(context_lens), _ptr(k_cache),
            _ptr(v_cache), S, Hq, Hkv, D, BS, block_table.shape[1], NB, int(max_context_len),
            float(scale), float(k_scale), float(v_scale), _dtype_code(query),
            int(partition_size), _ptr(workspace), ws_bytes, _stream(dev, stream))
    hl, hold = _host_lens(host_context_lens, S)
    args = args + (hl,)
    keep = (query, block_table, context_lens, k_cache, v_cache, out, workspace, hold)
    return args, out, keep, made


def paged_attention_fp8(query: torch.Tensor, block_table: torch.Tensor,
                        context_lens: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                        scale: float, k_scale: float, v_scale: float, *, max_context_len: int,
                        out: torch.Tensor | None = None, partition_size: int = 0,
                        workspace: torch.Tensor | None = None, stream=None,
                        host_context_lens=None) -> torch.Tensor:
    """Decode attention of bf16 query [S, Hq, D] over FP8 pools (see pagedattn.h)."""
    args, out, _, made = _attention_fp8_args(query, block_table, context_lens, k_cache, v_cache,
                                             scale, k_scale, v_scale, max_context_len, out,
                                             partition_size, workspace, stream,
                                             host_context_lens)
    _check(load_library().pa_paged_attention_fp8(*args), "pa_paged_attention_fp8")
    _record(stream, made)
    return out


def _decode_step_fp8_args(query, key, value, slot_mapping, block_table, context_lens, k_cache,
                          v_cache, scale, k_scale, v_scale, max_context_len, out,
                          partition_size, workspace, stream, host_context_lens=None):
    dev = query.device
    NB, Hkv, D, BS = _fp8_cache_dims(k_cache, v_cache)
    S = query.shape[0] if query.dim() == 3 else -1
    for t, name in ((key, "key"), (value, "value")):
        _require(t, name, dev, query.dtype)
    _require(slot_mapping, "slot_mapping", dev, torch.int64)
    if tuple(key.shape) != (S, Hkv, D) or tuple(value.shape) != (S, Hkv, D) or \
            tuple(slot_mapping.shape) != (S,):
        raise ValueError(f"key/value must be [{S}, {Hkv}, {D}] and slot_mapping [{S}]")
    args, out, keep, made = _attention_fp8_args(query, block_table, context_lens, k_cache,
                                                v_cache, scale, k_scale, v_scale,
                                                max_context_len, out, partition_size, workspace,
                                                stream, host_context_lens)
    # pa_decode_step_fp8 takes key, value and slot_mapping after query
    args = args[:2] + (_ptr(key), _ptr(value), _ptr(slot_mapping)) + args[2:]
    return args, out, keep + (key, value, slot_mapping), made


def decode_step_fp8(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                    slot_mapping: torch.Tensor, block_table: torch.Tensor,
                    context_lens: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    scale: float, k_scale: float, v_scale: float, *, max_context_len: int,
                    out: torch.Tensor | None = None, partition_size: int = 0,
                    workspace: torch.Tensor | None = None, stream=None,
                    host_context_lens=None) -> torch.Tensor:
    """One fused step over FP8 pools: quantise key/value [S, Hkv, D] (bf16) into
    slot_mapping [S], then decode attention of query [S, Hq, D] (see pa_decode_step_fp8)."""
    args, out, _, made = _decode_step_fp8_args(query, key, value, slot_mapping, block_table,
                                               context_lens, k_cache, v_cache, scale, k_scale,
                                               v_scale, max_context_len, out, partition_size,
                                               workspace, stream, host_context_lens)
    _check(load_library().pa_decode_step_fp8(*args), "pa_decode_step_fp8")
    _record(stream, made)
    return out


def paged_prefill(query: torch.Tensor, query_start_loc: torch.Tensor, block_table: torch.Tensor,
                  context_lens: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                  scale: float, *, max_query_len: int, out: torch.Tensor | None = None,
                  stream=None) -> torch.Tensor:
    """Causal attention of each sequence's chunk of new tokens (query [T, Hq, D], rows
    query_start_loc[s] .. query_start_loc[s+1] - 1) over its paged K/V (pa_paged_prefill)."""
    lib = load_library()
    dev = query.device
    _require(query, "query", dev)
    NB, Hkv, D, BS = _cache_dims(k_cache, v_cache)
    _require(k_cache, "k_cache", dev, query.dtype)
    _require(v_cache, "v_cache", dev, query.dtype)
    _require(query_start_loc, "query_start_loc", dev, torch.int32)
    _require(block_table, "block_table", dev, torch.int32)
    _require(context_lens, "context_lens", dev, torch.int32)
    if query.dim() != 3 or query.shape[2] != D:
        raise ValueError(f"query must be [T, Hq, {D}], got {tuple(query.shape)}")
    T, Hq, _ = query.shape
    S = context_lens.shape[0]
    if tuple(query_start_loc.shape) != (S + 1,) or block_table.dim() != 2 or \
            block_table.shape[0] != S:
        raise ValueError("query_start_loc must be [S + 1] and block_table [S, MB]")
    made = []
    if out is None:
        out = torch.empty_like(query)
        made.append(out)
    _require(out, "out", dev, query.dtype)
    if tuple(out.shape) != tuple(query.shape):
        raise ValueError("out must have the shape of query")
    st = lib.pa_paged_prefill(_ptr(out), _ptr(query), _ptr(query_start_loc), _ptr(block_table),
                              _ptr(context_lens), _ptr(k_cache), _ptr(v_cache), S, Hq, Hkv, D,
                              BS, block_table.shape[1], NB, T, int(max_query_len), float(scale),
                              _dtype_code(query), _stream(dev, stream))
    _check(st, "pa_paged_prefill")
    _record(stream, made)
    return out


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, block_mapping: torch.Tensor,
                stream=None) -> None:
    """Copy physical block src to dst for every (src, dst) row of block_mapping [n, 2]
    (int64), in place (see pa_copy_blocks)."""
    lib = load_library()
    dev = k_cache.device
    NB, Hkv, D, BS = _cache_dims(k_cache, v_cache)
    _require(k_cache, "k_cache", dev)
    _require(v_cache, "v_cache", dev, k_cache.dtype)
    _require(block_mapping, "block_mapping", dev, torch.int64)
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [n, 2] (src, dst)")
    _pool_code(k_cache)
    st = lib.pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(block_mapping),
                            block_mapping.shape[0], Hkv, D, BS, NB, _pool_code(k_cache),
                            _stream(dev, stream))
    _check(st, "pa_copy_blocks")


def prepare_copy_blocks(k_cache, v_cache, block_mapping, stream=None) -> PreparedCall:
    """Check the arguments of copy_blocks once and return a re-launchable call."""
    lib = load_library()
    copy_blocks(k_cache, v_cache, block_mapping, stream=stream)
    NB, Hkv, D, BS = _cache_dims(k_cache, v_cache)
    args = (_ptr(k_cache), _ptr(v_cache), _ptr(block_mapping), block_mapping.shape[0], Hkv, D,
            BS, NB, _pool_code(k_cache), _stream(k_cache.device, stream))
    return PreparedCall(lib.pa_copy_blocks, args, "pa_copy_blocks",
                        (k_cache, v_cache, block_mapping))


def _pool_code(t: torch.Tensor) -> int:
    if t.dtype not in _POOL_CODES:
        raise TypeError(f"unsupported pool dtype {t.dtype}; use float32, bfloat16 or uint8 (FP8)")
    return _POOL_CODES[t.dtype]


def _gpu_reachable(t: torch.Tensor, name: str) -> None:
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError(f"{name} must be on the GPU or in pinned host memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _swap_args(src_k, src_v, dst_k, dst_v, block_mapping, stream):
    for t, name in ((src_k, "src_k"), (src_v, "src_v"), (dst_k, "dst_k"), (dst_v, "dst_v"),
                    (block_mapping, "block_mapping")):
        _gpu_reachable(t, name)
    sNB, Hkv, D, BS = _cache_dims(src_k, src_v)
    dNB, dHkv, dD, dBS = _cache_dims(dst_k, dst_v)
    if (dHkv, dD, dBS) != (Hkv, D, BS) or dst_k.dtype != src_k.dtype:
        raise ValueError("source and destination pools must share layout and dtype")
    if block_mapping.dtype != torch.int64 or block_mapping.dim() != 2 or \
            block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be an int64 [n, 2] tensor (src, dst)")
    dev = next((t.device for t in (src_k, dst_k, block_mapping) if t.is_cuda), None)
    if dev is None:
        raise ValueError("one side of a swap must be on the GPU")
    return (_ptr(src_k), _ptr(src_v), _ptr(dst_k), _ptr(dst_v), _ptr(block_mapping),
            block_mapping.shape[0], Hkv, D, BS, sNB, dNB, _pool_code(src_k), _stream(dev, stream))


def swap_blocks(src_k: torch.Tensor, src_v: torch.Tensor, dst_k: torch.Tensor,
                dst_v: torch.Tensor, block_mapping: torch.Tensor, stream=None) -> None:
    """Copy block s of the source pools to block d of the destination pools for every (s, d)
    row of block_mapping; one side is typically in pinned host memory (see pa_swap_blocks)."""
    args = _swap_args(src_k, src_v, dst_k, dst_v, block_mapping, stream)
    _check(load_library().pa_swap_blocks(*args), "pa_swap_blocks")


def prepare_swap_blocks(src_k, src_v, dst_k, dst_v, block_mapping, stream=None) -> PreparedCall:
    """Check the arguments of swap_blocks once and return a re-launchable call."""
    args = _swap_args(src_k, src_v, dst_k, dst_v, block_mapping, stream)
    call = PreparedCall(load_library().pa_swap_blocks, args, "pa_swap_blocks",
                        (src_k, src_v, dst_k, dst_v, block_mapping))
    call()
    return call


def gather_kv(block_table: torch.Tensor, context_lens: torch.Tensor, k_cache: torch.Tensor,
              v_cache: torch.Tensor, *, seq_offsets: torch.Tensor, total_tokens: int,
              max_context_len: int, stream=None):
    """Contiguous K and V [total_tokens, Hkv, D] of every sequence (diagnostic copy)."""
    lib = load_library()
    dev = k_cache.device
    NB, Hkv, D, BS = _cache_dims(k_cache, v_cache)
    _require(k_cache, "k_cache", dev)
    _require(v_cache, "v_cache", dev)
    _require(block_table, "block_table", dev, torch.int32)
    _require(context_lens, "context_lens", dev, torch.int32)
    _require(seq_offsets, "seq_offsets", dev, torch.int64)
    S, MB = block_table.shape
    k_out = torch.empty((total_tokens, Hkv, D), dtype=k_cache.dtype, device=dev)
    v_out = torch.empty_like(k_out)
    st = lib.pa_gather_kv(_ptr(k_out), _ptr(v_out), _ptr(seq_offsets), _ptr(block_table),
                          _ptr(context_lens), _ptr(k_cache), _ptr(v_cache), S, Hkv, D, BS, MB,
                          NB, int(max_context_len), _dtype_code(k_cache), _stream(dev, stream))
    _check(st, "pa_gather_kv")
    _record(stream, (k_out, v_out))
    return k_out, v_out


def read_probe(buf: torch.Tensor, piece_offsets: torch.Tensor, piece_bytes: int,
               workgroups: int, in_flight: int, sink: torch.Tensor, stream=None,
               nontemporal: bool = False) -> None:
    """Read-bandwidth probe (pa_read_probe): read the pieces of `buf` at `piece_offsets`
    (int64 byte offsets) and leave checksums in `sink` (int32, workgroups * 256), with
    default-policy or streaming (nt) loads."""
    dev = buf.device
    _require(buf, "buf", dev)
    _require(piece_offsets, "piece_offsets", dev, torch.int64)
    _require(sink, "sink", dev, torch.int32)
    if sink.numel() < workgroups * 256:
        raise ValueError(f"sink must hold {workgroups * 256} entries")
    n = piece_offsets.numel()
    size = buf.numel() * buf.element_size()
    if n and piece_bytes > size:
        raise ValueError("pieces larger than the buffer")
    _check(load_library().pa_read_probe(_ptr(buf), _ptr(piece_offsets), n, int(piece_bytes),
                                        int(workgroups), int(in_flight), int(bool(nontemporal)),
                                        _ptr(sink), _stream(dev, stream)), "pa_read_probe")


COEXEC_MODES = {"mfma": 0, "valu": 1, "interleaved": 2, "split": 3, "placement": 4}


def coexec_probe(mode: str, workgroups: int, waves_per_workgroup: int, iters: int,
                 out: torch.Tensor, stream=None) -> None:
    """Co-execution probe (pa_coexec_probe): MFMA work, VALU work, both interleaved in
    every wave, or split between the two waves of each SIMD; time it with events.  Mode
    "placement" does no work and writes, per thread, the SIMD its wave runs on."""
    dev = out.device
    _require(out, "out", dev, torch.float32)
    if mode not in COEXEC_MODES:
        raise ValueError(f"mode must be one of {sorted(COEXEC_MODES)}")
    if out.numel() < workgroups * waves_per_workgroup * 64:
        raise ValueError(f"out must hold {workgroups * waves_per_workgroup * 64} floats")
    _check(load_library().pa_coexec_probe(COEXEC_MODES[mode], int(workgroups),
                                          int(waves_per_workgroup), int(iters), _ptr(out),
                                          _stream(dev, stream)), "pa_coexec_probe")


def plan_pairs(host_lens, block_size: int, max_len: int, step_tokens: int,
               waves: int) -> np.ndarray:
    """The paired mode's host plan (pa_plan_pairs; no GPU work): uint32 [pairs, 2] of
    (sA | sB << 16, blocks of sA | blocks of sB << 12 | waves of sA << 24)."""
    lens = np.ascontiguousarray(np.asarray(host_lens, dtype=np.int32))
    if lens.ndim != 1:
        raise ValueError("host_lens must be one-dimensional")
    out = np.zeros(((lens.size + 1) // 2, 2), dtype=np.uint32)
    _check(load_library().pa_plan_pairs(lens.ctypes.data, int(lens.size), int(block_size),
                                        int(max_len), int(step_tokens), int(waves),
                                        out.ctypes.data), "pa_plan_pairs")
    return out


DECODE_MATH = {"mfma": 0, "valu": 1}


def set_decode_math(math: str) -> None:
    """Arithmetic of the bf16 decode calls from now on (pa_set_decode_math): "mfma"
    (matrix cores, the default) or "valu" (vector ALU; group sizes 1, 2 and 4)."""
    if math not in DECODE_MATH:
        raise ValueError(f"decode math must be one of {sorted(DECODE_MATH)}")
    _check(load_library().pa_set_decode_math(DECODE_MATH[math]), "pa_set_decode_math")


def get_decode_math() -> str:
    code = load_library().pa_get_decode_math()
    return {v: k for k, v in DECODE_MATH.items()}[code]


@contextlib.contextmanager
def decode_math(math: str):
    """Run the enclosed calls with the given decode arithmetic, then restore it."""
    before = get_decode_math()
    set_decode_math(math)
    try:
        yield
    finally:
        set_decode_math(before)


# ---------------------------------------------------------------------------
# prepared calls: validate once, then launch with fixed pointers (tight loops)
# ---------------------------------------------------------------------------
class PreparedCall:
    """A library call whose tensors were checked once; calling it launches again.

    The tensors are held so their memory stays valid; the stream is read at
    preparation time.
    """

    def __init__(self, fn, args: tuple, what: str, keep: tuple):
        self._fn, self._args, self._what, self._keep = fn, args, what, keep

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != PA_OK:
            _check(st, self._what)


def prepare_paged_attention(query, block_table, context_lens, k_cache, v_cache, scale, *,
                            max_context_len: int, out, partition_size: int = 0,
                            workspace=None, stream=None, host_context_lens=None) -> PreparedCall:
    """Check the arguments as paged_attention does and return a re-launchable call."""
    lib = load_library()
    dev = query.device
    need = workspace_size(query.shape[0], query.shape[1], k_cache.shape[1],
                          k_cache.shape[3], max_context_len, partition_size,
                          query.dtype) if k_cache.dim() == 4 and query.dim() == 3 else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    # one checked call validates every argument (and runs once)
    paged_attention(query, block_table, context_lens, k_cache, v_cache, scale,
                    max_context_len=max_context_len, out=out, partition_size=partition_size,
                    workspace=workspace, stream=stream, host_context_lens=host_context_lens)
    NB, Hkv, D, BS = _cache_dims(k_cache, v_cache)
    S, Hq, _ = query.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    hl, hold = _host_lens(host_context_lens, S)
    args = (_ptr(out), _ptr(query), _ptr(block_table), _ptr(context_lens), _ptr(k_cache),
            _ptr(v_cache), S, Hq, Hkv, D, BS, block_table.shape[1], NB, int(max_context_len),
            float(scale), _dtype_code(query), int(partition_size), _ptr(workspace), ws_bytes,
            _stream(dev, stream), hl)
    return PreparedCall(lib.pa_paged_attention, args, "pa_paged_attention",
                        (query, block_table, context_lens, k_cache, v_cache, out, workspace,
                         hold))


def prepare_reshape_and_cache(key, value, slot_mapping, k_cache, v_cache,
                              stream=None) -> PreparedCall:
    """Check the arguments as reshape_and_cache does and return a re-launchable call."""
    lib = load_library()
    reshape_and_cache(key, value, slot_mapping, k_cache, v_cache, stream=stream)
    NB, Hkv, D, BS = _cache_dims(k_cache, v_cache)
    args = (_ptr(key), _ptr(value), _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache),
            key.shape[0], Hkv, D, BS, NB, _dtype_code(key), _stream(key.device, stream))
    return PreparedCall(lib.pa_reshape_and_cache, args, "pa_reshape_and_cache",
                        (key, value, slot_mapping, k_cache, v_cache))


def prepare_decode_step(query, key, value, slot_mapping, block_table, context_lens, k_cache,
                        v_cache, scale, *, max_context_len: int, out, partition_size: int = 0,
                        workspace=None, stream=None, host_context_lens=None) -> PreparedCall:
    """Check the arguments of decode_step once and return a re-launchable call."""
    lib = load_library()
    args, out, keep, _ = _decode_step_args(query, key, value, slot_mapping, block_table,
                                           context_lens, k_cache, v_cache, scale,
                                           max_context_len, out, partition_size, workspace,
                                           stream, host_context_lens)
    call = PreparedCall(lib.pa_decode_step, args, "pa_decode_step", keep)
    call()
    return call


def prepare_reshape_and_cache_fp8(key, value, slot_mapping, k_cache, v_cache, k_scale, v_scale,
                                  stream=None) -> PreparedCall:
    """Check the arguments of reshape_and_cache_fp8 once and return a re-launchable call."""
    args = _reshape_fp8_args(key, value, slot_mapping, k_cache, v_cache, k_scale, v_scale,
                             stream)
    call = PreparedCall(load_library().pa_reshape_and_cache_fp8, args,
                        "pa_reshape_and_cache_fp8", (key, value, slot_mapping, k_cache, v_cache))
    call()
    return call


def prepare_paged_attention_fp8(query, block_table, context_lens, k_cache, v_cache, scale,
                                k_scale, v_scale, *, max_context_len: int, out,
                                partition_size: int = 0, workspace=None,
                                stream=None, host_context_lens=None) -> PreparedCall:
    """Check the arguments of paged_attention_fp8 once and return a re-launchable call."""
    args, out, keep, _ = _attention_fp8_args(query, block_table, context_lens, k_cache,
                                             v_cache, scale, k_scale, v_scale, max_context_len,
                                             out, partition_size, workspace, stream,
                                             host_context_lens)
    call = PreparedCall(load_library().pa_paged_attention_fp8, args, "pa_paged_attention_fp8",
                        keep)
    call()
    return call


def prepare_decode_step_fp8(query, key, value, slot_mapping, block_table, context_lens, k_cache,
                            v_cache, scale, k_scale, v_scale, *, max_context_len: int, out,
                            partition_size: int = 0, workspace=None,
                            stream=None, host_context_lens=None) -> PreparedCall:
    """Check the arguments of decode_step_fp8 once and return a re-launchable call."""
    args, out, keep, _ = _decode_step_fp8_args(query, key, value, slot_mapping, block_table,
                                               context_lens, k_cache, v_cache, scale, k_scale,
                                               v_scale, max_context_len, out, partition_size,
                                               workspace, stream, host_context_lens)
    call = PreparedCall(load_library().pa_decode_step_fp8, args, "pa_decode_step_fp8", keep)
    call()
    return call
