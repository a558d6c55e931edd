"""Python binding of libpagedattn.so (paged KV-cache attention for MI355X / gfx950).

Argument marshalling only: every function passes tensor data pointers, sizes
and the current HIP stream to the C entry point of the same name (declared in
include/pa.h) and raises on a non-OK status.  PyTorch is used for device
memory and streams; all compute runs in the library's HIP kernels.  There is
no fallback: importing this package fails if the library is not built.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedattn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python paged_kv_cache_134_amd/build.py` "
        "(or __graft_entry__.build()) first")

# Load torch first so that the library binds to the HIP runtime torch already
# loaded (same soname): device memory, streams and kernels then live in one
# runtime.  Without torch only the host-side block pool is usable.
try:
    import torch as _torch_mod  # noqa: F401
except ImportError:  # pragma: no cover
    _torch_mod = None

_lib = ctypes.CDLL(LIB_PATH)

# ---------------------------------------------------------------- constants
PA_OK = 0
STATUS_NAMES = {0: "PA_OK", 1: "PA_ERR_INVALID_ARGUMENT", 2: "PA_ERR_UNSUPPORTED",
                3: "PA_ERR_WORKSPACE_TOO_SMALL", 4: "PA_ERR_OUT_OF_BLOCKS", 5: "PA_ERR_HIP",
                6: "PA_ERR_METADATA"}
PA_F32, PA_BF16, PA_F16, PA_FP8_E4M3 = 0, 1, 2, 3
KV_DTYPE = {"f32": PA_F32, "bf16": PA_BF16, "f16": PA_F16, "e4m3": PA_FP8_E4M3}  # dtype names
NHD, HND = 0, 1

EXPORTED = [
    "pa_status_string", "pa_last_error", "pa_reshape_and_cache", "pa_reshape_and_cache_fp8",
    "pa_copy_blocks", "pa_swap_blocks", "pa_decode_workspace_size", "pa_decode_auto_partition", "pa_decode",
    "pa_decode_fp8", "pa_decode_partitions_fp8", "pa_decode_partitions",
    "pa_decode_reduce", "pa_decode_cascade_workspace_size", "pa_decode_cascade", "pa_decode_cascade_fp8", "pa_prefill", "pa_prefill_fp8",
    "pa_check_metadata", "pa_pool_create", "pa_pool_destroy", "pa_pool_add_seq", "pa_pool_fork",
    "pa_pool_append", "pa_pool_free_seq", "pa_pool_block_table", "pa_pool_seq_len",
    "pa_pool_num_free", "pa_pool_refcount", "pa_pool_add_seq_cached", "pa_pool_num_cached",
    "pa_stream_read_probe_sink_words", "pa_stream_read_probe", "pa_decode_static_scratch",
]

_i32, _i64, _f32, _vp, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
_pi32 = ctypes.POINTER(ctypes.c_int32)
_pi64 = ctypes.POINTER(ctypes.c_int64)

_sig = {
    "pa_status_string": (ctypes.c_char_p, [_i32]),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_reshape_and_cache": (_i32, [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                    _i32, _i32, _i32, _vp]),
    "pa_reshape_and_cache_fp8": (_i32, [_vp, _vp, _i32, _i64, _i64, _vp, _vp, _vp, _i32, _i32,
                                        _i32, _i32, _i32, _i32, _f32, _f32, _vp]),
    "pa_copy_blocks": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pa_swap_blocks": (_i32, [_vp, _vp, _vp, _vp, _pi32, _i32, _i64, _i32, _i32, _vp]),
    "pa_decode_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pa_decode_auto_partition": (_i32, [_i32, _i32, _i32, _i32, _i32, _i64]),
    "pa_decode": (_i32, [_vp, _i32, _vp, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _i32, _i32,
                         _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp]),
    "pa_decode_fp8": (_i32, [_vp, _i32, _vp, _i32, _vp, _vp, _f32, _f32, _i32, _vp, _i32, _vp,
                             _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp]),
    "pa_decode_partitions_fp8": (_i32, [_vp, _i32, _vp, _i32, _vp, _vp, _f32, _f32, _i32, _vp, _i32,
                                        _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                                        _vp, _sz, _vp]),
    "pa_decode_partitions": (_i32, [_vp, _i32, _vp, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _i32, _i32,
                                    _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp]),
    "pa_decode_reduce": (_i32, [_vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _sz, _vp]),
    "pa_decode_cascade_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode_cascade": (_i32, [_vp, _i32, _vp, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _i32,
                                 _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp]),
    "pa_decode_cascade_fp8": (_i32, [_vp, _i32, _vp, _i32, _vp, _vp, _f32, _f32, _i32, _vp, _i32,
                                     _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                     _i32, _vp, _sz, _vp]),
    "pa_prefill": (_i32, [_vp, _i32, _vp, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _vp, _i32, _i32,
                          _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp]),
    "pa_prefill_fp8": (_i32, [_vp, _i32, _vp, _i32, _vp, _vp, _f32, _f32, _i32, _vp, _i32, _vp, _vp,
                              _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp]),
    "pa_check_metadata": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pa_pool_create": (_i32, [_i32, _i32, _pi32, ctypes.POINTER(_vp)]),
    "pa_pool_destroy": (None, [_vp]),
    "pa_pool_add_seq": (_i32, [_vp, _pi32]),
    "pa_pool_fork": (_i32, [_vp, _i32, _pi32]),
    "pa_pool_add_seq_cached": (_i32, [_vp, _pi32, _i32, ctypes.c_uint64, _pi32, _pi32]),
    "pa_pool_num_cached": (_i32, [_vp]),
    "pa_pool_append": (_i32, [_vp, _i32, _i32, _pi64, _pi32, _i32, _pi32]),
    "pa_pool_free_seq": (_i32, [_vp, _i32]),
    "pa_pool_block_table": (_i32, [_vp, _i32, _pi32, _i32, _pi32]),
    "pa_pool_seq_len": (_i32, [_vp, _i32]),
    "pa_pool_num_free": (_i32, [_vp]),
    "pa_pool_refcount": (_i32, [_vp, _i32]),
    "pa_stream_read_probe_sink_words": (_i32, []),
    "pa_stream_read_probe": (_i32, [_vp, _sz, _vp, _vp]),
    "pa_decode_static_scratch": (_i32, [_vp, _i32, _vp, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32,
                                        _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp]),
}
PA_STATIC_SCRATCH_BYTES = 96 << 20  # the static split-K workspace of pa_decode_static_scratch
for _name, (_res, _args) in _sig.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class PagedAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        self.status_name = STATUS_NAMES.get(status, str(status))
        detail = _lib.pa_last_error().decode(errors="replace")
        super().__init__(f"{fn}: {self.status_name}: {detail}")


class OutOfBlocks(PagedAttnError):
    pass


def _check(fn: str, st: int) -> None:
    if st != PA_OK:
        raise (OutOfBlocks if st == 4 else PagedAttnError)(fn, st)


# ------------------------------------------------------------ torch helpers
def _torch():
    import torch  # imported lazily: the block pool needs no torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.float16: PA_F16,
         torch.uint8: PA_FP8_E4M3, torch.float8_e4m3fn: PA_FP8_E4M3}  # 1-byte caches hold E4M3 codes
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _dev(t, name: str, dtype=None, contiguous: bool = True):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _geom(key_cache, layout: int) -> Tuple[int, int, int, int]:
    """(num_blocks, block_size, num_kv_heads, head_size) of a pool tensor."""
    if key_cache.dim() != 4:
        raise ValueError("cache must be 4-D")
    nb, a, b, d = key_cache.shape
    return (nb, a, b, d) if layout == NHD else (nb, b, a, d)


# ---------------------------------------------------------------- entry points
def pa_reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, layout: int = NHD,
                         stream=None) -> None:
    """Scatter rows key/value [T, Hkv, D] into the pools at slot_mapping [T] (int64)."""
    torch = _torch()
    nb, bs, hkv, d = _geom(key_cache, layout)
    if key.dim() != 3 or key.shape[1:] != (hkv, d) or value.shape != key.shape:
        raise ValueError("key/value must be [T, num_kv_heads, head_size] matching the cache")
    if key.stride(2) != 1 or key.stride(1) != d or value.stride(2) != 1 or value.stride(1) != d:
        raise ValueError("key/value rows must be contiguous")
    if value_cache.shape != key_cache.shape or value_cache.dtype != key_cache.dtype:
        raise ValueError("value_cache must match key_cache")
    if key.dtype != key_cache.dtype or value.dtype != key_cache.dtype:
        raise TypeError("key/value dtype must equal the cache dtype")
    T = key.shape[0]
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [T]")
    _check("pa_reshape_and_cache", _lib.pa_reshape_and_cache(
        _dev(key, "key", contiguous=False), _dev(value, "value", contiguous=False),
        key.stride(0), value.stride(0), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(slot_mapping, "slot_mapping", torch.int64),
        T, hkv, d, bs, nb, _dtype_code(key_cache), layout, _stream(stream)))


def pa_reshape_and_cache_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale: float,
                             v_scale: float, layout: int = NHD, stream=None) -> None:
    """Quantising cache write: rows key/value [T, Hkv, D] (f32/bf16/f16) stored as
    E4M3 codes of x / k_scale and x / v_scale into uint8 pools at slot_mapping [T]."""
    torch = _torch()
    nb, bs, hkv, d = _geom(key_cache, layout)
    if key.dim() != 3 or key.shape[1:] != (hkv, d) or value.shape != key.shape:
        raise ValueError("key/value must be [T, num_kv_heads, head_size] matching the cache")
    if key.stride(2) != 1 or key.stride(1) != d or value.stride(2) != 1 or value.stride(1) != d:
        raise ValueError("key/value rows must be contiguous")
    if value_cache.shape != key_cache.shape or value_cache.dtype != key_cache.dtype:
        raise ValueError("value_cache must match key_cache")
    if _dtype_code(key_cache) != PA_FP8_E4M3 or key.dtype != value.dtype:
        raise TypeError("FP8 pools are uint8 (or float8_e4m3fn); key and value share a dtype")
    T = key.shape[0]
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [T]")
    _check("pa_reshape_and_cache_fp8", _lib.pa_reshape_and_cache_fp8(
        _dev(key, "key", contiguous=False), _dev(value, "value", contiguous=False),
        _dtype_code(key), key.stride(0), value.stride(0), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(slot_mapping, "slot_mapping", torch.int64),
        T, hkv, d, bs, nb, layout, float(k_scale), float(v_scale), _stream(stream)))


def pa_copy_blocks(key_cache, value_cache, block_pairs, layout: int = NHD, stream=None) -> None:
    """Copy whole blocks: block_pairs int32 [n, 2] = (source, destination)."""
    torch = _torch()
    nb, bs, hkv, d = _geom(key_cache, layout)
    n = int(block_pairs.shape[0]) if block_pairs.numel() else 0
    _check("pa_copy_blocks", _lib.pa_copy_blocks(
        _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
        _dev(block_pairs, "block_pairs", torch.int32) if n else None, n, hkv, d, bs, nb,
        _dtype_code(key_cache), _stream(stream)))


def pa_swap_blocks(src_key, src_value, dst_key, dst_value, block_pairs, stream=None) -> None:
    """Copy whole blocks between pools (device or pinned host tensors of one
    geometry and dtype): block_pairs [n, 2] (host ints) = (source block,
    destination block)."""
    torch = _torch()
    for t, name in ((src_key, "src_key"), (src_value, "src_value"), (dst_key, "dst_key"),
                    (dst_value, "dst_value")):
        if not isinstance(t, torch.Tensor) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor")
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError(f"{name} must be device memory or pinned host memory")
    if src_value.shape != src_key.shape or dst_key.shape[1:] != src_key.shape[1:] or \
            dst_value.shape != dst_key.shape or len({t.dtype for t in (src_key, src_value, dst_key, dst_value)}) != 1:
        raise ValueError("pools must share block geometry and dtype")
    pairs = np.ascontiguousarray(np.asarray(block_pairs, dtype=np.int32).reshape(-1, 2))
    block_bytes = src_key[0].numel() * src_key.element_size()
    _check("pa_swap_blocks", _lib.pa_swap_blocks(
        src_key.data_ptr(), src_value.data_ptr(), dst_key.data_ptr(), dst_value.data_ptr(),
        pairs.ctypes.data_as(_pi32), len(pairs), block_bytes, src_key.shape[0], dst_key.shape[0],
        _stream(stream)))


def pa_decode_workspace_size(num_seqs: int, num_heads: int, head_size: int, max_context_len: int,
                             partition_size: int) -> int:
    return int(_lib.pa_decode_workspace_size(num_seqs, num_heads, head_size, max_context_len,
                                             partition_size))


def pa_decode_auto_partition(num_seqs: int, num_heads: int, num_kv_heads: int, kv_dtype: int,
                             max_context_len: int, total_context_len: int = 0) -> int:
    return int(_lib.pa_decode_auto_partition(num_seqs, num_heads, num_kv_heads, kv_dtype,
                                             max_context_len, total_context_len))


def pa_decode(out, query, key_cache, value_cache, block_tables, context_lens, max_context_len: int,
              scale: float, layout: int = NHD, partition_size: int = -1, workspace=None,
              stream=None) -> None:
    """Decode attention; out [S, H, D] (float32 or the cache dtype)."""
    torch = _torch()
    nb, bs, hkv, d = _geom(key_cache, layout)
    S, H, D = query.shape
    if D != d or out.shape != query.shape:
        raise ValueError("query/out must be [num_seqs, num_heads, head_size]")
    if query.dtype != key_cache.dtype:
        raise TypeError("query dtype must equal the cache dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables [S, max_blocks] and context_lens [S] required")
    ws_ptr, ws_bytes = (None, 0)
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    _check("pa_decode", _lib.pa_decode(
        _dev(out, "out"), _dtype_code(out), _dev(query, "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dtype_code(key_cache), layout,
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), int(max_context_len), S, H, hkv, d, bs,
        nb, float(scale), int(partition_size), ws_ptr, ws_bytes, _stream(stream)))


def pa_decode_static_scratch(out, query, key_cache, value_cache, block_tables, context_lens,
                             max_context_len: int, scale: float, layout: int = NHD,
                             partition_size: int = -1, stream=None) -> None:
    """pa_decode without a workspace argument (for callers that cannot
    allocate): the split-K workspace is the library's static per-GPU array
    of PA_STATIC_SCRATCH_BYTES; calls overlapping on one GPU race."""
    torch = _torch()
    nb, bs, hkv, d = _geom(key_cache, layout)
    S, H, D = query.shape
    if D != d or out.shape != query.shape:
        raise ValueError("query/out must be [num_seqs, num_heads, head_size]")
    if query.dtype != key_cache.dtype:
        raise TypeError("query dtype must equal the cache dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables [S, max_blocks] and context_lens [S] required")
    _check("pa_decode_static_scratch", _lib.pa_decode_static_scratch(
        _dev(out, "out"), _dtype_code(out), _dev(query, "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dtype_code(key_cache), layout,
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), int(max_context_len), S, H, hkv, d, bs,
        nb, float(scale), int(partition_size), _stream(stream)))


def pa_decode_fp8(out, query, key_cache, value_cache, block_tables, context_lens,
                  max_context_len: int, scale: float, k_scale: float, v_scale: float,
                  layout: int = NHD, partition_size: int = -1, workspace=None,
                  stream=None) -> None:
    """Decode attention over E4M3 pools (uint8); query bf16/f16, out float32 or the query type."""
    _decode_fp8("pa_decode_fp8", out, query, key_cache, value_cache, block_tables, context_lens,
                max_context_len, scale, k_scale, v_scale, layout, partition_size, workspace,
                stream)


def pa_decode_partitions_fp8(out, query, key_cache, value_cache, block_tables, context_lens,
                             max_context_len: int, scale: float, k_scale: float, v_scale: float,
                             partition_size: int, workspace, layout: int = NHD,
                             stream=None) -> None:
    """Partition half of split-K decode over E4M3 pools (finish with pa_decode_reduce)."""
    _decode_fp8("pa_decode_partitions_fp8", out, query, key_cache, value_cache, block_tables,
                context_lens, max_context_len, scale, k_scale, v_scale, layout, partition_size,
                workspace, stream)


def _decode_fp8(fn, out, query, key_cache, value_cache, block_tables, context_lens,
                max_context_len, scale, k_scale, v_scale, layout, partition_size, workspace,
                stream) -> None:
    torch = _torch()
    nb, bs, hkv, d = _geom(key_cache, layout)
    S, H, D = query.shape
    if D != d or out.shape != query.shape:
        raise ValueError("query/out must be [num_seqs, num_heads, head_size]")
    if _dtype_code(key_cache) != PA_FP8_E4M3 or value_cache.dtype != key_cache.dtype:
        raise TypeError("FP8 pools are uint8 (or float8_e4m3fn)")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables [S, max_blocks] and context_lens [S] required")
    ws_ptr, ws_bytes = (None, 0)
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    _check(fn, getattr(_lib, fn)(
        _dev(out, "out"), _dtype_code(out), _dev(query, "query"), _dtype_code(query),
        _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"), float(k_scale),
        float(v_scale), layout, _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32),
        int(max_context_len), S, H, hkv, d, bs, nb, float(scale), int(partition_size), ws_ptr,
        ws_bytes, _stream(stream)))


def pa_decode_cascade_workspace_size(num_seqs: int, num_heads: int, head_size: int,
                                     max_context_len: int, common_prefix_len: int,
                                     partition_size: int = -1) -> int:
    return int(_lib.pa_decode_cascade_workspace_size(num_seqs, num_heads, head_size,
                                                     max_context_len, common_prefix_len,
                                                     partition_size))


def pa_decode_cascade(out, query, key_cache, value_cache, block_tables, context_lens,
                      max_context_len: int, common_prefix_len: int, scale: float, workspace,
                      layout: int = NHD, partition_size: int = -1, stream=None) -> None:
    """Decode with a shared prefix attended once (same result as pa_decode)."""
    torch = _torch()
    nb, bs, hkv, d = _geom(key_cache, layout)
    S, H, D = query.shape
    if D != d or out.shape != query.shape:
        raise ValueError("query/out must be [num_seqs, num_heads, head_size]")
    if query.dtype != key_cache.dtype:
        raise TypeError("query dtype must equal the cache dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables [S, max_blocks] and context_lens [S] required")
    _check("pa_decode_cascade", _lib.pa_decode_cascade(
        _dev(out, "out"), _dtype_code(out), _dev(query, "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dtype_code(key_cache), layout,
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), int(max_context_len),
        int(common_prefix_len), S, H, hkv, d, bs, nb, float(scale), int(partition_size),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)))



def pa_decode_cascade_fp8(out, query, key_cache, value_cache, block_tables, context_lens,
                          max_context_len: int, common_prefix_len: int, scale: float,
                          k_scale: float, v_scale: float, workspace, layout: int = NHD,
                          partition_size: int = -1, stream=None) -> None:
    """pa_decode_cascade over E4M3 pools (uint8); query bf16/f16."""
    torch = _torch()
    nb, bs, hkv, d = _geom(key_cache, layout)
    S, H, D = query.shape
    if D != d or out.shape != query.shape:
        raise ValueError("query/out must be [num_seqs, num_heads, head_size]")
    if _dtype_code(key_cache) != PA_FP8_E4M3 or value_cache.dtype != key_cache.dtype:
        raise TypeError("FP8 pools are uint8 (or float8_e4m3fn)")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables [S, max_blocks] and context_lens [S] required")
    _check("pa_decode_cascade_fp8", _lib.pa_decode_cascade_fp8(
        _dev(out, "out"), _dtype_code(out), _dev(query, "query"), _dtype_code(query),
        _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"), float(k_scale),
        float(v_scale), layout, _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32),
        int(max_context_len), int(common_prefix_len), S, H, hkv, d, bs, nb, float(scale),
        int(partition_size), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))

def pa_decode_partitions(out, query, key_cache, value_cache, block_tables, context_lens,
                         max_context_len: int, scale: float, partition_size: int, workspace,
                         layout: int = NHD, stream=None) -> None:
    """Split-K first half: per-partition (max, sum, unnormalised output) into
    workspace; rows of single-partition contexts go straight to out."""
    torch = _torch()
    nb, bs, hkv, d = _geom(key_cache, layout)
    S, H, D = query.shape
    if D != d or query.dtype != key_cache.dtype or out.shape != query.shape:
        raise ValueError("query/out must be [num_seqs, num_heads, head_size] of the cache dtype")
    _check("pa_decode_partitions", _lib.pa_decode_partitions(
        _dev(out, "out"), _dtype_code(out), _dev(query, "query"), _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
        _dtype_code(key_cache), layout, _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32),
        int(max_context_len), S, H, hkv, d, bs, nb, float(scale), int(partition_size),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def pa_decode_reduce(out, context_lens, max_context_len: int, num_kv_heads: int,
                     partition_size: int, workspace, stream=None) -> None:
    """Split-K second half: merge the partitions into out [S, H, D]."""
    torch = _torch()
    S, H, D = out.shape
    _check("pa_decode_reduce", _lib.pa_decode_reduce(
        _dev(out, "out"), _dtype_code(out), _dev(context_lens, "context_lens", torch.int32),
        int(max_context_len), S, H, int(num_kv_heads), D, int(partition_size),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def pa_prefill(out, query, key_cache, value_cache, block_tables, query_start_loc, context_lens,
               max_query_len: int, max_context_len: int, scale: float, layout: int = NHD,
               stream=None) -> None:
    """Causal packed prefill; query/out [num_tokens, H, D]."""
    torch = _torch()
    nb, bs, hkv, d = _geom(key_cache, layout)
    T, H, D = query.shape
    S = context_lens.shape[0]
    if D != d or out.shape != query.shape:
        raise ValueError("query/out must be [num_tokens, num_heads, head_size]")
    if query.dtype != key_cache.dtype:
        raise TypeError("query dtype must equal the cache dtype")
    if query_start_loc.shape != (S + 1,) or block_tables.shape[0] != S:
        raise ValueError("query_start_loc [S+1] and block_tables [S, max_blocks] required")
    _check("pa_prefill", _lib.pa_prefill(
        _dev(out, "out"), _dtype_code(out), _dev(query, "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dtype_code(key_cache), layout,
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(query_start_loc, "query_start_loc", torch.int32),
        _dev(context_lens, "context_lens", torch.int32), S, T, int(max_query_len),
        int(max_context_len), H, hkv, d, bs, nb, float(scale), _stream(stream)))


def pa_prefill_fp8(out, query, key_cache, value_cache, block_tables, query_start_loc,
                   context_lens, max_query_len: int, max_context_len: int, scale: float,
                   k_scale: float, v_scale: float, layout: int = NHD, stream=None) -> None:
    """Causal packed prefill over E4M3 pools (uint8); query bf16/f16 [T, H, D]."""
    torch = _torch()
    nb, bs, hkv, d = _geom(key_cache, layout)
    T, H, D = query.shape
    if D != d or out.shape != query.shape:
        raise ValueError("query/out must be [num_tokens, num_heads, head_size]")
    if _dtype_code(key_cache) != PA_FP8_E4M3 or value_cache.dtype != key_cache.dtype:
        raise TypeError("FP8 pools are uint8 (or float8_e4m3fn)")
    S = block_tables.shape[0]
    if query_start_loc.shape != (S + 1,) or context_lens.shape != (S,):
        raise ValueError("query_start_loc [S+1] and context_lens [S] required")
    _check("pa_prefill_fp8", _lib.pa_prefill_fp8(
        _dev(out, "out"), _dtype_code(out), _dev(query, "query"), _dtype_code(query),
        _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"), float(k_scale),
        float(v_scale), layout, _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(query_start_loc, "query_start_loc", torch.int32),
        _dev(context_lens, "context_lens", torch.int32), S, T, int(max_query_len),
        int(max_context_len), H, hkv, d, bs, nb, float(scale), _stream(stream)))


def pa_check_metadata(block_tables, context_lens, slot_mapping, num_blocks: int, block_size: int,
                      max_context_len: Optional[int] = None, common_prefix_len: int = 0,
                      num_seqs: Optional[int] = None, stream=None) -> None:
    """Synchronous host check of device metadata; raises PagedAttnError(PA_ERR_METADATA).

    Any of the three arrays may be None (its checks are skipped).
    max_context_len defaults to the table's capacity (max_blocks x
    block_size), or to 2^31 - 1 without a table.  num_seqs defaults to the
    rows of context_lens or block_tables."""
    if num_seqs is None:
        num_seqs = context_lens.shape[0] if context_lens is not None else (
            block_tables.shape[0] if block_tables is not None else 0)
    mb = block_tables.shape[1] if block_tables is not None else 0
    if max_context_len is None:
        max_context_len = mb * block_size if block_tables is not None else 0x7FFFFFFF
    T = slot_mapping.shape[0] if slot_mapping is not None else 0
    for t, name, dt in ((block_tables, "block_tables", "int32"), (context_lens, "context_lens", "int32"),
                        (slot_mapping, "slot_mapping", "int64")):
        if t is not None:
            _dev(t, name, getattr(_torch(), dt))
    p = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    _check("pa_check_metadata", _lib.pa_check_metadata(
        p(block_tables), p(context_lens), p(slot_mapping), num_seqs, mb, max_context_len, T,
        block_size, num_blocks, common_prefix_len, _stream(stream)))


def pa_stream_read_probe_sink_words() -> int:
    return int(_lib.pa_stream_read_probe_sink_words())


def pa_stream_read_probe(buf, sink, stream=None) -> None:
    """Measurement aid: read every byte of the device tensor `buf` once
    (16-byte non-temporal loads); `sink` is a device int32/uint32 tensor of
    pa_stream_read_probe_sink_words() elements that receives digests."""
    torch = _torch()
    _dev(buf, "buf")
    _dev(sink, "sink", torch.int32)
    if sink.numel() < pa_stream_read_probe_sink_words():
        raise ValueError("sink too small")
    nbytes = buf.numel() * buf.element_size()
    _check("pa_stream_read_probe", _lib.pa_stream_read_probe(buf.data_ptr(), nbytes,
                                                             sink.data_ptr(), _stream(stream)))


# ------------------------------------------------------------------ block pool
class BlockPool:
    """Host block manager (pa_pool_*): FIFO free queue, reference counts,
    fork and append with copy-on-write."""

    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence[int]] = None):
        self.block_size = int(block_size)
        self.num_blocks = int(num_blocks)
        h = _vp()
        if free_order is None:
            st = _lib.pa_pool_create(num_blocks, block_size, None, ctypes.byref(h))
        else:
            arr = np.ascontiguousarray(free_order, dtype=np.int32)
            st = _lib.pa_pool_create(num_blocks, block_size, arr.ctypes.data_as(_pi32),
                                     ctypes.byref(h))
        _check("pa_pool_create", st)
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:  # the module may be torn down first at exit
            _lib.pa_pool_destroy(h)
            self._h = None

    def add_seq(self) -> int:
        sid = ctypes.c_int32()
        _check("pa_pool_add_seq", _lib.pa_pool_add_seq(self._h, ctypes.byref(sid)))
        return sid.value

    def add_seq_cached(self, tokens, extra: int = 0) -> Tuple[int, int]:
        """New sequence for a prompt, reusing cached full blocks from the
        left; returns (sequence id, tokens covered by reused blocks)."""
        arr = np.ascontiguousarray(tokens, dtype=np.int32)
        sid, hit = ctypes.c_int32(), ctypes.c_int32()
        st = _lib.pa_pool_add_seq_cached(self._h, arr.ctypes.data_as(_pi32), arr.size,
                                         ctypes.c_uint64(int(extra)), ctypes.byref(sid),
                                         ctypes.byref(hit))
        _check("pa_pool_add_seq_cached", st)
        return sid.value, hit.value

    def num_cached(self) -> int:
        return int(_lib.pa_pool_num_cached(self._h))

    def fork(self, parent: int) -> int:
        c = ctypes.c_int32()
        _check("pa_pool_fork", _lib.pa_pool_fork(self._h, parent, ctypes.byref(c)))
        return c.value

    def append(self, seq: int, n: int) -> Tuple[np.ndarray, List[Tuple[int, int]]]:
        """Append n tokens; returns (slots int64 [n], copy-on-write pairs)."""
        slots = np.empty(n, np.int64)
        pairs = np.empty(2, np.int32)
        ncow = ctypes.c_int32()
        _check("pa_pool_append", _lib.pa_pool_append(
            self._h, seq, n, slots.ctypes.data_as(_pi64), pairs.ctypes.data_as(_pi32), 1,
            ctypes.byref(ncow)))
        return slots, [(int(pairs[0]), int(pairs[1]))] if ncow.value else []

    def free_seq(self, seq: int) -> None:
        _check("pa_pool_free_seq", _lib.pa_pool_free_seq(self._h, seq))

    def block_table(self, seq: int) -> np.ndarray:
        n = ctypes.c_int32()
        _check("pa_pool_block_table", _lib.pa_pool_block_table(self._h, seq, None, 0,
                                                               ctypes.byref(n)))
        out = np.empty(n.value, np.int32)
        _check("pa_pool_block_table", _lib.pa_pool_block_table(
            self._h, seq, out.ctypes.data_as(_pi32), n.value, ctypes.byref(n)))
        return out

    def seq_len(self, seq: int) -> int:
        return int(_lib.pa_pool_seq_len(self._h, seq))

    def num_free(self) -> int:
        return int(_lib.pa_pool_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(_lib.pa_pool_refcount(self._h, block))
