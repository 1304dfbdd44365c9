"""ctypes binding of libpa.so.

Argument marshalling only: each function checks the tensors it is handed
(device, dtype, contiguity, shape), passes raw device pointers and the current
HIP stream to the C entry point of the same name, and raises ``PAError`` on a
non-zero status.  All paged-attention work runs in the library's HIP kernels;
there is no fallback path.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

import numpy as np

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")
# The same entry points built with PA_CHECK_INDICES: kernels record out-of-range
# indices on the device (pa_take_index_errors) instead of skipping them silently.
CHECK_LIB_PATH = os.path.join(_HERE, "libpa_check.so")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP = 0, -1, -2, -3, -4
PA_ERR_NO_BLOCKS, PA_ERR_BAD_INDEX = -5, -6
PA_INDEX_ERR_BLOCK_ID, PA_INDEX_ERR_SLOT, PA_INDEX_ERR_CONTEXT_LEN, PA_INDEX_ERR_QUERY_LOC = 1, 2, 4, 8
PA_F16, PA_BF16 = 0, 1

_libs = {}
_checked = False      # calls go to libpa_check.so inside checked_indices()
_lock = threading.Lock()


class PAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def _declare(lib):
    c_int, c_i64, c_sz, c_vp, c_f = (ctypes.c_int, ctypes.c_int64, ctypes.c_size_t,
                                       ctypes.c_void_p, ctypes.c_float)
    lib.pa_version.restype = c_int
    lib.pa_version.argtypes = []
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_status_string.argtypes = [c_int]
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_last_error.argtypes = []
    lib.pa_check_indices_enabled.restype = c_int
    lib.pa_check_indices_enabled.argtypes = []
    lib.pa_take_index_errors.restype = c_int
    lib.pa_take_index_errors.argtypes = [c_vp, c_vp, c_vp, c_vp]
    lib.pa_set_kernel_events.restype = c_int
    lib.pa_set_kernel_events.argtypes = [c_vp, c_vp]
    lib.pa_cache_flush.restype = c_int
    lib.pa_cache_flush.argtypes = [c_vp, c_sz, c_vp]
    lib.pa_stream_read.restype = c_int
    lib.pa_stream_read.argtypes = [c_vp, c_sz, c_vp]
    lib.pa_reshape_and_cache.restype = c_int
    lib.pa_reshape_and_cache.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_int, c_int, c_int,
                                         c_i64, c_int, c_vp]
    lib.pa_decode_partition_hint.restype = c_int
    lib.pa_decode_partition_hint.argtypes = [c_int, c_int, c_int, c_int]
    lib.pa_decode_workspace_size.restype = c_sz
    lib.pa_decode_workspace_size.argtypes = [c_int, c_int, c_int, c_int, c_int]
    lib.pa_decode.restype = c_int
    lib.pa_decode.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int,
                              c_int, c_i64, c_int, c_int, c_f, c_int, c_vp, c_sz, c_int, c_vp]
    lib.pa_decode_partitions.restype = c_int
    lib.pa_decode_partitions.argtypes = lib.pa_decode.argtypes
    lib.pa_decode_merge.restype = c_int
    lib.pa_decode_merge.argtypes = [c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int, c_int, c_vp, c_sz,
                                    c_int, c_vp]
    lib.pa_decode_step.restype = c_int
    lib.pa_decode_step.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                   c_int, c_int, c_int, c_int, c_int, c_i64, c_int, c_int, c_f,
                                   c_int, c_vp, c_sz, c_int, c_vp]
    lib.pa_decode_step_scratch.restype = c_int
    lib.pa_decode_step_scratch.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                           c_vp, c_int, c_int, c_int, c_int, c_int, c_i64, c_int,
                                           c_int, c_f, c_int, c_int, c_vp]
    lib.pa_decode_order.restype = c_int
    lib.pa_decode_order.argtypes = [c_vp, c_int, c_vp]
    lib.pa_prefill_chunk.restype = c_int
    lib.pa_prefill_chunk.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_i64,
                                     c_int, c_int, c_int, c_int, c_i64, c_int, c_int, c_f, c_int,
                                     c_vp]
    c_pp = ctypes.POINTER(c_vp)
    lib.pa_bm_create.restype = c_int
    lib.pa_bm_create.argtypes = [c_i64, c_int, c_pp]
    lib.pa_bm_destroy.restype = None
    lib.pa_bm_destroy.argtypes = [c_vp]
    lib.pa_bm_add.restype = c_int
    lib.pa_bm_add.argtypes = [c_vp, c_i64, c_i64, c_vp]
    lib.pa_bm_fork.restype = c_int
    lib.pa_bm_fork.argtypes = [c_vp, c_i64, c_i64, c_i64]
    lib.pa_bm_append.restype = c_int
    lib.pa_bm_append.argtypes = [c_vp, c_i64, c_i64, c_vp]
    lib.pa_bm_free.restype = c_int
    lib.pa_bm_free.argtypes = [c_vp, c_i64]
    lib.pa_bm_tables.restype = c_int
    lib.pa_bm_tables.argtypes = [c_vp, c_vp, c_int, c_int, c_vp, c_vp]
    lib.pa_bm_take_copies.restype = c_i64
    lib.pa_bm_take_copies.argtypes = [c_vp, c_vp, c_vp, c_i64]
    for name in ("pa_bm_num_free", "pa_bm_num_seqs"):
        getattr(lib, name).restype = c_i64
        getattr(lib, name).argtypes = [c_vp]
    lib.pa_bm_num_tokens.restype = c_i64
    lib.pa_bm_num_tokens.argtypes = [c_vp, c_i64]
    lib.pa_bm_ref_count.restype = c_int
    lib.pa_bm_ref_count.argtypes = [c_vp, c_i64]
    lib.pa_reshape_and_cache_int8.restype = c_int
    lib.pa_reshape_and_cache_int8.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_int,
                                              c_int, c_int, c_i64, c_int, c_vp]
    lib.pa_decode_int8.restype = c_int
    lib.pa_decode_int8.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int,
                                   c_int, c_int, c_int, c_i64, c_int, c_int, c_f, c_int, c_vp, c_sz,
                                   c_int, c_vp]
    lib.pa_decode_step_int8.restype = c_int
    lib.pa_decode_step_int8.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                        c_vp, c_vp, c_int, c_int, c_int, c_int, c_int, c_i64, c_int,
                                        c_int, c_f, c_int, c_vp, c_sz, c_int, c_vp]
    lib.pa_rope_reshape_and_cache.restype = c_int
    lib.pa_rope_reshape_and_cache.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                              c_i64, c_int, c_int, c_int, c_int, c_i64, c_i64,
                                              c_int, c_vp]
    lib.pa_decode_step_rope.restype = c_int
    lib.pa_decode_step_rope.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_vp,
                                        c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int, c_int,
                                        c_i64, c_int, c_int, c_f, c_int, c_vp, c_sz, c_int, c_vp]
    lib.pa_decode_partial.restype = c_int
    lib.pa_decode_partial.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int,
                                      c_int, c_int, c_int, c_i64, c_int, c_int, c_f, c_int, c_vp,
                                      c_sz, c_int, c_vp]
    lib.pa_merge_partials.restype = c_int
    lib.pa_merge_partials.argtypes = [c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int, c_int,
                                      c_vp]
    lib.pa_copy_blocks.restype = c_int
    lib.pa_copy_blocks.argtypes = [c_vp, c_vp, c_vp, c_vp, c_i64, c_int, c_int, c_int, c_i64, c_int,
                                   c_vp]
    return lib


def load_library(build_if_missing: bool = True, checked: bool | None = None):
    """Load libpa.so, or libpa_check.so inside checked_indices() or with checked=True
    (building both first only if the library is not built)."""
    path = CHECK_LIB_PATH if (_checked if checked is None else checked) else LIB_PATH
    with _lock:
        lib = _libs.get(path)
        if lib is not None:
            return lib
        if not os.path.exists(path):
            if not build_if_missing:
                raise ImportError(f"{path} is not built")
            from .build import build_library
            build_library()
        lib = _libs[path] = _declare(ctypes.CDLL(path))
        return lib


@contextlib.contextmanager
def checked_indices():
    """Within the block, every call of this module goes to libpa_check.so, whose kernels
    record out-of-range block ids, slots and lengths (read them with pa_take_index_errors).
    Not thread-safe: it switches the whole module."""
    global _checked
    prev = _checked
    _checked = True
    try:
        yield load_library()
    finally:
        _checked = prev


def pa_take_index_errors(stream=None):
    """Wait for the stream and return ``(status, kinds, first_kind, first_value)`` of the index
    errors the checking library's kernels recorded on its device since the last call
    (status PA_OK or PA_ERR_BAD_INDEX), clearing them.  Uses libpa_check.so."""
    lib = load_library(checked=True)
    if stream is None:
        stream = torch.cuda.current_stream()
    s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    kinds, first_kind, first_value = ctypes.c_uint32(), ctypes.c_uint32(), ctypes.c_int64()
    st = lib.pa_take_index_errors(s, ctypes.byref(kinds), ctypes.byref(first_kind),
                                  ctypes.byref(first_value))
    if st not in (PA_OK, PA_ERR_BAD_INDEX):
        raise PAError(st, f"{lib.pa_status_string(st).decode()}: {lib.pa_last_error().decode()}")
    return st, kinds.value, first_kind.value, first_value.value


def _event_handle(ev) -> int | None:
    if ev is None:
        return None
    if isinstance(ev, int):
        return ev
    handle = ev.cuda_event
    if not handle:
        raise ValueError("a torch.cuda.Event has no HIP event until it is first recorded")
    return handle


def pa_set_kernel_events(start=None, stop=None) -> None:
    """Arm timing events on this thread (no arguments: disarm).  While armed, every kernel the
    library launches records ``stop`` as it ends; ``start``, if given, is recorded by the first
    one as it begins.  Takes torch.cuda.Event objects (enable_timing=True, recorded once so that
    their HIP event exists) or raw hipEvent_t handles."""
    _check(load_library().pa_set_kernel_events(_event_handle(start), _event_handle(stop)))


def pa_cache_flush(buf: torch.Tensor, stream=None) -> None:
    """Read all of the device tensor ``buf`` and write nothing (evicts the caches' contents
    when ``buf`` is larger than them)."""
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    _check(load_library().pa_cache_flush(buf.data_ptr(), buf.numel() * buf.element_size(),
                                         _stream(buf, stream)))


def pa_stream_read(buf: torch.Tensor, stream=None) -> None:
    """Read all of the device tensor ``buf`` with non-temporal loads and write nothing (a
    streaming-read rate reference; the caches' contents are left alone)."""
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    _check(load_library().pa_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                         _stream(buf, stream)))


def _check(status: int) -> None:
    if status != PA_OK:
        lib = load_library()
        detail = lib.pa_last_error().decode()
        raise PAError(status, f"{lib.pa_status_string(status).decode()}: {detail}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return PA_F16
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise TypeError(f"expected float16 or bfloat16, got {t.dtype}")


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(t: torch.Tensor, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def pa_version() -> int:
    return load_library().pa_version()


def pa_decode_workspace_size(num_seqs: int, num_heads: int, head_dim: int, max_context_len: int,
                             partition_size: int) -> int:
    return int(load_library().pa_decode_workspace_size(num_seqs, num_heads, head_dim,
                                                       max_context_len, partition_size))


def pa_decode_partition_hint(num_seqs: int, num_kv_heads: int, max_context_len: int,
                             block_size: int) -> int:
    """A partition_size suited to the current device (0 = no split)."""
    lib = load_library()
    r = int(lib.pa_decode_partition_hint(num_seqs, num_kv_heads, max_context_len, block_size))
    if r < 0:
        raise PAError(r, lib.pa_last_error().decode())
    return r


def decode_workspace(num_seqs: int, num_heads: int, head_dim: int, max_context_len: int,
                     partition_size: int, device) -> torch.Tensor:
    """A workspace of the size pa_decode needs (one byte if none)."""
    n = pa_decode_workspace_size(num_seqs, num_heads, head_dim, max_context_len, partition_size)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def pa_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """Write key/value ``[T][Hkv][D]`` into caches ``[NB][BS][Hkv][D]`` at ``slot_mapping`` (int64)."""
    lib = load_library()
    T, Hkv, D = key.shape
    NB, BS, Hkv2, D2 = k_cache.shape
    if value.shape != key.shape or v_cache.shape != k_cache.shape or (Hkv2, D2) != (Hkv, D):
        raise ValueError("reshape_and_cache: inconsistent shapes")
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [num_tokens]")
    dt = _dtype_code(key)
    for n, x in (("value", value), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(x, n, key.dtype)
    _check(lib.pa_reshape_and_cache(_dev(key, "key"), value.data_ptr(), k_cache.data_ptr(),
                                    v_cache.data_ptr(), _dev(slot_mapping, "slot_mapping", torch.int64),
                                    T, Hkv, D, BS, NB, dt, _stream(key, stream)))


def pa_rope_reshape_and_cache(q, key, value, k_cache, v_cache, positions, cos, sin, slot_mapping,
                              stream=None) -> None:
    """Rotate keys (and ``q`` in place, if given) by the rotary tables at ``positions`` and
    write keys and values into caches ``[NB][BS][Hkv][D]`` at ``slot_mapping``."""
    lib = load_library()
    T, Hkv, D = key.shape
    NB, BS, Hkv2, D2 = k_cache.shape
    if value.shape != key.shape or v_cache.shape != k_cache.shape or (Hkv2, D2) != (Hkv, D):
        raise ValueError("rope_reshape_and_cache: inconsistent shapes")
    if positions.shape != (T,) or slot_mapping.shape != (T,):
        raise ValueError("positions and slot_mapping must be [num_tokens]")
    if cos.dim() != 2 or cos.shape[1] != D // 2 or sin.shape != cos.shape:
        raise ValueError("cos/sin must be [max_position][head_dim / 2]")
    Hq = 0
    if q is not None:
        if q.dim() != 3 or q.shape[0] != T or q.shape[2] != D:
            raise ValueError("q must be [num_tokens][num_heads][head_dim]")
        Hq = q.shape[1]
        _dev(q, "q", key.dtype)
    dt = _dtype_code(key)
    for n, x in (("value", value), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(x, n, key.dtype)
    _check(lib.pa_rope_reshape_and_cache(
        None if q is None else q.data_ptr(), _dev(key, "key"), value.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), _dev(positions, "positions", torch.int64),
        _dev(cos, "cos", torch.float32), _dev(sin, "sin", torch.float32),
        _dev(slot_mapping, "slot_mapping", torch.int64), T, Hq, Hkv, D, BS, NB, cos.shape[0], dt,
        _stream(key, stream)))


def _decode_common(q, k_cache, v_cache, block_tables, context_lens, seq_order, out,
                   max_context_len, partition_size, workspace, cache_dtype=None, head_major=False):
    lib = load_library()
    B, Hq, D = q.shape
    if head_major:
        NB, Hkv, BS, D2 = k_cache.shape
    else:
        NB, BS, Hkv, D2 = k_cache.shape
    if out.shape != q.shape or v_cache.shape != k_cache.shape or D2 != D:
        raise ValueError("decode: inconsistent shapes")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("decode: block_tables must be [B][max_blocks], context_lens [B]")
    if seq_order is not None and seq_order.shape != (B,):
        raise ValueError("decode: seq_order must be [B]")
    dt = _dtype_code(q)
    _dev(out, "out", q.dtype)
    for n, x in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(x, n, q.dtype if cache_dtype is None else cache_dtype)
    need = lib.pa_decode_workspace_size(B, Hq, D, max_context_len, partition_size)
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    order_ptr = None if seq_order is None else _dev(seq_order, "seq_order", torch.int32)
    return (lib, B, Hq, Hkv, D, BS, NB, dt, ws_ptr, ws_bytes, order_ptr)


def pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale: float,
              max_context_len: int, partition_size: int = 512, workspace=None, seq_order=None,
              stream=None) -> torch.Tensor:
    """Paged decode: ``out[i][h] = softmax(scale q K^T) V`` over each sequence's paged context."""
    lib, B, Hq, Hkv, D, BS, NB, dt, ws_ptr, ws_bytes, order_ptr = _decode_common(
        q, k_cache, v_cache, block_tables, context_lens, seq_order, out, max_context_len,
        partition_size, workspace)
    _check(lib.pa_decode(_dev(out, "out"), _dev(q, "q"), k_cache.data_ptr(), v_cache.data_ptr(),
                         _dev(block_tables, "block_tables", torch.int32),
                         _dev(context_lens, "context_lens", torch.int32), order_ptr,
                         B, Hq, Hkv, D, BS, NB, block_tables.shape[1], int(max_context_len),
                         float(scale), int(partition_size), ws_ptr, ws_bytes, dt,
                         _stream(q, stream)))
    return out


def pa_decode_partitions(out, q, k_cache, v_cache, block_tables, context_lens, scale: float,
                         max_context_len: int, partition_size: int = 512, workspace=None,
                         seq_order=None, stream=None) -> torch.Tensor:
    """The partition phase of pa_decode alone: rows of contexts that span several
    partitions stay in ``workspace`` (which must then be given) until pa_decode_merge."""
    lib, B, Hq, Hkv, D, BS, NB, dt, ws_ptr, ws_bytes, order_ptr = _decode_common(
        q, k_cache, v_cache, block_tables, context_lens, seq_order, out, max_context_len,
        partition_size, workspace)
    if ws_ptr is not None and workspace is None:
        raise ValueError("decode partitions: pass the workspace the merge will read")
    _check(lib.pa_decode_partitions(_dev(out, "out"), _dev(q, "q"), k_cache.data_ptr(),
                                    v_cache.data_ptr(),
                                    _dev(block_tables, "block_tables", torch.int32),
                                    _dev(context_lens, "context_lens", torch.int32), order_ptr,
                                    B, Hq, Hkv, D, BS, NB, block_tables.shape[1],
                                    int(max_context_len), float(scale), int(partition_size),
                                    ws_ptr, ws_bytes, dt, _stream(q, stream)))
    return out


def pa_decode_merge(out, context_lens, max_context_len: int, partition_size: int, workspace,
                    seq_order=None, stream=None) -> torch.Tensor:
    """The merge phase of a split decode alone, over the partials a preceding split decode
    left in ``workspace``; ``out`` is ``[num_seqs][num_heads][head_dim]``."""
    lib = load_library()
    B, Hq, D = out.shape
    if context_lens.shape != (B,) or (seq_order is not None and seq_order.shape != (B,)):
        raise ValueError("decode merge: context_lens and seq_order must be [num_seqs]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    order_ptr = None if seq_order is None else _dev(seq_order, "seq_order", torch.int32)
    _check(lib.pa_decode_merge(_dev(out, "out"), _dev(context_lens, "context_lens", torch.int32),
                               order_ptr, B, Hq, D, int(max_context_len), int(partition_size),
                               ws_ptr, ws_bytes, _dtype_code(out), _stream(out, stream)))
    return out


def pa_decode_step(out, q, key, value, slot_mapping, k_cache, v_cache, block_tables,
                   context_lens, scale: float, max_context_len: int, partition_size: int = 512,
                   workspace=None, seq_order=None, stream=None) -> torch.Tensor:
    """One decode step: store each sequence's new K/V token at its slot and attend, in one launch."""
    lib, B, Hq, Hkv, D, BS, NB, dt, ws_ptr, ws_bytes, order_ptr = _decode_common(
        q, k_cache, v_cache, block_tables, context_lens, seq_order, out, max_context_len,
        partition_size, workspace)
    if key.shape != (B, Hkv, D) or value.shape != key.shape or slot_mapping.shape != (B,):
        raise ValueError("decode step: key/value must be [B][Hkv][D], slot_mapping [B]")
    _dev(key, "key", q.dtype)
    _dev(value, "value", q.dtype)
    _check(lib.pa_decode_step(_dev(out, "out"), _dev(q, "q"), key.data_ptr(), value.data_ptr(),
                              _dev(slot_mapping, "slot_mapping", torch.int64),
                              k_cache.data_ptr(), v_cache.data_ptr(),
                              _dev(block_tables, "block_tables", torch.int32),
                              _dev(context_lens, "context_lens", torch.int32), order_ptr,
                              B, Hq, Hkv, D, BS, NB, block_tables.shape[1], int(max_context_len),
                              float(scale), int(partition_size), ws_ptr, ws_bytes, dt,
                              _stream(q, stream)))
    return out


def pa_decode_step_scratch(out, q, key, value, slot_mapping, k_cache, v_cache, block_tables,
                           context_lens, scale: float, max_context_len: int,
                           partition_size: int = 512, seq_order=None, stream=None) -> torch.Tensor:
    """pa_decode_step without a workspace: split-K partials go to the library's static
    scratch on the device (nothing is allocated by the call)."""
    lib, B, Hq, Hkv, D, BS, NB, dt, _, _, order_ptr = _decode_common(
        q, k_cache, v_cache, block_tables, context_lens, seq_order, out, max_context_len, 0, None)
    if key.shape != (B, Hkv, D) or value.shape != key.shape or slot_mapping.shape != (B,):
        raise ValueError("decode step: key/value must be [B][Hkv][D], slot_mapping [B]")
    _dev(key, "key", q.dtype)
    _dev(value, "value", q.dtype)
    _check(lib.pa_decode_step_scratch(_dev(out, "out"), _dev(q, "q"), key.data_ptr(),
                                      value.data_ptr(),
                                      _dev(slot_mapping, "slot_mapping", torch.int64),
                                      k_cache.data_ptr(), v_cache.data_ptr(),
                                      _dev(block_tables, "block_tables", torch.int32),
                                      _dev(context_lens, "context_lens", torch.int32), order_ptr,
                                      B, Hq, Hkv, D, BS, NB, block_tables.shape[1],
                                      int(max_context_len), float(scale), int(partition_size), dt,
                                      _stream(q, stream)))
    return out


def pa_decode_partial(out, out_ml, q, k_cache, v_cache, block_tables, context_lens, scale: float,
                      max_context_len: int, partition_size: int = 0, workspace=None, seq_order=None,
                      stream=None):
    """Shard-local decode writing the partial row: normalised ``out [B][Hq][D]`` and float32
    ``out_ml [B][Hq][2]`` = (log2-domain max, sum) over the shard's keys."""
    lib, B, Hq, Hkv, D, BS, NB, dt, ws_ptr, ws_bytes, order_ptr = _decode_common(
        q, k_cache, v_cache, block_tables, context_lens, seq_order, out, max_context_len,
        partition_size, workspace)
    if out_ml.shape != (B, Hq, 2):
        raise ValueError("decode partial: out_ml must be [B][Hq][2]")
    _check(lib.pa_decode_partial(_dev(out, "out"), _dev(out_ml, "out_ml", torch.float32),
                                 _dev(q, "q"), k_cache.data_ptr(), v_cache.data_ptr(),
                                 _dev(block_tables, "block_tables", torch.int32),
                                 _dev(context_lens, "context_lens", torch.int32), order_ptr,
                                 B, Hq, Hkv, D, BS, NB, block_tables.shape[1], int(max_context_len),
                                 float(scale), int(partition_size), ws_ptr, ws_bytes, dt,
                                 _stream(q, stream)))
    return out, out_ml


def pa_merge_partials(out, partial_o, partial_ml, out_ml=None, stream=None) -> torch.Tensor:
    """Merge shard partials ``partial_o [N][B][Hq][D]``, ``partial_ml [N][B][Hq][2]`` into
    ``out [B][Hq][D]`` (and, when given, the merged (max, sum) into ``out_ml [B][Hq][2]``)."""
    lib = load_library()
    N, B, Hq, D = partial_o.shape
    if out.shape != (B, Hq, D) or partial_ml.shape != (N, B, Hq, 2):
        raise ValueError("merge partials: inconsistent shapes")
    if out_ml is not None and out_ml.shape != (B, Hq, 2):
        raise ValueError("merge partials: out_ml must be [B][Hq][2]")
    dt = _dtype_code(out)
    ml_ptr = None if out_ml is None else _dev(out_ml, "out_ml", torch.float32)
    _check(lib.pa_merge_partials(_dev(out, "out"), ml_ptr, _dev(partial_o, "partial_o", out.dtype),
                                 _dev(partial_ml, "partial_ml", torch.float32), N, B, Hq, D, dt,
                                 _stream(out, stream)))
    return out


def pa_decode_step_rope(out, q, key, value, slot_mapping, positions, cos, sin, k_cache, v_cache,
                        block_tables, context_lens, scale: float, max_context_len: int,
                        partition_size: int = 512, workspace=None, seq_order=None,
                        stream=None) -> torch.Tensor:
    """pa_decode_step with the rotary embedding of q and of the new key (rows ``positions`` of
    the float32 tables ``cos``/``sin`` [max_position][D/2]) folded into the same launch."""
    lib, B, Hq, Hkv, D, BS, NB, dt, ws_ptr, ws_bytes, order_ptr = _decode_common(
        q, k_cache, v_cache, block_tables, context_lens, seq_order, out, max_context_len,
        partition_size, workspace)
    if key.shape != (B, Hkv, D) or value.shape != key.shape or slot_mapping.shape != (B,):
        raise ValueError("decode step: key/value must be [B][Hkv][D], slot_mapping [B]")
    if positions.shape != (B,) or cos.dim() != 2 or cos.shape[1] != D // 2 or sin.shape != cos.shape:
        raise ValueError("positions must be [B], cos/sin [max_position][D/2]")
    _dev(key, "key", q.dtype)
    _dev(value, "value", q.dtype)
    _check(lib.pa_decode_step_rope(
        _dev(out, "out"), _dev(q, "q"), key.data_ptr(), value.data_ptr(),
        _dev(slot_mapping, "slot_mapping", torch.int64), _dev(positions, "positions", torch.int64),
        _dev(cos, "cos", torch.float32), _dev(sin, "sin", torch.float32), cos.shape[0],
        k_cache.data_ptr(), v_cache.data_ptr(), _dev(block_tables, "block_tables", torch.int32),
        _dev(context_lens, "context_lens", torch.int32), order_ptr, B, Hq, Hkv, D, BS, NB,
        block_tables.shape[1], int(max_context_len), float(scale), int(partition_size), ws_ptr,
        ws_bytes, dt, _stream(q, stream)))
    return out


def pa_decode_step_int8(out, q, key, value, slot_mapping, k_codes, v_codes, k_scales, v_scales,
                        block_tables, context_lens, scale: float, max_context_len: int,
                        partition_size: int = 512, workspace=None, seq_order=None,
                        stream=None) -> torch.Tensor:
    """One decode step over an INT8 cache: quantise each sequence's new K/V token into its
    slot and attend, in one launch (see :func:`pa_reshape_and_cache_int8`)."""
    lib, B, Hq, Hkv, D, BS, NB, dt, ws_ptr, ws_bytes, order_ptr = _decode_common(
        q, k_codes, v_codes, block_tables, context_lens, seq_order, out, max_context_len,
        partition_size, workspace, cache_dtype=torch.int8, head_major=True)
    if key.shape != (B, Hkv, D) or value.shape != key.shape or slot_mapping.shape != (B,):
        raise ValueError("decode_step_int8: key/value must be [B][Hkv][D], slot_mapping [B]")
    if k_scales.shape != (NB, Hkv, BS) or v_scales.shape != k_scales.shape:
        raise ValueError("decode_step_int8: scales must be [num_blocks][num_kv_heads][block_size]")
    _dev(key, "key", q.dtype)
    _dev(value, "value", q.dtype)
    ks = _dev(k_scales, "k_scales", torch.float32)
    vs = _dev(v_scales, "v_scales", torch.float32)
    _check(lib.pa_decode_step_int8(
        out.data_ptr(), q.data_ptr(), key.data_ptr(), value.data_ptr(),
        _dev(slot_mapping, "slot_mapping", torch.int64), k_codes.data_ptr(), v_codes.data_ptr(),
        ks, vs, _dev(block_tables, "block_tables", torch.int32),
        _dev(context_lens, "context_lens", torch.int32), order_ptr, B, Hq, Hkv, D, BS, NB,
        block_tables.shape[1], int(max_context_len), float(scale), int(partition_size), ws_ptr,
        ws_bytes, dt, _stream(q, stream)))
    return out


def pa_decode_order(context_lens) -> "numpy.ndarray":
    """Longest-first visiting order of the sequences (host computation) as int32."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    order = np.empty(lens.shape[0], dtype=np.int32)
    _check(load_library().pa_decode_order(lens.ctypes.data, lens.shape[0], order.ctypes.data))
    return order


def pa_prefill_chunk(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                     max_query_len: int, scale: float, seq_order=None, stream=None) -> torch.Tensor:
    """Chunked prefill: query rows of each sequence attend causally over its paged context."""
    lib = load_library()
    T, Hq, D = q.shape
    NB, BS, Hkv, D2 = k_cache.shape
    B = context_lens.shape[0]
    if out.shape != q.shape or v_cache.shape != k_cache.shape or D2 != D:
        raise ValueError("prefill: inconsistent shapes")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or query_start_loc.shape != (B + 1,):
        raise ValueError("prefill: block_tables must be [B][max_blocks], query_start_loc [B+1]")
    if seq_order is not None and seq_order.shape != (B,):
        raise ValueError("prefill: seq_order must be [B]")
    dt = _dtype_code(q)
    for n, x in (("out", out), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(x, n, q.dtype)
    order_ptr = None if seq_order is None else _dev(seq_order, "seq_order", torch.int32)
    _check(lib.pa_prefill_chunk(_dev(out, "out"), _dev(q, "q"), k_cache.data_ptr(), v_cache.data_ptr(),
                                _dev(block_tables, "block_tables", torch.int32),
                                _dev(context_lens, "context_lens", torch.int32),
                                _dev(query_start_loc, "query_start_loc", torch.int32), order_ptr,
                                B, T, Hq, Hkv, D, BS, NB, block_tables.shape[1], int(max_query_len),
                                float(scale), dt, _stream(q, stream)))
    return out


class BlockManager:
    """Host block manager of the library (``pa_bm_*``): physical blocks with
    reference counts, per-sequence block tables, prefix sharing by ``fork`` and
    copy on write.  Slot mappings, tables and copy pairs are host numpy arrays;
    upload them for the device calls."""

    def __init__(self, num_blocks: int, block_size: int):
        self._lib = load_library()
        h = ctypes.c_void_p()
        _check(self._lib.pa_bm_create(num_blocks, block_size, ctypes.byref(h)))
        self._h = h
        self.num_blocks, self.block_size = num_blocks, block_size

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def add(self, seq: int, num_tokens: int) -> np.ndarray:
        slots = np.empty(max(num_tokens, 0), dtype=np.int64)
        _check(self._lib.pa_bm_add(self._h, seq, num_tokens,
                                   slots.ctypes.data if num_tokens > 0 else None))
        return slots

    def fork(self, parent: int, child: int, num_tokens: int) -> None:
        _check(self._lib.pa_bm_fork(self._h, parent, child, num_tokens))

    def append(self, seq: int, n: int = 1) -> np.ndarray:
        slots = np.empty(max(n, 0), dtype=np.int64)
        _check(self._lib.pa_bm_append(self._h, seq, n, slots.ctypes.data if n > 0 else None))
        return slots

    def free(self, seq: int) -> None:
        _check(self._lib.pa_bm_free(self._h, seq))

    def tables(self, seqs, max_blocks_per_seq: int):
        """``(block_tables int32 [B][max_blocks], context_lens int32 [B])``."""
        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        bt = np.empty((ids.shape[0], max_blocks_per_seq), dtype=np.int32)
        lens = np.empty(ids.shape[0], dtype=np.int32)
        _check(self._lib.pa_bm_tables(self._h, ids.ctypes.data, ids.shape[0], max_blocks_per_seq,
                                      bt.ctypes.data, lens.ctypes.data))
        return bt, lens

    def take_copies(self, capacity: int = 1 << 16):
        """Queued copy-on-write pairs ``(src, dst)`` as int64 arrays (and clears them)."""
        src = np.empty(capacity, dtype=np.int64)
        dst = np.empty(capacity, dtype=np.int64)
        n = int(self._lib.pa_bm_take_copies(self._h, src.ctypes.data, dst.ctypes.data, capacity))
        if n < 0:
            _check(n)
        return src[:n].copy(), dst[:n].copy()

    @property
    def num_free(self) -> int:
        return int(self._lib.pa_bm_num_free(self._h))

    @property
    def num_seqs(self) -> int:
        return int(self._lib.pa_bm_num_seqs(self._h))

    def num_tokens(self, seq: int) -> int:
        return int(self._lib.pa_bm_num_tokens(self._h, seq))

    def ref_count(self, block: int) -> int:
        return int(self._lib.pa_bm_ref_count(self._h, block))


def pa_copy_blocks(k_cache, v_cache, src, dst, stream=None) -> None:
    """Copy whole blocks ``src[i] -> dst[i]`` (int64 device tensors) in both caches
    ``[NB][BS][Hkv][D]``: the copy-on-write step of :class:`BlockManager`."""
    lib = load_library()
    NB, BS, Hkv, D = k_cache.shape
    if v_cache.shape != k_cache.shape or src.shape != dst.shape or src.dim() != 1:
        raise ValueError("copy_blocks: inconsistent shapes")
    dt = _dtype_code(k_cache)
    _dev(k_cache, "k_cache"); _dev(v_cache, "v_cache", k_cache.dtype)
    n = src.shape[0]
    sp = _dev(src, "src", torch.int64) if n else None
    dp = _dev(dst, "dst", torch.int64) if n else None
    _check(lib.pa_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), sp, dp, n, Hkv, D, BS, NB, dt,
                              _stream(k_cache, stream)))


def pa_reshape_and_cache_int8(key, value, k_codes, v_codes, k_scales, v_scales, slot_mapping,
                              stream=None) -> None:
    """Quantise key/value ``[T][Hkv][D]`` (16-bit) into an INT8 cache at ``slot_mapping``:
    codes ``int8 [NB][Hkv][BS][D]`` (head-major), scales ``float32 [NB][Hkv][BS]``."""
    lib = load_library()
    T, Hkv, D = key.shape
    NB, Hkv2, BS, D2 = k_codes.shape
    if (value.shape != key.shape or v_codes.shape != k_codes.shape or (Hkv2, D2) != (Hkv, D)
            or k_scales.shape != (NB, Hkv, BS) or v_scales.shape != k_scales.shape):
        raise ValueError("reshape_and_cache_int8: inconsistent shapes")
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [num_tokens]")
    dt = _dtype_code(key)
    _dev(value, "value", key.dtype)
    for n, x in (("k_codes", k_codes), ("v_codes", v_codes)):
        _dev(x, n, torch.int8)
    for n, x in (("k_scales", k_scales), ("v_scales", v_scales)):
        _dev(x, n, torch.float32)
    _check(lib.pa_reshape_and_cache_int8(
        _dev(key, "key"), value.data_ptr(), k_codes.data_ptr(), v_codes.data_ptr(),
        k_scales.data_ptr(), v_scales.data_ptr(), _dev(slot_mapping, "slot_mapping", torch.int64),
        T, Hkv, D, BS, NB, dt, _stream(key, stream)))


def pa_decode_int8(out, q, k_codes, v_codes, k_scales, v_scales, block_tables, context_lens,
                   scale: float, max_context_len: int, partition_size: int = 512, workspace=None,
                   seq_order=None, stream=None) -> torch.Tensor:
    """Paged decode over an INT8 cache (see :func:`pa_reshape_and_cache_int8`)."""
    lib, B, Hq, Hkv, D, BS, NB, dt, ws_ptr, ws_bytes, order_ptr = _decode_common(
        q, k_codes, v_codes, block_tables, context_lens, seq_order, out, max_context_len,
        partition_size, workspace, cache_dtype=torch.int8, head_major=True)
    if k_scales.shape != (NB, Hkv, BS) or v_scales.shape != k_scales.shape:
        raise ValueError("decode_int8: scales must be [num_blocks][num_kv_heads][block_size]")
    ks = _dev(k_scales, "k_scales", torch.float32)
    vs = _dev(v_scales, "v_scales", torch.float32)
    _check(lib.pa_decode_int8(
        out.data_ptr(), q.data_ptr(), k_codes.data_ptr(), v_codes.data_ptr(), ks, vs,
        _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
        order_ptr, B, Hq, Hkv, D, BS, NB, block_tables.shape[1], max_context_len, scale,
        partition_size, ws_ptr, ws_bytes, dt, _stream(q, stream)))
    return out
