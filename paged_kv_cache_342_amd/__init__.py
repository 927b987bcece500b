"""Paged decode attention for AMD Instinct MI355X (gfx950).

A thin ctypes binding over libpa.so (see include/pa.h): it marshals torch
tensors into device pointers and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  The library must be built
first (``python -m paged_kv_cache_342_amd.build``); nothing here falls back to
another implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from .blocks import BlockManager, slot_mapping  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpa.so")
# the same library whose entry points also check the device-side contract on
# the device and reject a violating call (include/pa.h, "Checked build")
LIB_CHECKED_PATH = os.path.join(_PKG, "libpa_checked.so")

F32, F16, BF16, FP8_E4M3, FP4_E2M1 = 0, 1, 2, 3, 4
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_NO_BLOCKS, ERR_CONTRACT = 0, -1, -2, -3, -4, -5, -6
VIOLATION_BLOCK_ID, VIOLATION_CONTEXT_LEN, VIOLATION_SLOT, VIOLATION_SLOT_REPEATED = 0x01, 0x02, 0x04, 0x08
VIOLATION_COPY_ID, VIOLATION_COPY_DST_REPEATED, VIOLATION_COPY_DST_IS_SRC, VIOLATION_QUERY_START = 0x10, 0x20, 0x40, 0x80
VIOLATION_APPEND_BLOCK_SHARED, VIOLATION_PREFIX_GROUP = 0x100, 0x200

# an FP4 cache holds two E2M1 codes per byte: torch.float4_e2m1fn_x2, last dim head_dim / 2
_TORCH_CODE = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16, torch.float8_e4m3fn: FP8_E4M3,
               torch.float4_e2m1fn_x2: FP4_E2M1}


def _head_dim(cache: torch.Tensor) -> int:
    """head_dim of a cache [num_blocks, Hkv, bs, row]: the row holds two FP4 codes per element."""
    return cache.shape[-1] * (2 if cache.dtype == torch.float4_e2m1fn_x2 else 1)

_libs = {}
_checked = os.environ.get("PA_LIBRARY", "") == "checked"


class PagedAttentionError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def library() -> ctypes.CDLL:
    """The library every call goes through: libpa.so, or libpa_checked.so after
    use_checked_library() (or with PA_LIBRARY=checked in the environment).
    Raises if it has not been built."""
    path = LIB_CHECKED_PATH if _checked else LIB_PATH
    if path not in _libs:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_cache_342_amd.build`")
        _libs[path] = _load(path)
    return _libs[path]


def use_checked_library(checked: bool = True) -> None:
    """Route the calls that follow through libpa_checked.so (True) or libpa.so
    (False).  The checked library validates the device-side contract before
    each call's work and raises PagedAttentionError(ERR_CONTRACT) on a
    violation; every call then waits for its stream."""
    global _checked
    _checked = bool(checked)
    library()


def _load(path: str) -> ctypes.CDLL:
    lib = ctypes.CDLL(path)
    p, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.pa_reshape_and_cache.argtypes = [p, p, p, p, p, i32, i32, i32, i32, i64, i32, i32, f32, f32, p]
    lib.pa_reshape_and_cache.restype = ctypes.c_int
    lib.pa_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.pa_decode_workspace_size.restype = sz
    lib.pa_decode.argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, i32, i64, i32, i32, f32, f32, f32,
                              i32, i32, i32, p, sz, p]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode_window.argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, i32, i64, i32, i32, i32, i32, f32, f32,
                                     f32, i32, i32, i32, p, sz, p]
    lib.pa_decode_window.restype = ctypes.c_int
    lib.pa_decode_shared_prefix_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
    lib.pa_decode_shared_prefix_workspace_size.restype = sz
    lib.pa_decode_shared_prefix.argtypes = [p, p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32, i64, i32, i32,
                                            f32, f32, f32, i32, i32, i32, p, sz, p]
    lib.pa_decode_shared_prefix.restype = ctypes.c_int
    lib.pa_decode_append.argtypes = [p, p, p, p, p, p, i32, p, p, i32, i32, i32, i32, i32, i64, i32, i32, f32,
                                     f32, f32, i32, i32, i32, p, sz, p]
    lib.pa_decode_append.restype = ctypes.c_int
    lib.pa_reshape_and_cache_scaled.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i64, i32, i32, p]
    lib.pa_reshape_and_cache_scaled.restype = ctypes.c_int
    lib.pa_decode_scaled.argtypes = [p, p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i64, i32, i32, f32, i32, i32,
                                     i32, p, sz, p]
    lib.pa_decode_scaled.restype = ctypes.c_int
    lib.pa_decode_multi_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.pa_decode_multi_workspace_size.restype = sz
    lib.pa_decode_multi.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32, i64, i32, i32, f32, f32,
                                    f32, i32, i32, i32, p, sz, p]
    lib.pa_decode_multi.restype = ctypes.c_int
    lib.pa_copy_blocks.argtypes = [p, p, p, i32, i32, i32, i32, i64, i32, p]
    lib.pa_copy_blocks.restype = ctypes.c_int
    lib.pa_copy_blocks_scaled.argtypes = [p, p, p, p, p, i32, i32, i32, i32, i64, i32, p]
    lib.pa_copy_blocks_scaled.restype = ctypes.c_int
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_last_error_message.argtypes = []
    lib.pa_last_error_message.restype = ctypes.c_char_p
    lib.pa_version.argtypes = []
    lib.pa_version.restype = ctypes.c_char_p
    lib.pa_decode_append_noalloc.argtypes = [p, p, p, p, p, p, i32, p, p, i32, i32, i32, i32, i32, i64, i32, i32,
                                             f32, f32, f32, i32, i32, i32, p]
    lib.pa_decode_append_noalloc.restype = ctypes.c_int
    lib.pa_time_next_attention_kernel.argtypes = [p, p]
    lib.pa_time_next_attention_kernel.restype = ctypes.c_int
    lib.pa_read_probe.argtypes = [p, ctypes.c_size_t, i32, p, ctypes.c_size_t, p]
    lib.pa_read_probe.restype = ctypes.c_int
    lib.pa_is_checked_build.argtypes = []
    lib.pa_is_checked_build.restype = ctypes.c_int32
    lib.pa_bm_create.argtypes = [i64, i32]
    lib.pa_bm_create.restype = p
    lib.pa_bm_destroy.argtypes = [p]
    lib.pa_bm_destroy.restype = None
    lib.pa_bm_add.argtypes = [p, i64]
    lib.pa_bm_add.restype = ctypes.c_int
    lib.pa_bm_fork.argtypes = [p, i64, i64]
    lib.pa_bm_fork.restype = ctypes.c_int
    lib.pa_bm_append.argtypes = [p, i64, i32, p, p, p]
    lib.pa_bm_append.restype = ctypes.c_int
    lib.pa_bm_append_batch.argtypes = [p, p, i32, p, p, p, p]
    lib.pa_bm_append_batch.restype = ctypes.c_int
    lib.pa_bm_free.argtypes = [p, i64]
    lib.pa_bm_free.restype = ctypes.c_int
    lib.pa_bm_evict.argtypes = [p, i64, i64, i64, p]
    lib.pa_bm_evict.restype = ctypes.c_int
    lib.pa_bm_table.argtypes = [p, i64, p, i32]
    lib.pa_bm_table.restype = ctypes.c_int32
    lib.pa_bm_tables.argtypes = [p, p, i32, p, i32, p, i32]
    lib.pa_bm_tables.restype = ctypes.c_int
    lib.pa_bm_length.argtypes = [p, i64]
    lib.pa_bm_length.restype = ctypes.c_int64
    lib.pa_bm_get_stats.argtypes = [p, p]
    lib.pa_bm_get_stats.restype = ctypes.c_int
    return lib


def _check(status: int):
    if status != OK:
        lib = library()
        msg = lib.pa_last_error_message().decode() or lib.pa_status_string(status).decode()
        raise PagedAttentionError(status, msg)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _require(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _out(out: Optional[torch.Tensor], shape, out_dtype, like: torch.Tensor) -> torch.Tensor:
    """The caller's output tensor after checking that it has the call's shape
    (a wrong shape would make the kernels write outside it), or a new one."""
    if out is None:
        return torch.empty(shape, dtype=out_dtype or like.dtype, device=like.device)
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out must have shape {tuple(shape)}, got {tuple(out.shape)}")
    _require(out, "out", (torch.float32, torch.float16, torch.bfloat16))
    return out


def _max_context(max_context_len: Optional[int], M: int, bs: int) -> int:
    """The host-side length bound a call plans with: None or <= 0 means every
    table entry, M * block_size (as the C calls read <= 0)."""
    return M * bs if max_context_len is None or int(max_context_len) <= 0 else int(max_context_len)


def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      slot_mapping: torch.Tensor, k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """Write key/value rows [T, Hkv, D] into the slots slot_mapping[T] (int64, negative = skip)
    of the caches [num_blocks, Hkv, block_size, D] (same dtype as the rows, or float8_e4m3fn)."""
    for t, n in ((key, "key"), (value, "value"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _require(t, n)
    _require(slot_mapping, "slot_mapping", torch.int64)
    T, Hkv, D = key.shape
    nb, Hkv2, bs, D2 = k_cache.shape
    if value.shape != key.shape or v_cache.shape != k_cache.shape or (Hkv2, D2) != (Hkv, D) or slot_mapping.shape != (T,):
        raise ValueError("shape mismatch between key/value, caches and slot_mapping")
    _check(library().pa_reshape_and_cache(
        _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), T, Hkv, D, bs, nb,
        _TORCH_CODE.get(key.dtype, -9), _TORCH_CODE.get(k_cache.dtype, -9), k_scale, v_scale, _stream(k_cache)))


def decode_workspace_size(B: int, num_kv_heads: int, group: int, head_dim: int, block_size: int,
                          max_context_len: int) -> int:
    return int(library().pa_decode_workspace_size(B, num_kv_heads, group, head_dim, block_size, max_context_len))


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
           context_lens: torch.Tensor, scale: float, max_context_len: Optional[int] = None,
           k_scale: float = 1.0, v_scale: float = 1.0, out: Optional[torch.Tensor] = None,
           out_dtype: Optional[torch.dtype] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Paged decode attention: q [B, Hq, D] over the caches through block_tables [B, M] (int32)
    and context_lens [B] (int32).  Returns out [B, Hq, D] (out_dtype, default q's dtype)."""
    _require(q, "q")
    _require(k_cache, "k_cache")
    _require(v_cache, "v_cache")
    _require(block_tables, "block_tables", torch.int32)
    _require(context_lens, "context_lens", torch.int32)
    B, Hq, D = q.shape
    nb, Hkv, bs, D2 = k_cache.shape
    if D2 != D or v_cache.shape != k_cache.shape or Hq % Hkv:
        raise ValueError("q, k_cache and v_cache shapes do not agree")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [B, M] and context_lens [B]")
    M = block_tables.shape[1]
    mcl = _max_context(max_context_len, M, bs)
    out = _out(out, (B, Hq, D), out_dtype, q)
    need = decode_workspace_size(B, Hkv, Hq // Hkv, D, bs, mcl) if B else 0
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().pa_decode(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        B, Hkv, Hq // Hkv, D, bs, nb, M, mcl, scale, k_scale, v_scale,
        _TORCH_CODE.get(q.dtype, -9), _TORCH_CODE.get(k_cache.dtype, -9), _TORCH_CODE.get(out.dtype, -9),
        _ptr(workspace), ws_bytes, _stream(q)))
    return out


def decode_shared_prefix_workspace_size(B: int, num_groups: int, max_group_size: int, num_kv_heads: int, group: int,
                                        head_dim: int, block_size: int, max_context_len: int) -> int:
    return int(library().pa_decode_shared_prefix_workspace_size(B, num_groups, max_group_size, num_kv_heads, group,
                                                                head_dim, block_size, max_context_len))


def decode_shared_prefix(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                         context_lens: torch.Tensor, group_start: torch.Tensor, prefix_lens: torch.Tensor,
                         max_group_size: int, scale: float, max_context_len: Optional[int] = None,
                         k_scale: float = 1.0, v_scale: float = 1.0, out: Optional[torch.Tensor] = None,
                         out_dtype: Optional[torch.dtype] = None,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """decode() over sequences grouped by a shared prefix: group p is sequences
    group_start[p] .. group_start[p+1]-1 (int32 [P+1] on the device), which share
    their first prefix_lens[p] positions (int32 [P]); each prefix is read once
    per group.  max_group_size: host bound of members per group."""
    _require(q, "q")
    _require(k_cache, "k_cache")
    _require(v_cache, "v_cache")
    _require(block_tables, "block_tables", torch.int32)
    _require(context_lens, "context_lens", torch.int32)
    _require(group_start, "group_start", torch.int32)
    _require(prefix_lens, "prefix_lens", torch.int32)
    B, Hq, D = q.shape
    nb, Hkv, bs, D2 = k_cache.shape
    if D2 != D or v_cache.shape != k_cache.shape or Hq % Hkv:
        raise ValueError("q, k_cache and v_cache shapes do not agree")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [B, M] and context_lens [B]")
    P = prefix_lens.shape[0] if prefix_lens.dim() == 1 else -1
    if P < 1 or group_start.shape != (P + 1,):
        raise ValueError("prefix_lens must be [P] and group_start [P + 1]")
    M = block_tables.shape[1]
    mcl = _max_context(max_context_len, M, bs)
    out = _out(out, (B, Hq, D), out_dtype, q)
    need = decode_shared_prefix_workspace_size(B, P, max_group_size, Hkv, Hq // Hkv, D, bs, mcl) if B else 0
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().pa_decode_shared_prefix(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), _ptr(group_start),
        _ptr(prefix_lens), B, P, int(max_group_size), Hkv, Hq // Hkv, D, bs, nb, M, mcl, scale, k_scale, v_scale,
        _TORCH_CODE.get(q.dtype, -9), _TORCH_CODE.get(k_cache.dtype, -9), _TORCH_CODE.get(out.dtype, -9),
        _ptr(workspace), ws_bytes, _stream(q)))
    return out


def decode_window(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                  context_lens: torch.Tensor, scale: float, sink_tokens: int, window_tokens: int,
                  max_context_len: Optional[int] = None, k_scale: float = 1.0, v_scale: float = 1.0,
                  out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """decode() over each sequence's attention sinks and sliding window only:
    positions t < sink_tokens and t >= L - window_tokens (window_tokens >= 1)."""
    _require(q, "q")
    _require(k_cache, "k_cache")
    _require(v_cache, "v_cache")
    _require(block_tables, "block_tables", torch.int32)
    _require(context_lens, "context_lens", torch.int32)
    B, Hq, D = q.shape
    nb, Hkv, bs, D2 = k_cache.shape
    if D2 != D or v_cache.shape != k_cache.shape or Hq % Hkv:
        raise ValueError("q, k_cache and v_cache shapes do not agree")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [B, M] and context_lens [B]")
    M = block_tables.shape[1]
    mcl = _max_context(max_context_len, M, bs)
    out = _out(out, (B, Hq, D), out_dtype, q)
    need = decode_workspace_size(B, Hkv, Hq // Hkv, D, bs, mcl) if B else 0
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().pa_decode_window(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        B, Hkv, Hq // Hkv, D, bs, nb, M, mcl, int(sink_tokens), int(window_tokens), scale, k_scale, v_scale,
        _TORCH_CODE.get(q.dtype, -9), _TORCH_CODE.get(k_cache.dtype, -9), _TORCH_CODE.get(out.dtype, -9),
        _ptr(workspace), ws_bytes, _stream(q)))
    return out


def decode_append(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, key: torch.Tensor,
                  value: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                  max_context_len: Optional[int] = None, k_scale: float = 1.0, v_scale: float = 1.0,
                  out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step: append key/value [B, Hkv, D] (the row of position context_lens[s] - 1 of
    each sequence) into the caches, then attend as decode() does.  Returns out [B, Hq, D]."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (key, "key"), (value, "value")):
        _require(t, n)
    _require(block_tables, "block_tables", torch.int32)
    _require(context_lens, "context_lens", torch.int32)
    B, Hq, D = q.shape
    nb, Hkv, bs, D2 = k_cache.shape
    if D2 != D or v_cache.shape != k_cache.shape or Hq % Hkv:
        raise ValueError("q, k_cache and v_cache shapes do not agree")
    if key.shape != (B, Hkv, D) or value.shape != key.shape:
        raise ValueError("key and value must be [B, num_kv_heads, head_dim]")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [B, M] and context_lens [B]")
    M = block_tables.shape[1]
    mcl = _max_context(max_context_len, M, bs)
    out = _out(out, (B, Hq, D), out_dtype, q)
    need = decode_workspace_size(B, Hkv, Hq // Hkv, D, bs, mcl) if B else 0
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().pa_decode_append(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(key), _ptr(value), _TORCH_CODE.get(key.dtype, -9),
        _ptr(block_tables), _ptr(context_lens), B, Hkv, Hq // Hkv, D, bs, nb, M, mcl, scale, k_scale, v_scale,
        _TORCH_CODE.get(q.dtype, -9), _TORCH_CODE.get(k_cache.dtype, -9), _TORCH_CODE.get(out.dtype, -9),
        _ptr(workspace), ws_bytes, _stream(q)))
    return out


def decode_append_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, key: torch.Tensor,
                          value: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                          out: torch.Tensor, max_context_len: Optional[int] = None, k_scale: float = 1.0,
                          v_scale: float = 1.0) -> torch.Tensor:
    """decode_append() through pa_decode_append_noalloc, which allocates
    nothing: the split partials live in the library's own per-device scratch
    array (64 MiB).  The caller passes every tensor, `out` included; sizes
    whose partials do not fit raise PagedAttentionError(ERR_WORKSPACE).
    Calls that overlap on one device share that array and race."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (key, "key"), (value, "value")):
        _require(t, n)
    _require(block_tables, "block_tables", torch.int32)
    _require(context_lens, "context_lens", torch.int32)
    B, Hq, D = q.shape
    nb, Hkv, bs, D2 = k_cache.shape
    if D2 != D or v_cache.shape != k_cache.shape or Hq % Hkv:
        raise ValueError("q, k_cache and v_cache shapes do not agree")
    if key.shape != (B, Hkv, D) or value.shape != key.shape:
        raise ValueError("key and value must be [B, num_kv_heads, head_dim]")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [B, M] and context_lens [B]")
    M = block_tables.shape[1]
    out = _out(out, (B, Hq, D), None, q)
    _check(library().pa_decode_append_noalloc(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(key), _ptr(value), _TORCH_CODE.get(key.dtype, -9),
        _ptr(block_tables), _ptr(context_lens), B, Hkv, Hq // Hkv, D, bs, nb, M, _max_context(max_context_len, M, bs),
        scale, k_scale, v_scale, _TORCH_CODE.get(q.dtype, -9), _TORCH_CODE.get(k_cache.dtype, -9),
        _TORCH_CODE.get(out.dtype, -9), _stream(q)))
    return out


def reshape_and_cache_scaled(key: torch.Tensor, value: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                             k_scales: torch.Tensor, v_scales: torch.Tensor, slot_mapping: torch.Tensor) -> None:
    """Write key/value rows [T, Hkv, D] (f16/bf16) into an FP8 cache [num_blocks, Hkv, bs, D]
    (float8_e4m3fn) or an FP4 cache [num_blocks, Hkv, bs, D / 2] (float4_e2m1fn_x2), each (token,
    head) row against its own scale (largest magnitude / 448, or / 6), stored in k_scales / v_scales
    [num_blocks, Hkv, bs] float32."""
    for t, n in ((key, "key"), (value, "value"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _require(t, n)
    _require(k_scales, "k_scales", torch.float32)
    _require(v_scales, "v_scales", torch.float32)
    _require(slot_mapping, "slot_mapping", torch.int64)
    T, Hkv, D = key.shape
    nb, Hkv2, bs, _ = k_cache.shape
    if (value.shape != key.shape or v_cache.shape != k_cache.shape or (Hkv2, _head_dim(k_cache)) != (Hkv, D)
            or slot_mapping.shape != (T,) or k_scales.shape != (nb, Hkv, bs) or v_scales.shape != k_scales.shape):
        raise ValueError("shape mismatch between key/value, caches, scale pools and slot_mapping")
    _scaled_cache(k_cache, v_cache)
    _check(library().pa_reshape_and_cache_scaled(
        _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales), _ptr(slot_mapping),
        T, Hkv, D, bs, nb, _TORCH_CODE.get(key.dtype, -9), _TORCH_CODE[k_cache.dtype], _stream(k_cache)))


def _scaled_cache(k_cache: torch.Tensor, v_cache: torch.Tensor) -> None:
    ok = (torch.float8_e4m3fn, torch.float4_e2m1fn_x2)
    if k_cache.dtype not in ok or v_cache.dtype != k_cache.dtype:
        raise ValueError("row scales are for FP8 (float8_e4m3fn) and FP4 (float4_e2m1fn_x2) caches")


def decode_scaled(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, k_scales: torch.Tensor,
                  v_scales: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                  max_context_len: Optional[int] = None, out: Optional[torch.Tensor] = None,
                  out_dtype: Optional[torch.dtype] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """decode() over an FP8 or FP4 cache whose rows carry their own scales ([num_blocks, Hkv, bs] float32)."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _require(t, n)
    _require(k_scales, "k_scales", torch.float32)
    _require(v_scales, "v_scales", torch.float32)
    _require(block_tables, "block_tables", torch.int32)
    _require(context_lens, "context_lens", torch.int32)
    B, Hq, D = q.shape
    nb, Hkv, bs, _ = k_cache.shape
    _scaled_cache(k_cache, v_cache)
    if _head_dim(k_cache) != D or v_cache.shape != k_cache.shape or Hq % Hkv or k_scales.shape != (nb, Hkv, bs) \
            or v_scales.shape != k_scales.shape:
        raise ValueError("q, caches and scale pools do not agree")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [B, M] and context_lens [B]")
    M = block_tables.shape[1]
    mcl = _max_context(max_context_len, M, bs)
    out = _out(out, (B, Hq, D), out_dtype, q)
    need = decode_workspace_size(B, Hkv, Hq // Hkv, D, bs, mcl) if B else 0
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().pa_decode_scaled(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales), _ptr(block_tables),
        _ptr(context_lens), B, Hkv, Hq // Hkv, D, bs, nb, M, mcl, scale, _TORCH_CODE.get(q.dtype, -9),
        _TORCH_CODE[k_cache.dtype], _TORCH_CODE.get(out.dtype, -9), _ptr(workspace), ws_bytes, _stream(q)))
    return out


def decode_multi_workspace_size(B: int, num_kv_heads: int, group: int, head_dim: int, block_size: int,
                                max_context_len: int, max_queries: int) -> int:
    return int(library().pa_decode_multi_workspace_size(B, num_kv_heads, group, head_dim, block_size,
                                                        max_context_len, max_queries))


def decode_multi(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                 context_lens: torch.Tensor, query_start: torch.Tensor, max_queries: int, scale: float,
                 max_context_len: Optional[int] = None, k_scale: float = 1.0, v_scale: float = 1.0,
                 out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Several queries per sequence: q [T, Hq, D], sequence s owning rows query_start[s] ..
    query_start[s+1]-1 (int32 [B+1] on the device), its last positions, causal within them.
    max_queries: host-side bound of queries per sequence.  Returns out [T, Hq, D]."""
    _require(q, "q")
    _require(k_cache, "k_cache")
    _require(v_cache, "v_cache")
    _require(block_tables, "block_tables", torch.int32)
    _require(context_lens, "context_lens", torch.int32)
    _require(query_start, "query_start", torch.int32)
    T, Hq, D = q.shape
    nb, Hkv, bs, D2 = k_cache.shape
    if D2 != D or v_cache.shape != k_cache.shape or Hq % Hkv:
        raise ValueError("q, k_cache and v_cache shapes do not agree")
    B = context_lens.shape[0]
    if block_tables.dim() != 2 or block_tables.shape[0] != B or query_start.shape != (B + 1,):
        raise ValueError("block_tables must be [B, M], context_lens [B] and query_start [B + 1]")
    M = block_tables.shape[1]
    mcl = _max_context(max_context_len, M, bs)
    out = _out(out, (T, Hq, D), out_dtype, q)
    need = decode_multi_workspace_size(B, Hkv, Hq // Hkv, D, bs, mcl, max_queries) if B else 0
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().pa_decode_multi(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), _ptr(query_start),
        B, T, int(max_queries), Hkv, Hq // Hkv, D, bs, nb, M, mcl, scale, k_scale, v_scale,
        _TORCH_CODE.get(q.dtype, -9), _TORCH_CODE.get(k_cache.dtype, -9), _TORCH_CODE.get(out.dtype, -9),
        _ptr(workspace), ws_bytes, _stream(q)))
    return out


def _pairs_shape(block_mapping: torch.Tensor) -> None:
    if block_mapping.numel() and (block_mapping.dim() != 2 or block_mapping.shape[1] != 2):
        raise ValueError(f"block_mapping must be [N, 2], got {tuple(block_mapping.shape)}")


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, block_mapping: torch.Tensor) -> None:
    """Copy-on-write: k_cache[dst] = k_cache[src] (and V) for each (src, dst) row of block_mapping [N, 2] int64."""
    _require(k_cache, "k_cache")
    _require(v_cache, "v_cache")
    _require(block_mapping, "block_mapping", torch.int64)
    _pairs_shape(block_mapping)
    nb, Hkv, bs, _ = k_cache.shape
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes do not agree")
    N = block_mapping.shape[0] if block_mapping.numel() else 0
    _check(library().pa_copy_blocks(
        _ptr(k_cache), _ptr(v_cache), _ptr(block_mapping) if N else None, N, Hkv, _head_dim(k_cache), bs, nb,
        _TORCH_CODE.get(k_cache.dtype, -9), _stream(k_cache)))


def copy_blocks_scaled(k_cache: torch.Tensor, v_cache: torch.Tensor, k_scales: torch.Tensor, v_scales: torch.Tensor,
                       block_mapping: torch.Tensor) -> None:
    """copy_blocks() for an FP8 or FP4 cache with row scales: the blocks' rows and their scales."""
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _require(t, n)
    _require(k_scales, "k_scales", torch.float32)
    _require(v_scales, "v_scales", torch.float32)
    _require(block_mapping, "block_mapping", torch.int64)
    _pairs_shape(block_mapping)
    _scaled_cache(k_cache, v_cache)
    nb, Hkv, bs, _ = k_cache.shape
    if v_cache.shape != k_cache.shape or k_scales.shape != (nb, Hkv, bs) or v_scales.shape != k_scales.shape:
        raise ValueError("caches and scale pools do not agree")
    N = block_mapping.shape[0] if block_mapping.numel() else 0
    _check(library().pa_copy_blocks_scaled(
        _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales), _ptr(block_mapping) if N else None, N, Hkv,
        _head_dim(k_cache), bs, nb, _TORCH_CODE[k_cache.dtype], _stream(k_cache)))


def time_next_attention_kernel(start: torch.cuda.Event, stop: torch.cuda.Event) -> None:
    """Have the next decode call on this thread record `start` when its first
    attention kernel begins and `stop` when its last one ends, on the call's
    stream (timing events, enable_timing=True); start.elapsed_time(stop) is
    then the attention kernel alone, without the split merge."""
    for ev in (start, stop):
        if not ev.cuda_event:  # torch creates the underlying event on its first record
            ev.record()
    _check(library().pa_time_next_attention_kernel(start.cuda_event, stop.cuda_event))


def read_probe(buf: torch.Tensor, chunk_bytes: int = 4096, sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Stream the bytes of `buf` (a contiguous device tensor) once through the
    read-bandwidth probe in chunks of `chunk_bytes` (each wave reading whole
    chunks); returns the sink (per workgroup, the XOR of the 32-bit words it
    read).  For timing the device's read rate."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    if sink is None:
        sink = torch.empty(256, dtype=torch.int32, device=buf.device)
    _check(library().pa_read_probe(_ptr(buf), buf.numel() * buf.element_size(), chunk_bytes, _ptr(sink),
                                   sink.numel() * sink.element_size(), _stream(buf)))
    return sink


def version() -> str:
    return library().pa_version().decode()
