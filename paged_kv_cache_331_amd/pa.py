"""ctypes binding of the C-ABI HIP library (``include/pa.h``).

Argument marshalling only: tensors become device pointers and sizes, the
current torch stream becomes the ``hipStream_t``, and a non-zero status
becomes :class:`PagedAttentionError`. Every step of the computation runs in
the HIP kernels; there is no fallback. If the built library is missing,
loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa_gfx950.so")

PA_DTYPE_FP16 = 0
PA_DTYPE_BF16 = 1
PA_OK = 0
STATUS = {0: "PA_OK", -1: "PA_ERR_NULL", -2: "PA_ERR_SHAPE", -3: "PA_ERR_DTYPE",
          -4: "PA_ERR_UNSUPPORTED", -5: "PA_ERR_WORKSPACE", -6: "PA_ERR_HIP",
          -7: "PA_ERR_NO_BLOCKS", -8: "PA_ERR_STATE"}

_i32, _i64, _f32, _vp, _sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                              ctypes.c_void_p, ctypes.c_size_t)

# name -> (restype, argtypes); mirrors include/pa.h
SIGNATURES = {
    "pa_abi_version": (ctypes.c_int, []),
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_decode_slot_mapping": (ctypes.c_int, [_vp, _i32, _vp, _i32, _i32, _vp, _vp]),
    "pa_cache_write": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32,
                                      _i32, _vp]),
    "pa_decode_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pa_decode_partition_size": (_i32, [_i32, _i32, _i32, _i32, _i32]),
    "pa_decode": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _f32, _vp, _i32, _i32, _i32, _i32,
                                 _i32, _i64, _i32, _i32, _i32, _i32, _vp, _sz, _vp]),
    "pa_cache_write_fp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32,
                                          _i32, _f32, _f32, _vp]),
    "pa_decode_cascade_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode_cascade": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _f32, _vp, _i32, _i32, _i32,
                                         _i32, _i32, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _sz,
                                         _vp]),
    "pa_prefill_slot_mapping": (ctypes.c_int, [_vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                                               _i32, _vp, _vp]),
    "pa_prefill": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _i32, _i32, _i32,
                                  _i32, _i32, _i32, _i32, _i64, _i32, _i32, _i32, _vp]),
    "pa_prefill_fp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _f32, _f32, _f32, _vp, _i32,
                                      _i32, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _i32,
                                      _vp]),
    "pa_pool_create": (_vp, [_i32]),
    "pa_pool_destroy": (None, [_vp]),
    "pa_pool_num_free": (_i32, [_vp]),
    "pa_pool_ref_count": (_i32, [_vp, _i32]),
    "pa_pool_allocate": (ctypes.c_int, [_vp, _i32, _vp]),
    "pa_pool_free": (ctypes.c_int, [_vp, _vp, _i32]),
    "pa_pool_share": (ctypes.c_int, [_vp, _vp, _i32]),
    "pa_pool_copy_on_write": (ctypes.c_int, [_vp, _vp, _vp, _vp]),
    "pa_copy_blocks": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32, _i32, _vp]),
    "pa_decode_fp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _f32, _f32, _f32, _vp, _i32, _i32,
                                     _i32, _i32, _i32, _i64, _i32, _i32, _i32, _i32, _vp, _sz,
                                     _vp]),
    "pa_decode_append": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _i32,
                                        _i32, _i32, _i32, _i32, _i64, _i32, _i32, _i32, _i32,
                                        _i32, _vp, _sz, _vp]),
    "pa_decode_append_static": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp,
                                               _vp, _i32, _i32, _i32, _i32, _i32, _i64, _i32,
                                               _i32, _i32, _i32, _i32, _vp]),
    "pa_decode_append_fp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _f32, _f32,
                                            _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i64, _i32,
                                            _i32, _i32, _i32, _vp, _sz, _vp]),
}

_lib: Optional[ctypes.CDLL] = None


class PagedAttentionError(RuntimeError):
    """A library call returned a non-zero status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({status_string(status)})")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing "
                           "(run `python -m paged_kv_cache_331_amd.build`)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().pa_status_string(int(status)).decode()


def abi_version() -> int:
    return int(load().pa_abi_version())


def _check(fn: str, status: int) -> None:
    if status != PA_OK:
        raise PagedAttentionError(fn, status)


def dtype_code(t: torch.dtype) -> int:
    if t == torch.float16:
        return PA_DTYPE_FP16
    if t == torch.bfloat16:
        return PA_DTYPE_BF16
    raise TypeError(f"unsupported storage dtype {t}")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return int(getattr(stream, "cuda_stream", stream))


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def decode_slot_mapping(block_tables: torch.Tensor, context_lens: torch.Tensor,
                        block_size: int, out: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """Slot of each sequence's newest token (position L-1), -1 for L == 0."""
    B, MB = block_tables.shape
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=block_tables.device)
    st = load().pa_decode_slot_mapping(_dev(block_tables, "block_tables"), MB,
                                       _dev(context_lens, "context_lens"), B, int(block_size),
                                       _dev(out, "slot_mapping"), _stream(stream))
    _check("pa_decode_slot_mapping", st)
    return out


def cache_write(k: torch.Tensor, v: torch.Tensor, key_cache: torch.Tensor,
                value_cache: torch.Tensor, slot_mapping: torch.Tensor, stream=None) -> None:
    """Store k[i], v[i] ([T, Hkv, D]) at slot_mapping[i] of the caches, in place."""
    NB, bs, Hkv, D = key_cache.shape
    T = k.shape[0]
    st = load().pa_cache_write(_dev(k, "k"), _dev(v, "v"), _dev(key_cache, "key_cache"),
                               _dev(value_cache, "value_cache"),
                               _dev(slot_mapping, "slot_mapping"), T, NB, bs, Hkv, D,
                               dtype_code(key_cache.dtype), _stream(stream))
    _check("pa_cache_write", st)


def cache_write_fp8(k: torch.Tensor, v: torch.Tensor, key_cache: torch.Tensor,
                    value_cache: torch.Tensor, slot_mapping: torch.Tensor, k_scale: float,
                    v_scale: float, stream=None) -> None:
    """Quantize k[i], v[i] ([T, Hkv, D], fp16/bf16) into the uint8 E4M3 caches at slot_mapping[i]."""
    if key_cache.dtype != torch.uint8 or value_cache.dtype != torch.uint8:
        raise TypeError("FP8 caches are uint8 tensors of E4M3 codes")
    NB, bs, Hkv, D = key_cache.shape
    T = k.shape[0]
    st = load().pa_cache_write_fp8(_dev(k, "k"), _dev(v, "v"), _dev(key_cache, "key_cache"),
                                   _dev(value_cache, "value_cache"),
                                   _dev(slot_mapping, "slot_mapping"), T, NB, bs, Hkv, D,
                                   dtype_code(k.dtype), float(k_scale), float(v_scale),
                                   _stream(stream))
    _check("pa_cache_write_fp8", st)


def decode_workspace_size(num_seqs: int, num_q_heads: int, head_size: int,
                          max_context_len: int, partition_size: int = 0) -> int:
    return int(load().pa_decode_workspace_size(num_seqs, num_q_heads, head_size,
                                               max_context_len, partition_size))


def decode_partition_size(num_seqs: int, num_kv_heads: int, max_context_len: int,
                          cache_elem_bytes: int = 2, num_cus: int = 0) -> int:
    """Tokens per partition of the automatic split (-1: single pass); cache_elem_bytes
    is 2 for pa_decode / the cascade, 1 for an FP8 cache."""
    return int(load().pa_decode_partition_size(num_seqs, num_kv_heads, max_context_len,
                                               cache_elem_bytes, num_cus))


def decode(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
           block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
           max_context_len: int, out: Optional[torch.Tensor] = None,
           partition_size: int = 0, workspace: Optional[torch.Tensor] = None,
           stream=None) -> torch.Tensor:
    """One paged decode-attention step; returns ``out`` ([B, Hq, D], dtype of q)."""
    B, Hq, D = q.shape
    NB, bs, Hkv, _ = key_cache.shape
    MB = block_tables.shape[1]
    if out is None:
        out = torch.empty_like(q)
    need = decode_workspace_size(B, Hq, D, max_context_len, partition_size)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().pa_decode(_dev(q, "q"), _dev(key_cache, "key_cache"),
                          _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables"),
                          _dev(context_lens, "context_lens"), float(scale), _dev(out, "out"),
                          B, Hq, Hkv, D, bs, NB, MB, int(max_context_len), int(partition_size),
                          dtype_code(q.dtype), ws_ptr, ws_len, _stream(stream))
    _check("pa_decode", st)
    return out


def decode_fp8(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
               block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
               k_scale: float, v_scale: float, max_context_len: int,
               out: Optional[torch.Tensor] = None, partition_size: int = 0,
               workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode step over uint8 E4M3 caches with per-tensor scales; ``out`` has q's dtype."""
    if key_cache.dtype != torch.uint8 or value_cache.dtype != torch.uint8:
        raise TypeError("FP8 caches are uint8 tensors of E4M3 codes")
    B, Hq, D = q.shape
    NB, bs, Hkv, _ = key_cache.shape
    MB = block_tables.shape[1]
    if out is None:
        out = torch.empty_like(q)
    need = decode_workspace_size(B, Hq, D, max_context_len, partition_size)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().pa_decode_fp8(_dev(q, "q"), _dev(key_cache, "key_cache"),
                              _dev(value_cache, "value_cache"),
                              _dev(block_tables, "block_tables"),
                              _dev(context_lens, "context_lens"), float(scale), float(k_scale),
                              float(v_scale), _dev(out, "out"), B, Hq, Hkv, D, bs, NB, MB,
                              int(max_context_len), int(partition_size), dtype_code(q.dtype),
                              ws_ptr, ws_len, _stream(stream))
    _check("pa_decode_fp8", st)
    return out


def decode_cascade_workspace_size(num_seqs: int, num_q_heads: int, head_size: int,
                                  block_size: int, max_context_len: int,
                                  shared_prefix_blocks: int, partition_size: int = 0) -> int:
    return int(load().pa_decode_cascade_workspace_size(num_seqs, num_q_heads, head_size,
                                                       block_size, max_context_len,
                                                       shared_prefix_blocks, partition_size))


def decode_cascade(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                   block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                   max_context_len: int, shared_prefix_blocks: int,
                   out: Optional[torch.Tensor] = None, partition_size: int = 0,
                   workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode step whose tables share their first ``shared_prefix_blocks`` entries."""
    B, Hq, D = q.shape
    NB, bs, Hkv, _ = key_cache.shape
    MB = block_tables.shape[1]
    if out is None:
        out = torch.empty_like(q)
    need = decode_cascade_workspace_size(B, Hq, D, bs, max_context_len, shared_prefix_blocks,
                                         partition_size)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().pa_decode_cascade(_dev(q, "q"), _dev(key_cache, "key_cache"),
                                  _dev(value_cache, "value_cache"),
                                  _dev(block_tables, "block_tables"),
                                  _dev(context_lens, "context_lens"), float(scale),
                                  _dev(out, "out"), B, Hq, Hkv, D, bs, NB, MB,
                                  int(max_context_len), int(shared_prefix_blocks),
                                  int(partition_size), dtype_code(q.dtype), ws_ptr, ws_len,
                                  _stream(stream))
    _check("pa_decode_cascade", st)
    return out


def decode_append(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, key_cache: torch.Tensor,
                  value_cache: torch.Tensor, block_tables: torch.Tensor,
                  context_lens: torch.Tensor, scale: float, max_context_len: int,
                  shared_prefix_blocks: int = 0, out: Optional[torch.Tensor] = None,
                  slot_mapping: Optional[torch.Tensor] = None, partition_size: int = 0,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Whole decode step in one call: store each sequence's new k/v ([B, Hkv, D]) at the
    slot of position L-1 (written to ``slot_mapping`` if given), then attend."""
    B, Hq, D = q.shape
    NB, bs, Hkv, _ = key_cache.shape
    MB = block_tables.shape[1]
    if out is None:
        out = torch.empty_like(q)
    need = decode_cascade_workspace_size(B, Hq, D, bs, max_context_len, shared_prefix_blocks,
                                         partition_size)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    slots_ptr = _dev(slot_mapping, "slot_mapping") if slot_mapping is not None else None
    st = load().pa_decode_append(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"),
                                 _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
                                 _dev(block_tables, "block_tables"),
                                 _dev(context_lens, "context_lens"), float(scale),
                                 _dev(out, "out"), slots_ptr, B, Hq, Hkv, D, bs, NB, MB,
                                 int(max_context_len), int(shared_prefix_blocks),
                                 int(partition_size), dtype_code(q.dtype), ws_ptr, ws_len,
                                 _stream(stream))
    _check("pa_decode_append", st)
    return out


STATIC_SCRATCH_BYTES = 32 << 20   # PA_STATIC_SCRATCH_BYTES of include/pa.h


def decode_append_static(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         key_cache: torch.Tensor, value_cache: torch.Tensor,
                         block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                         max_context_len: int, shared_prefix_blocks: int = 0,
                         out: Optional[torch.Tensor] = None,
                         slot_mapping: Optional[torch.Tensor] = None, partition_size: int = 0,
                         stream=None) -> torch.Tensor:
    """decode_append with its split-K workspace in the library's fixed device array
    (no allocation by the library; ``out`` is allocated here only when not given)."""
    B, Hq, D = q.shape
    NB, bs, Hkv, _ = key_cache.shape
    MB = block_tables.shape[1]
    if out is None:
        out = torch.empty_like(q)
    slots_ptr = _dev(slot_mapping, "slot_mapping") if slot_mapping is not None else None
    st = load().pa_decode_append_static(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"),
                                        _dev(key_cache, "key_cache"),
                                        _dev(value_cache, "value_cache"),
                                        _dev(block_tables, "block_tables"),
                                        _dev(context_lens, "context_lens"), float(scale),
                                        _dev(out, "out"), slots_ptr, B, Hq, Hkv, D, bs, NB, MB,
                                        int(max_context_len), int(shared_prefix_blocks),
                                        int(partition_size), dtype_code(q.dtype),
                                        _stream(stream))
    _check("pa_decode_append_static", st)
    return out


def decode_append_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      key_cache: torch.Tensor, value_cache: torch.Tensor,
                      block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                      k_scale: float, v_scale: float, max_context_len: int,
                      out: Optional[torch.Tensor] = None,
                      slot_mapping: Optional[torch.Tensor] = None, partition_size: int = 0,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """decode_append over uint8 E4M3 caches: the new rows are quantized with the scales."""
    if key_cache.dtype != torch.uint8 or value_cache.dtype != torch.uint8:
        raise TypeError("FP8 caches are uint8 tensors of E4M3 codes")
    B, Hq, D = q.shape
    NB, bs, Hkv, _ = key_cache.shape
    MB = block_tables.shape[1]
    if out is None:
        out = torch.empty_like(q)
    need = decode_workspace_size(B, Hq, D, max_context_len, partition_size)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    slots_ptr = _dev(slot_mapping, "slot_mapping") if slot_mapping is not None else None
    st = load().pa_decode_append_fp8(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"),
                                     _dev(key_cache, "key_cache"),
                                     _dev(value_cache, "value_cache"),
                                     _dev(block_tables, "block_tables"),
                                     _dev(context_lens, "context_lens"), float(scale),
                                     float(k_scale), float(v_scale), _dev(out, "out"), slots_ptr,
                                     B, Hq, Hkv, D, bs, NB, MB, int(max_context_len),
                                     int(partition_size), dtype_code(q.dtype), ws_ptr, ws_len,
                                     _stream(stream))
    _check("pa_decode_append_fp8", st)
    return out


def prefill_slot_mapping(block_tables: torch.Tensor, context_lens: torch.Tensor,
                         query_start: torch.Tensor, num_tokens: int, max_query_len: int,
                         block_size: int, max_context_len: int,
                         out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Slot of every new token of a prefill batch (int32 [num_tokens])."""
    B, MB = block_tables.shape
    if out is None:
        out = torch.empty(num_tokens, dtype=torch.int32, device=block_tables.device)
    st = load().pa_prefill_slot_mapping(_dev(block_tables, "block_tables"), MB,
                                        _dev(context_lens, "context_lens"),
                                        _dev(query_start, "query_start"), B, int(num_tokens),
                                        int(max_query_len), int(block_size),
                                        int(max_context_len), _dev(out, "slot_mapping"),
                                        _stream(stream))
    _check("pa_prefill_slot_mapping", st)
    return out


def prefill(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
            block_tables: torch.Tensor, context_lens: torch.Tensor, query_start: torch.Tensor,
            scale: float, max_query_len: int, max_context_len: int,
            out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Causal paged attention of the new tokens (q, out: [num_tokens, Hq, D])."""
    T, Hq, D = q.shape
    NB, bs, Hkv, _ = key_cache.shape
    B, MB = block_tables.shape
    if out is None:
        out = torch.empty_like(q)
    st = load().pa_prefill(_dev(q, "q"), _dev(key_cache, "key_cache"),
                           _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables"),
                           _dev(context_lens, "context_lens"), _dev(query_start, "query_start"),
                           float(scale), _dev(out, "out"), B, T, int(max_query_len), Hq, Hkv, D,
                           bs, NB, MB, int(max_context_len), dtype_code(q.dtype),
                           _stream(stream))
    _check("pa_prefill", st)
    return out


def prefill_fp8(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                block_tables: torch.Tensor, context_lens: torch.Tensor,
                query_start: torch.Tensor, scale: float, k_scale: float, v_scale: float,
                max_query_len: int, max_context_len: int, out: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """prefill over uint8 E4M3 caches whose codes stand for value * k_scale / v_scale."""
    T, Hq, D = q.shape
    NB, bs, Hkv, _ = key_cache.shape
    B, MB = block_tables.shape
    if out is None:
        out = torch.empty_like(q)
    st = load().pa_prefill_fp8(_dev(q, "q"), _dev(key_cache, "key_cache"),
                               _dev(value_cache, "value_cache"),
                               _dev(block_tables, "block_tables"),
                               _dev(context_lens, "context_lens"),
                               _dev(query_start, "query_start"), float(scale), float(k_scale),
                               float(v_scale), _dev(out, "out"), B, T, int(max_query_len), Hq,
                               Hkv, D, bs, NB, MB, int(max_context_len), dtype_code(q.dtype),
                               _stream(stream))
    _check("pa_prefill_fp8", st)
    return out


class BlockPool:
    """The library's host block pool (reference counts, free queue, copy-on-write)."""

    def __init__(self, num_blocks: int):
        self._lib = load()
        self._h = self._lib.pa_pool_create(int(num_blocks))
        if not self._h:
            raise ValueError("pa_pool_create failed")
        self.num_blocks = int(num_blocks)

    def close(self) -> None:
        if self._h:
            self._lib.pa_pool_destroy(self._h)
            self._h = None

    def __del__(self):  # pragma: no cover
        try:
            self.close()
        except Exception:
            pass

    def num_free(self) -> int:
        return int(self._lib.pa_pool_num_free(self._h))

    def ref_count(self, block: int) -> int:
        return int(self._lib.pa_pool_ref_count(self._h, int(block)))

    def allocate(self, n: int):
        buf = (ctypes.c_int32 * max(n, 1))()
        _check("pa_pool_allocate", self._lib.pa_pool_allocate(self._h, int(n), buf))
        return list(buf[:n])

    def free(self, blocks) -> None:
        arr = (ctypes.c_int32 * max(len(blocks), 1))(*blocks)
        _check("pa_pool_free", self._lib.pa_pool_free(self._h, arr, len(blocks)))

    def share(self, blocks) -> None:
        arr = (ctypes.c_int32 * max(len(blocks), 1))(*blocks)
        _check("pa_pool_share", self._lib.pa_pool_share(self._h, arr, len(blocks)))

    def copy_on_write(self, block: int):
        """(block to write into, (src, dst) copy or None)."""
        b, s, d = ctypes.c_int32(int(block)), ctypes.c_int32(-1), ctypes.c_int32(-1)
        st = self._lib.pa_pool_copy_on_write(self._h, ctypes.byref(b), ctypes.byref(s),
                                             ctypes.byref(d))
        if st < 0:
            raise PagedAttentionError("pa_pool_copy_on_write", st)
        return b.value, ((s.value, d.value) if st == 1 else None)


def copy_blocks(key_cache: torch.Tensor, value_cache: torch.Tensor, block_pairs: torch.Tensor,
                stream=None) -> None:
    """block dst := block src of both caches for every row (src, dst) of block_pairs."""
    NB, bs, Hkv, D = key_cache.shape
    n = block_pairs.shape[0] if block_pairs.numel() else 0
    st = load().pa_copy_blocks(_dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
                               _dev(block_pairs, "block_pairs") if n else None, n, NB, bs, Hkv,
                               D, key_cache.element_size(), _stream(stream))
    _check("pa_copy_blocks", st)
