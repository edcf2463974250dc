"""ctypes binding of libpa.so (declared in include/pa.h).

Argument marshalling only: torch tensors become device pointers, shapes become
ints, and work goes on the caller's current HIP stream.  Every computation
happens in the library's kernels.  If the library is not built, or a tensor is
not on the GPU, the call raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libpa.so"
_lib = None

(PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP,
 PA_ERR_POOL_EXHAUSTED) = range(6)
PA_F32, PA_BF16 = 0, 1
_DTYPE = {torch.float32: PA_F32, torch.bfloat16: PA_BF16}

# Every symbol include/pa.h declares, with its ctypes signature.
_vp, _i32, _i64, _sz, _f = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                            ctypes.c_float)
SIGNATURES = {
    "pa_abi_version": (_i32, []),
    "pa_status_string": (ctypes.c_char_p, [_i32]),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_reshape_and_cache": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, _i32,
                                    _vp]),
    "pa_decode_auto_partition_size": (_i32, [_i32, _i32, _i32, _i32]),
    "pa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode_needs_reduce": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i64,
                         _i32, _i32, _f, _i32, _vp, _sz, _vp]),
    "pa_decode_no_alloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                  _i32, _i64, _i32, _i32, _f, _i32, _vp]),
    "pa_decode_no_alloc_max_workspace": (_sz, []),
    "pa_decode_partitions": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                    _i32, _i64, _i32, _i32, _f, _i32, _vp, _sz, _vp]),
    "pa_decode_reduce": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                _vp, _sz, _vp]),
    "pa_decode_append": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                _i32, _i32, _i64, _i32, _i32, _f, _i32, _vp, _sz, _vp]),
    "pa_decode_append_partitions": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                           _i32, _i32, _i32, _i32, _i64, _i32, _i32, _f, _i32,
                                           _vp, _sz, _vp]),
    "pa_prefill_chunk": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                _i32, _i32, _i64, _f, _i32, _vp]),
    "pa_copy_blocks": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _vp]),
    "pa_prefill_chunk_append": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                       _i32, _i32, _i32, _i32, _i32, _i64, _f, _i32, _vp]),
    "pa_decode_shared_prefix": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                       _i32, _i32, _i64, _i32, _i32, _f, _vp, _sz, _vp]),
    "pa_decode_shared_prefix_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_probe_sink_words": (_i64, []),
    "pa_probe_stream_read": (_i32, [_vp, _i64, _vp, _vp]),
    "pa_probe_mfma_bf16": (_i32, [_vp, _i32, ctypes.POINTER(ctypes.c_double), _vp]),
    "pa_reshape_and_cache_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64,
                                        _i32, _f, _f, _vp]),
    "pa_decode_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                             _i64, _i32, _f, _f, _f, _vp, _sz, _vp]),
    "pa_decode_fp8_append": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                    _i32, _i32, _i32, _i64, _i32, _f, _f, _f, _vp, _sz, _vp]),
    "pa_decode_fp8_append_partitions": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                               _i32, _i32, _i32, _i32, _i32, _i64, _i32, _f, _f,
                                               _f, _vp, _sz, _vp]),
    "pa_prefill_chunk_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                    _i32, _i32, _i32, _i64, _f, _f, _f, _vp]),
    "pa_decode_fp8_partitions": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                        _i32, _i32, _i64, _i32, _f, _f, _f, _vp, _sz, _vp]),
    "pa_decode_fp8_shared_prefix": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                           _i32, _i32, _i64, _i32, _i32, _f, _f, _f, _vp, _sz,
                                           _vp]),
    "pa_bm_create": (_i32, [_i64, _i32, _i32, _vp]),
    "pa_bm_destroy": (None, [_vp]),
    "pa_bm_add_sequence": (_i32, [_vp, _i64, _vp, _i32, _vp, _vp]),
    "pa_bm_append": (_i32, [_vp, _i64, _i32, _vp]),
    "pa_bm_fork": (_i32, [_vp, _i64, _i64]),
    "pa_bm_free": (_i32, [_vp, _i64]),
    "pa_bm_take_copies": (_i32, [_vp, _vp, _i32]),
    "pa_bm_block_table": (_i32, [_vp, _i64, _vp, _i32, _vp, _vp]),
    "pa_bm_get_stats": (_i32, [_vp, _vp]),
    "pa_bm_append_batch": (_i32, [_vp, _vp, _vp, _i32, _vp]),
    "pa_bm_block_tables": (_i32, [_vp, _vp, _i32, _vp, _i32, _i32, _vp]),
}


class PAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_status_name(status)}: {detail}")
        self.status = status


def library_path() -> str:
    return os.environ.get("PA_LIBRARY", os.path.join(_HERE, _LIB_NAME))


def load():
    """Load libpa.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -m "
                           f"paged_kv_cache_262_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _status_name(status: int) -> str:
    try:
        return load().pa_status_string(status).decode()
    except Exception:
        return f"status {status}"


def _check(status: int):
    if status != PA_OK:
        detail = load().pa_last_error().decode()
        if status in (PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE):
            raise PAError(status, detail)
        raise PAError(status, detail)


def _dev(t: Optional[torch.Tensor], name: str) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPE:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return _DTYPE[t.dtype]


def reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, stream=None):
    """Scatter new K/V [T, Hkv, D] into the pools [NB, Hkv, B, D] at slot_mapping."""
    T, Hkv, D = key.shape
    NB, _, B, _ = key_cache.shape
    if slot_mapping.dtype != torch.int64:
        raise ValueError("slot_mapping must be int64")
    _check(load().pa_reshape_and_cache(
        _dev(key, "key"), _dev(value, "value"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(slot_mapping, "slot_mapping"), T, Hkv, D, B, NB,
        _dtype(key), _stream(stream)))


def decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                           max_context_len, partition_size=0) -> int:
    return int(load().pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                block_size, max_context_len, partition_size))


def decode_needs_reduce(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                        max_context_len, partition_size=0) -> bool:
    """Whether pa_decode_reduce launches work for these sizes (False: the first
    phase finishes every row, one wave per (sequence, kv head) pair)."""
    return bool(load().pa_decode_needs_reduce(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                              block_size, max_context_len, partition_size))


def auto_partition_size(num_seqs, num_kv_heads, max_context_len, block_size) -> int:
    return int(load().pa_decode_auto_partition_size(num_seqs, num_kv_heads, max_context_len,
                                                    block_size))


def _decode_args(out, query, key_cache, value_cache, block_tables, context_lens,
                 max_context_len, partition_size, scale, workspace):
    S, Hq, D = query.shape
    NB, Hkv, B, _ = key_cache.shape
    mbs = block_tables.shape[1]
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    return (_dev(out, "out"), _dev(query, "query"), _dev(key_cache, "key_cache"),
            _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables"),
            _dev(context_lens, "context_lens"), S, Hq, Hkv, D, B, mbs, NB, int(max_context_len),
            int(partition_size), float(scale), _dtype(query), _dev(workspace, "workspace"),
            0 if workspace is None else workspace.numel() * workspace.element_size())


def make_workspace(query, key_cache, max_context_len, partition_size=0):
    S, Hq, D = query.shape
    _, Hkv, B, _ = key_cache.shape
    n = decode_workspace_bytes(S, Hq, Hkv, D, B, max_context_len, partition_size)
    return torch.empty(n, dtype=torch.uint8, device=query.device)


def decode(out, query, key_cache, value_cache, block_tables, context_lens, scale,
           max_context_len, partition_size=0, workspace=None, stream=None):
    """One query per sequence against the paged cache; writes ``out`` [S, Hq, D]."""
    if workspace is None:
        workspace = make_workspace(query, key_cache, max_context_len, partition_size)
    _check(load().pa_decode(*_decode_args(out, query, key_cache, value_cache, block_tables,
                                          context_lens, max_context_len, partition_size, scale,
                                          workspace), _stream(stream)))
    return out


def decode_no_alloc(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                    max_context_len, partition_size=0, stream=None):
    """pa_decode with the library's static per-GPU workspace (no allocation)."""
    args = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens,
                        max_context_len, partition_size, scale, None)[:-2]
    _check(load().pa_decode_no_alloc(*args, _stream(stream)))
    return out


def shared_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                  max_context_len, prefix_blocks) -> int:
    return int(load().pa_decode_shared_prefix_workspace_bytes(
        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len,
        prefix_blocks))


def make_shared_prefix_workspace(query, key_cache, max_context_len, prefix_blocks):
    S, Hq, D = query.shape
    _, Hkv, B, _ = key_cache.shape
    n = shared_prefix_workspace_bytes(S, Hq, Hkv, D, B, max_context_len, prefix_blocks)
    return torch.empty(n, dtype=torch.uint8, device=query.device)


def decode_shared_prefix(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                         max_context_len, prefix_blocks, workspace=None, stream=None):
    """Decode (bf16) for a batch whose block-table rows all start with the
    same prefix_blocks physical blocks; writes ``out`` [S, Hq, D]."""
    if workspace is None:
        workspace = make_shared_prefix_workspace(query, key_cache, max_context_len,
                                                 prefix_blocks)
    a = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens,
                     max_context_len, 0, scale, workspace)
    if a[16] != PA_BF16:
        raise PAError(PA_ERR_UNSUPPORTED, "pa_decode_shared_prefix takes bf16 pools (FP8 pools: "
                                          "decode_fp8_shared_prefix)")
    _check(load().pa_decode_shared_prefix(*a[:14], int(prefix_blocks), a[15], a[17], a[18],
                                          _stream(stream)))
    return out


def decode_no_alloc_max_workspace() -> int:
    return int(load().pa_decode_no_alloc_max_workspace())


def decode_partitions(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                      max_context_len, partition_size, workspace, stream=None):
    _check(load().pa_decode_partitions(*_decode_args(out, query, key_cache, value_cache,
                                                     block_tables, context_lens, max_context_len,
                                                     partition_size, scale, workspace),
                                       _stream(stream)))


def decode_reduce(out, context_lens, num_kv_heads, block_size, max_blocks_per_seq,
                  max_context_len, partition_size, workspace, stream=None):
    S, Hq, D = out.shape
    _check(load().pa_decode_reduce(
        _dev(out, "out"), _dev(context_lens, "context_lens"), S, Hq, num_kv_heads, D, block_size,
        max_blocks_per_seq, int(max_context_len), int(partition_size), _dtype(out),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def _append_args(out, query, new_key, new_value, key_cache, value_cache, block_tables,
                 context_lens, max_context_len, partition_size, scale, workspace):
    d = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens,
                     max_context_len, partition_size, scale, workspace)
    S, Hkv, D = query.shape[0], key_cache.shape[1], query.shape[2]
    for t, name in ((new_key, "new_key"), (new_value, "new_value")):
        if tuple(t.shape) != (S, Hkv, D) or t.dtype != query.dtype:
            raise ValueError(f"{name} must be [{S}, {Hkv}, {D}] {query.dtype}")
    return d[:2] + (_dev(new_key, "new_key"), _dev(new_value, "new_value")) + d[2:]


def decode_append(out, query, new_key, new_value, key_cache, value_cache, block_tables,
                  context_lens, scale, max_context_len, partition_size=0, workspace=None,
                  stream=None):
    """One decode step with its new tokens: writes new_key/new_value [S, Hkv, D] at
    position context_lens[s] - 1 of each sequence and attends over it; writes ``out``."""
    if workspace is None:
        workspace = make_workspace(query, key_cache, max_context_len, partition_size)
    _check(load().pa_decode_append(*_append_args(out, query, new_key, new_value, key_cache,
                                                 value_cache, block_tables, context_lens,
                                                 max_context_len, partition_size, scale,
                                                 workspace), _stream(stream)))
    return out


def decode_append_partitions(out, query, new_key, new_value, key_cache, value_cache,
                             block_tables, context_lens, scale, max_context_len, partition_size,
                             workspace, stream=None):
    _check(load().pa_decode_append_partitions(
        *_append_args(out, query, new_key, new_value, key_cache, value_cache, block_tables,
                      context_lens, max_context_len, partition_size, scale, workspace),
        _stream(stream)))


def _fp8_pools(key_cache, value_cache):
    """Shape of FP8 pools: K uint8 [NB, Hkv, B, D], V uint8 [NB, Hkv, D, B]."""
    if key_cache.dtype != torch.uint8 or value_cache.dtype != torch.uint8:
        raise ValueError("FP8 pools hold uint8 e4m3 codes")
    NB, Hkv, B, D = key_cache.shape
    if tuple(value_cache.shape) != (NB, Hkv, D, B):
        raise ValueError(f"value_cache must be [{NB}, {Hkv}, {D}, {B}] (pages transposed)")
    return NB, Hkv, B, D


def reshape_and_cache_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale,
                          stream=None):
    """Quantising cache write: e4m3 codes of key / k_scale and value / v_scale at the slots."""
    T, Hkv, D = key.shape
    NB, _, B, _ = _fp8_pools(key_cache, value_cache)
    if slot_mapping.dtype != torch.int64:
        raise ValueError("slot_mapping must be int64")
    _check(load().pa_reshape_and_cache_fp8(
        _dev(key, "key"), _dev(value, "value"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(slot_mapping, "slot_mapping"), T, Hkv, D, B, NB,
        _dtype(key), float(k_scale), float(v_scale), _stream(stream)))


def _fp8_decode_args(out, query, key_cache, value_cache, block_tables, context_lens,
                     max_context_len, scale, k_scale, v_scale, workspace):
    S, Hq, D = query.shape
    NB, Hkv, B, _ = _fp8_pools(key_cache, value_cache)
    if query.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise ValueError("FP8 decode takes a bf16 query and writes a bf16 output")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    return (_dev(out, "out"), _dev(query, "query"), _dev(key_cache, "key_cache"),
            _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables"),
            _dev(context_lens, "context_lens"), S, Hq, Hkv, D, B, block_tables.shape[1], NB,
            int(max_context_len), float(scale), float(k_scale), float(v_scale),
            _dev(workspace, "workspace"), workspace.numel() * workspace.element_size())


def _fp8_append_args(out, query, new_key, new_value, key_cache, value_cache, block_tables,
                     context_lens, max_context_len, scale, k_scale, v_scale, workspace):
    d = _fp8_decode_args(out, query, key_cache, value_cache, block_tables, context_lens,
                         max_context_len, scale, k_scale, v_scale, workspace)
    S, Hkv, D = query.shape[0], key_cache.shape[1], query.shape[2]
    for t, name in ((new_key, "new_key"), (new_value, "new_value")):
        if tuple(t.shape) != (S, Hkv, D) or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be [{S}, {Hkv}, {D}] bfloat16")
    return d[:2] + (_dev(new_key, "new_key"), _dev(new_value, "new_value")) + d[2:]


def decode_fp8_append(out, query, new_key, new_value, key_cache, value_cache, block_tables,
                      context_lens, scale, max_context_len, k_scale, v_scale, workspace=None,
                      stream=None):
    """One FP8 decode step with its new tokens: quantises new_key/new_value [S, Hkv, D] into
    position context_lens[s] - 1 of each sequence and attends over it; writes ``out``."""
    if workspace is None:
        workspace = make_fp8_workspace(query, key_cache, max_context_len)
    _check(load().pa_decode_fp8_append(*_fp8_append_args(
        out, query, new_key, new_value, key_cache, value_cache, block_tables, context_lens,
        max_context_len, scale, k_scale, v_scale, workspace), _stream(stream)))
    return out


def decode_fp8_append_partitions(out, query, new_key, new_value, key_cache, value_cache,
                                 block_tables, context_lens, scale, max_context_len, k_scale,
                                 v_scale, workspace, stream=None):
    _check(load().pa_decode_fp8_append_partitions(*_fp8_append_args(
        out, query, new_key, new_value, key_cache, value_cache, block_tables, context_lens,
        max_context_len, scale, k_scale, v_scale, workspace), _stream(stream)))


def make_fp8_workspace(query, key_cache, max_context_len):
    S, Hq, D = query.shape
    Hkv, B = key_cache.shape[1], key_cache.shape[2]
    n = decode_workspace_bytes(S, Hq, Hkv, D, B, max_context_len, 0)
    return torch.empty(n, dtype=torch.uint8, device=query.device)


def decode_fp8(out, query, key_cache, value_cache, block_tables, context_lens, scale,
               max_context_len, k_scale, v_scale, workspace=None, stream=None):
    """Decode over FP8 pools (see reshape_and_cache_fp8); writes bf16 ``out`` [S, Hq, D]."""
    if workspace is None:
        workspace = make_fp8_workspace(query, key_cache, max_context_len)
    _check(load().pa_decode_fp8(*_fp8_decode_args(out, query, key_cache, value_cache,
                                                  block_tables, context_lens, max_context_len,
                                                  scale, k_scale, v_scale, workspace),
                                _stream(stream)))
    return out


def decode_fp8_shared_prefix(out, query, key_cache, value_cache, block_tables, context_lens,
                             scale, max_context_len, prefix_blocks, k_scale, v_scale,
                             workspace=None, stream=None):
    """decode_shared_prefix over FP8 pools; writes bf16 ``out`` [S, Hq, D]."""
    if workspace is None:
        workspace = make_shared_prefix_workspace(query, key_cache, max_context_len,
                                                 prefix_blocks)
    a = _fp8_decode_args(out, query, key_cache, value_cache, block_tables, context_lens,
                         max_context_len, scale, k_scale, v_scale, workspace)
    _check(load().pa_decode_fp8_shared_prefix(*a[:14], int(prefix_blocks), *a[14:],
                                              _stream(stream)))
    return out


def decode_fp8_partitions(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                          max_context_len, k_scale, v_scale, workspace, stream=None):
    _check(load().pa_decode_fp8_partitions(*_fp8_decode_args(
        out, query, key_cache, value_cache, block_tables, context_lens, max_context_len, scale,
        k_scale, v_scale, workspace), _stream(stream)))


def prefill_chunk_fp8(out, query, key_cache, value_cache, block_tables, cu_query_lens,
                      context_lens, scale, max_query_len, k_scale, v_scale, stream=None):
    """Causal chunks [Tq, Hq, D] (bf16) against FP8 pools; writes bf16 ``out``."""
    Tq, Hq, D = query.shape
    NB, Hkv, B, _ = _fp8_pools(key_cache, value_cache)
    if query.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise ValueError("FP8 prefill takes a bf16 query and writes a bf16 output")
    C = context_lens.numel()
    _check(load().pa_prefill_chunk_fp8(
        _dev(out, "out"), _dev(query, "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables"),
        _dev(cu_query_lens, "cu_query_lens"), _dev(context_lens, "context_lens"), C,
        int(max_query_len), Hq, Hkv, D, B, block_tables.shape[1], NB, float(scale),
        float(k_scale), float(v_scale), _stream(stream)))
    return out


def prefill_chunk(out, query, key_cache, value_cache, block_tables, cu_query_lens,
                  context_lens, scale, max_query_len, stream=None):
    """Causal chunks [Tq, Hq, D] against the paged cache; writes ``out``."""
    Tq, Hq, D = query.shape
    NB, Hkv, B, _ = key_cache.shape
    C = context_lens.numel()
    _check(load().pa_prefill_chunk(
        _dev(out, "out"), _dev(query, "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables"),
        _dev(cu_query_lens, "cu_query_lens"), _dev(context_lens, "context_lens"), C,
        int(max_query_len), Hq, Hkv, D, B, block_tables.shape[1], NB, float(scale),
        _dtype(query), _stream(stream)))
    return out


def prefill_chunk_append(out, query, new_key, new_value, key_cache, value_cache, block_tables,
                         cu_query_lens, context_lens, scale, max_query_len, stream=None):
    """prefill_chunk that first places the chunks' own K/V rows (new_key,
    new_value [Tq, Hkv, D]) into their slots, inside the same pass."""
    Tq, Hq, D = query.shape
    NB, Hkv, B, _ = key_cache.shape
    C = context_lens.numel()
    if tuple(new_key.shape) != (Tq, Hkv, D) or tuple(new_value.shape) != (Tq, Hkv, D):
        raise ValueError("new_key / new_value must be [Tq, Hkv, D]")
    _check(load().pa_prefill_chunk_append(
        _dev(out, "out"), _dev(query, "query"), _dev(new_key, "new_key"),
        _dev(new_value, "new_value"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables"),
        _dev(cu_query_lens, "cu_query_lens"), _dev(context_lens, "context_lens"), C,
        int(max_query_len), Hq, Hkv, D, B, block_tables.shape[1], NB, float(scale),
        _dtype(query), _stream(stream)))
    return out


def copy_blocks(src_key_cache, src_value_cache, dst_key_cache, dst_value_cache, block_mapping,
                stream=None):
    """Copy whole blocks between pools: block_mapping [n, 2] int64 (source id,
    destination id).  Pools are [NB, Hkv, B, D] tensors on the GPU or in pinned
    host memory (pin_memory=True); the mapping likewise."""
    for t, name in ((src_key_cache, "src_key_cache"), (src_value_cache, "src_value_cache"),
                    (dst_key_cache, "dst_key_cache"), (dst_value_cache, "dst_value_cache"),
                    (block_mapping, "block_mapping")):
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError(f"{name} must be a GPU tensor or pinned host memory")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if block_mapping.dtype != torch.int64 or block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be int64 [n, 2]")
    if src_key_cache.shape[1:] != dst_key_cache.shape[1:] or src_key_cache.dtype != dst_key_cache.dtype:
        raise ValueError("source and destination pools differ in block shape or dtype")
    block_bytes = src_key_cache[0].numel() * src_key_cache.element_size()
    _check(load().pa_copy_blocks(
        src_key_cache.data_ptr(), src_value_cache.data_ptr(), dst_key_cache.data_ptr(),
        dst_value_cache.data_ptr(), block_mapping.data_ptr(), block_mapping.shape[0],
        src_key_cache.shape[0], dst_key_cache.shape[0], block_bytes, _stream(stream)))


def probe_sink(device=None) -> torch.Tensor:
    """A device buffer large enough for either probe's sink."""
    return torch.empty(int(load().pa_probe_sink_words()), dtype=torch.int32,
                       device=device or "cuda")


def probe_stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None):
    """Read every byte of buf once (a streaming-read ceiling); buf is a
    contiguous device tensor whose size is a multiple of 16 bytes."""
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    if sink.numel() * sink.element_size() < 4 * int(load().pa_probe_sink_words()):
        raise ValueError("sink is too small")
    _check(load().pa_probe_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                       sink.data_ptr(), _stream(stream)))


def probe_mfma_bf16(sink: torch.Tensor, iters: int, stream=None) -> float:
    """Launch the bf16 matrix-core probe; returns the flops it performs."""
    if sink.numel() * sink.element_size() < 4 * int(load().pa_probe_sink_words()):
        raise ValueError("sink is too small")
    flops = ctypes.c_double(0.0)
    _check(load().pa_probe_mfma_bf16(sink.data_ptr(), int(iters), ctypes.byref(flops),
                                     _stream(stream)))
    return flops.value


class _BmStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "num_blocks", "free_blocks", "used_blocks", "shared_blocks", "cached_blocks", "num_seqs",
        "seq_tokens", "seq_slots", "prefix_hits")]


class BlockManager:
    """The library's host block manager (pa_bm_* in include/pa.h): block tables,
    slot mappings, reference counts, copy-on-write pairs and the prefix cache."""

    def __init__(self, num_blocks: int, block_size: int, prefix_cache: bool = False):
        self._lib = load()
        h = ctypes.c_void_p()
        _check(self._lib.pa_bm_create(num_blocks, block_size, int(prefix_cache), ctypes.byref(h)))
        self._h = h
        self.block_size = block_size

    def close(self):
        if self._h:
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_sequence(self, seq_id: int, tokens):
        """Registers a sequence with its prompt; returns (slots, cached_tokens):
        slots[t] is the slot of prompt token t, or -1 if its block was reused."""
        toks = (ctypes.c_int32 * max(1, len(tokens)))(*tokens)
        slots = (ctypes.c_int64 * max(1, len(tokens)))()
        cached = ctypes.c_int32()
        _check(self._lib.pa_bm_add_sequence(self._h, seq_id, toks, len(tokens), slots,
                                            ctypes.byref(cached)))
        return list(slots)[:len(tokens)], cached.value

    def append(self, seq_id: int, token: int) -> int:
        slot = ctypes.c_int64()
        _check(self._lib.pa_bm_append(self._h, seq_id, token, ctypes.byref(slot)))
        return slot.value

    def fork(self, parent: int, child: int):
        _check(self._lib.pa_bm_fork(self._h, parent, child))

    def free(self, seq_id: int):
        _check(self._lib.pa_bm_free(self._h, seq_id))

    def take_copies(self):
        n = self._lib.pa_bm_take_copies(self._h, None, 0)
        if n <= 0:
            return []
        buf = (ctypes.c_int64 * (2 * n))()
        got = self._lib.pa_bm_take_copies(self._h, buf, n)
        assert got == n
        return [(buf[2 * i], buf[2 * i + 1]) for i in range(n)]

    def block_table(self, seq_id: int):
        nb, L = ctypes.c_int32(), ctypes.c_int32()
        _check(self._lib.pa_bm_block_table(self._h, seq_id, None, 0, ctypes.byref(nb),
                                           ctypes.byref(L)))
        row = (ctypes.c_int32 * max(1, nb.value))()
        _check(self._lib.pa_bm_block_table(self._h, seq_id, row, nb.value, None, None))
        return list(row)[:nb.value], L.value

    def append_batch(self, seq_ids, tokens) -> torch.Tensor:
        """One step: tokens[i] appended to seq_ids[i]; returns the int64 slots."""
        ids = torch.as_tensor(seq_ids, dtype=torch.int64).contiguous()
        tok = torch.as_tensor(tokens, dtype=torch.int32).contiguous()
        slots = torch.empty(ids.numel(), dtype=torch.int64)
        _check(self._lib.pa_bm_append_batch(self._h, ids.data_ptr(), tok.data_ptr(), ids.numel(),
                                            slots.data_ptr()))
        return slots

    def block_tables(self, seq_ids, max_blocks: int, fill: int = 0):
        """(int32 [n, max_blocks] tables padded with fill, int32 [n] lengths)."""
        ids = torch.as_tensor(seq_ids, dtype=torch.int64).contiguous()
        tables = torch.empty((ids.numel(), max_blocks), dtype=torch.int32)
        lens = torch.empty(ids.numel(), dtype=torch.int32)
        _check(self._lib.pa_bm_block_tables(self._h, ids.data_ptr(), ids.numel(),
                                            tables.data_ptr(), max_blocks, fill, lens.data_ptr()))
        return tables, lens

    def stats(self) -> dict:
        st = _BmStats()
        _check(self._lib.pa_bm_get_stats(self._h, ctypes.byref(st)))
        return {n: getattr(st, n) for n, _ in _BmStats._fields_}
