"""CPU oracle for paged KV-cache attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path never does.

Thin ctypes wrappers over ``liboracle.so`` (plain C, fp64, see pa_oracle.c).
Inputs are CPU torch tensors exactly as produced by the workload generator;
bf16 tensors are passed as their raw 16-bit patterns.

Parity pins: every function here is pinned by tests/test_oracle.py against
the pages' worked examples, closed forms, invariants and library routines
(torch's scaled_dot_product_attention in fp64).  None is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_DT = {torch.float32: 0, torch.bfloat16: 1}
STATUS = {0: "ok", 1: "invalid argument", 2: "block id out of range",
          3: "slot out of range", 4: "duplicate slot or destination block", 5: "out of memory",
          6: "block both source and destination of an in-place copy"}


class OracleError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"oracle status {code}: {STATUS.get(code, '?')}")
        self.code = code


def load(path: str | None = None):
    """Load (building first if absent) the oracle library."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(p)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.oracle_gather.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i64, i32]
    lib.oracle_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i64,
                                  ctypes.c_float, i32, vp]
    lib.oracle_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                   i64, ctypes.c_float, i32]
    lib.oracle_reshape_and_cache.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i64, i32]
    lib.oracle_copy_blocks.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, i32]
    f32 = ctypes.c_float
    lib.oracle_fp8_encode.argtypes = [vp, i32, f32, vp]
    lib.oracle_fp8_decode.argtypes = [vp, i32, vp]
    lib.oracle_reshape_and_cache_fp8.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i64, i32,
                                                 f32, f32]
    lib.oracle_decode_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i64,
                                      f32, i32, f32, f32]
    lib.oracle_prefill_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                       i64, f32, i32, f32, f32]
    for f in (lib.oracle_gather, lib.oracle_decode, lib.oracle_prefill,
              lib.oracle_reshape_and_cache, lib.oracle_copy_blocks, lib.oracle_fp8_encode,
              lib.oracle_fp8_decode, lib.oracle_reshape_and_cache_fp8, lib.oracle_decode_fp8,
              lib.oracle_prefill_fp8):
        f.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _ptr(t: torch.Tensor) -> int:
    assert t.device.type == "cpu" and t.is_contiguous()
    return t.data_ptr()


def _check(code: int):
    if code:
        raise OracleError(code)


def _i32(t) -> torch.Tensor:
    return torch.as_tensor(t, dtype=torch.int32).contiguous()


def gather(cache: torch.Tensor, block_table_row, length: int, kv_head: int, lib=None) -> np.ndarray:
    """Keys (or values) of one sequence and kv head in logical order: [L, D] fp64."""
    lib = lib or load()
    NB, Hkv, B, D = cache.shape
    bt = _i32(block_table_row)
    out = np.zeros((max(length, 0), D), dtype=np.float64)
    cache = cache.contiguous()
    _check(lib.oracle_gather(out.ctypes.data, _ptr(cache), _ptr(bt), length, Hkv, kv_head, B,
                             D, NB, _DT[cache.dtype]))
    return out


def decode(query, key_cache, value_cache, block_tables, context_lens, scale: float,
           return_weights: bool = False, lib=None):
    """fp64 decode attention: out [S, Hq, D] (and weights [S, Hq, MBS*B])."""
    lib = lib or load()
    S, Hq, D = query.shape
    NB, Hkv, B, D2 = key_cache.shape
    assert D == D2 and key_cache.dtype == query.dtype == value_cache.dtype
    bt, lens = _i32(block_tables), _i32(context_lens)
    mbs = bt.shape[1] if bt.dim() == 2 else 0
    out = np.zeros((S, Hq, D), dtype=np.float64)
    w = np.zeros((S, Hq, mbs * B), dtype=np.float64) if return_weights else None
    q, kc, vc = query.contiguous(), key_cache.contiguous(), value_cache.contiguous()
    _check(lib.oracle_decode(out.ctypes.data, _ptr(q), _ptr(kc), _ptr(vc), _ptr(bt),
                             _ptr(lens), S, Hq, Hkv, D, B, mbs, NB, ctypes.c_float(scale),
                             _DT[q.dtype], w.ctypes.data if w is not None else None))
    return (out, w) if return_weights else out


def prefill(query, key_cache, value_cache, block_tables, cu_query_lens, context_lens,
            scale: float, lib=None) -> np.ndarray:
    """fp64 causal chunk attention over the paged cache: out [Tq, Hq, D]."""
    lib = lib or load()
    Tq, Hq, D = query.shape
    NB, Hkv, B, _ = key_cache.shape
    bt, cu, lens = _i32(block_tables), _i32(cu_query_lens), _i32(context_lens)
    C = lens.numel()
    out = np.zeros((Tq, Hq, D), dtype=np.float64)
    q, kc, vc = query.contiguous(), key_cache.contiguous(), value_cache.contiguous()
    _check(lib.oracle_prefill(out.ctypes.data, _ptr(q), _ptr(kc), _ptr(vc), _ptr(bt), _ptr(cu),
                              _ptr(lens), C, Hq, Hkv, D, B, bt.shape[1], NB,
                              ctypes.c_float(scale), _DT[q.dtype]))
    return out


def reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, lib=None):
    """Bitwise scatter of new K/V into copies of the pools; returns (kc, vc)."""
    lib = lib or load()
    T, Hkv, D = key.shape
    NB, Hkv2, B, D2 = key_cache.shape
    assert Hkv == Hkv2 and D == D2
    kc, vc = key_cache.clone().contiguous(), value_cache.clone().contiguous()
    k, v = key.contiguous(), value.contiguous()
    slots = torch.as_tensor(slot_mapping, dtype=torch.int64).contiguous()
    _check(lib.oracle_reshape_and_cache(_ptr(k), _ptr(v), _ptr(kc), _ptr(vc), _ptr(slots), T,
                                        Hkv, D, B, NB, key.element_size()))
    return kc, vc


def copy_blocks(src_key, src_value, dst_key, dst_value, block_mapping, lib=None):
    """Copy whole blocks src -> dst (pairs of block ids, [n, 2] int64), K and V.

    Returns new destination pools (copies of dst_* with the blocks written).
    Passing the same tensors as source and destination is the in-place case
    (copy-on-write inside one pool)."""
    lib = lib or load()
    in_place = src_key is dst_key
    assert (src_value is dst_value) == in_place
    sk, sv = src_key.contiguous(), src_value.contiguous()
    dk, dv = dst_key.clone().contiguous(), dst_value.clone().contiguous()
    assert sk.shape[1:] == dk.shape[1:] and sk.dtype == dk.dtype
    m = torch.as_tensor(block_mapping, dtype=torch.int64).reshape(-1, 2).contiguous()
    block_bytes = sk[0].numel() * sk.element_size() if sk.shape[0] else dk[0].numel() * dk.element_size()
    _check(lib.oracle_copy_blocks(_ptr(sk), _ptr(sv), _ptr(dk), _ptr(dv), _ptr(m), m.shape[0],
                                  sk.shape[0], dk.shape[0], block_bytes, int(in_place)))
    return dk, dv


def fp8_encode(x, scale=1.0, lib=None):
    """e4m3 codes (uint8 tensor) of x / scale (x: float tensor; see pa_oracle.c)."""
    lib = lib or load()
    xf = torch.as_tensor(x, dtype=torch.float32).contiguous().reshape(-1)
    codes = torch.empty(xf.numel(), dtype=torch.uint8)
    _check(lib.oracle_fp8_encode(_ptr(xf), xf.numel(), ctypes.c_float(scale), _ptr(codes)))
    return codes.reshape(torch.as_tensor(x).shape)


def fp8_decode(codes, lib=None):
    """Values (float64 numpy) of e4m3 codes."""
    lib = lib or load()
    c = torch.as_tensor(codes, dtype=torch.uint8).contiguous().reshape(-1)
    out = np.empty(c.numel(), dtype=np.float64)
    _check(lib.oracle_fp8_decode(_ptr(c), c.numel(), out.ctypes.data))
    return out.reshape(tuple(torch.as_tensor(codes).shape))


def reshape_and_cache_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale,
                          lib=None):
    """FP8 cache write into copies of the uint8 pools (K [NB, Hkv, B, D], V
    [NB, Hkv, D, B]); returns (kc, vc)."""
    lib = lib or load()
    T, Hkv, D = key.shape
    NB, Hkv2, B, D2 = key_cache.shape
    assert Hkv == Hkv2 and D == D2 and tuple(value_cache.shape) == (NB, Hkv, D, B)
    kc, vc = key_cache.clone().contiguous(), value_cache.clone().contiguous()
    k, v = key.contiguous(), value.contiguous()
    slots = torch.as_tensor(slot_mapping, dtype=torch.int64).contiguous()
    _check(lib.oracle_reshape_and_cache_fp8(_ptr(k), _ptr(v), _ptr(kc), _ptr(vc), _ptr(slots), T,
                                            Hkv, D, B, NB, _DT[k.dtype], ctypes.c_float(k_scale),
                                            ctypes.c_float(v_scale)))
    return kc, vc


def decode_fp8(query, key_cache, value_cache, block_tables, context_lens, scale, k_scale,
               v_scale, lib=None):
    """fp64 decode over FP8 pools (K [NB, Hkv, B, D], V [NB, Hkv, D, B])."""
    lib = lib or load()
    S, Hq, D = query.shape
    NB, Hkv, B, _ = key_cache.shape
    out = np.zeros((S, Hq, D), dtype=np.float64)
    q = query.contiguous()
    bt = block_tables.to(torch.int32).contiguous()
    lens = context_lens.to(torch.int32).contiguous()
    _check(lib.oracle_decode_fp8(out.ctypes.data, _ptr(q), _ptr(key_cache.contiguous()),
                                 _ptr(value_cache.contiguous()), _ptr(bt), _ptr(lens), S, Hq, Hkv,
                                 D, B, bt.shape[1], NB, ctypes.c_float(scale), _DT[q.dtype],
                                 ctypes.c_float(k_scale), ctypes.c_float(v_scale)))
    return out


def prefill_fp8(query, key_cache, value_cache, block_tables, cu_query_lens, context_lens, scale,
                k_scale, v_scale, lib=None):
    """fp64 causal prefill chunks over FP8 pools (K [NB, Hkv, B, D], V [NB, Hkv, D, B])."""
    lib = lib or load()
    T, Hq, D = query.shape
    NB, Hkv, B, _ = key_cache.shape
    out = np.zeros((T, Hq, D), dtype=np.float64)
    q = query.contiguous()
    bt = block_tables.to(torch.int32).contiguous()
    cu = cu_query_lens.to(torch.int32).contiguous()
    lens = context_lens.to(torch.int32).contiguous()
    _check(lib.oracle_prefill_fp8(out.ctypes.data, _ptr(q), _ptr(key_cache.contiguous()),
                                  _ptr(value_cache.contiguous()), _ptr(bt), _ptr(cu), _ptr(lens),
                                  lens.numel(), Hq, Hkv, D, B, bt.shape[1], NB,
                                  ctypes.c_float(scale), _DT[q.dtype], ctypes.c_float(k_scale),
                                  ctypes.c_float(v_scale)))
    return out
