"""Helpers shared by the GPU parity tests: move a case to the device, run the
library through its C ABI (via the binding), compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from paged_kv_cache_262_amd import binding

TOL = {"f32": (1e-5, 1e-5), "bf16": (1e-2, 2e-2)}   # (atol, rtol) vs the fp64 oracle


def say(*a):
    """Name the case before each GPU step (flushed), so a failure can be traced."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().cuda()


def check_close(gpu: torch.Tensor, ref: np.ndarray, dtype: str, what: str):
    atol, rtol = TOL[dtype]
    g = gpu.float().cpu().double().numpy()
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} elements out of tolerance; max abs "
                             f"{err.max():.3e}; first {idx.tolist()} gpu "
                             f"{g[tuple(idx[0])]:.6f} ref {ref[tuple(idx[0])]:.6f}")
    return float(err.max())


def apply_cache_write_gpu(case, kc, vc):
    if case.slot_mapping.numel():
        binding.reshape_and_cache(dev(case.new_key), dev(case.new_value), kc, vc,
                                  dev(case.slot_mapping))


def oracle_pools(case):
    if case.slot_mapping.numel():
        return oracle.reshape_and_cache(case.new_key, case.new_value, case.key_cache,
                                        case.value_cache, case.slot_mapping)
    return case.key_cache, case.value_cache


def gpu_decode(case, kc, vc, partition_size=0, query=None, block_tables=None,
               context_lens=None, max_context_len=None):
    q = dev(case.query if query is None else query)
    bt = dev(case.block_tables if block_tables is None else block_tables)
    lens = case.context_lens if context_lens is None else context_lens
    maxL = int(lens.max()) if max_context_len is None else max_context_len
    out = torch.empty_like(q)
    binding.decode(out, q, kc, vc, bt, dev(lens), case.scale, maxL,
                   partition_size=partition_size)
    return out


def oracle_decode(case, kc, vc, query=None, block_tables=None, context_lens=None):
    return oracle.decode(case.query if query is None else query, kc, vc,
                         case.block_tables if block_tables is None else block_tables,
                         case.context_lens if context_lens is None else context_lens,
                         case.scale)
