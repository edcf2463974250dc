"""Seeded synthetic inputs for paged KV-cache attention.

This module only draws random numbers and lays out block tables the way a
block manager would: a pool of fixed-size physical blocks is handed out in
the order of a seeded random permutation, so that logically consecutive
blocks of a sequence land on scattered physical blocks ("vLLM High-Performance
Inference Engine: PagedAttention Principles and Deployment Guide", section
"PagedAttention Architecture Deep Dive"; "vLLM Guide: High-Throughput
Multi-GPU LLM Serving with PagedAttention", section "What Is PagedAttention?").
It holds none of the attention arithmetic, and it is the only code shared by
the CPU oracle and the GPU path: both consume exactly these tensors.

Everything is generated on the CPU with ``torch.Generator`` so that a case is
bit-identical wherever it is built.  Draw order per case: context lengths ->
block permutation -> queries -> key pool -> value pool -> new keys -> new
values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclasses.dataclass
class PagedCase:
    """One synthetic batch: a block pool, per-sequence block tables and queries.

    Layouts (all row-major, contiguous, CPU tensors):
      key_cache, value_cache : [num_blocks, num_kv_heads, block_size, head_dim]
      block_tables           : int32 [num_seqs, max_blocks_per_seq]
      context_lens           : int32 [num_seqs]   (tokens, incl. the new one)
      query                  : [num_seqs, num_q_heads, head_dim]   (decode)
      new_key, new_value     : [num_new, num_kv_heads, head_dim]
      slot_mapping           : int64 [num_new]   slot = block * block_size + offset
    Prefill chunks (optional):
      chunk_query            : [sum n_c, num_q_heads, head_dim]
      chunk_cu_query_lens    : int32 [C + 1]
      chunk_context_lens     : int32 [C]   (keys incl. the chunk's own tokens)
      chunk_block_tables     : int32 [C, chunk_max_blocks]
    """

    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    key_cache: torch.Tensor
    value_cache: torch.Tensor
    block_tables: torch.Tensor
    context_lens: torch.Tensor
    query: torch.Tensor
    new_key: torch.Tensor
    new_value: torch.Tensor
    slot_mapping: torch.Tensor
    chunk_query: Optional[torch.Tensor] = None
    chunk_cu_query_lens: Optional[torch.Tensor] = None
    chunk_context_lens: Optional[torch.Tensor] = None
    chunk_block_tables: Optional[torch.Tensor] = None
    # physical block ids owned by more than one table (shared prefix)
    shared_blocks: Optional[torch.Tensor] = None

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.numel())

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max().item()) if self.num_seqs else 0

    @property
    def num_chunks(self) -> int:
        return 0 if self.chunk_context_lens is None else int(self.chunk_context_lens.numel())


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def _normal(gen: torch.Generator, shape, dtype: str) -> torch.Tensor:
    # drawn in fp32 and rounded to the storage type (round-to-nearest-even)
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(DTYPES[dtype])


def _assign_blocks(perm: np.ndarray, cursor: int, n: int):
    ids = perm[cursor:cursor + n]
    assert len(ids) == n, "pool too small"
    return ids, cursor + n


def _table(rows: List[np.ndarray], width: int, fill: int = 0) -> torch.Tensor:
    t = np.full((len(rows), width), fill, dtype=np.int32)
    for i, r in enumerate(rows):
        t[i, : len(r)] = r
    return torch.from_numpy(t)


def _slot_of_position(blocks: np.ndarray, pos: int, block_size: int) -> int:
    """Slot of logical position ``pos`` of a sequence owning ``blocks``: the
    block manager's own bookkeeping of where it put that token."""
    return int(blocks[pos // block_size]) * block_size + pos % block_size


def make_case(
    name: str,
    seed: int,
    dtype: str,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    block_size: int,
    context_lens: List[int],
    new_positions: Optional[List[int]] = None,
    extra_blocks: int = 0,
    shared_prefix_tokens: int = 0,
    chunks: Optional[List[tuple]] = None,
    lens_drawn: Optional[torch.Tensor] = None,
    gen: Optional[torch.Generator] = None,
    scale: Optional[float] = None,
) -> PagedCase:
    """General builder.

    context_lens        : per decode sequence, tokens in the cache incl. new one
    new_positions       : per decode sequence, the logical position written by
                          the cache write (normally L-1), or None for no write
    shared_prefix_tokens: a prefix (multiple of block_size) whose physical blocks
                          appear in every decode table
    chunks              : list of (num_query_tokens, context_len) prefill chunks;
                          the chunk's own positions [L-n, L) are written too
    extra_blocks        : unused physical blocks added to the pool
    """
    if gen is None:
        gen = torch.Generator().manual_seed(seed)
    chunks = chunks or []
    B = block_size
    assert shared_prefix_tokens % B == 0
    n_prefix = shared_prefix_tokens // B
    own_blocks = [_cdiv(L, B) - n_prefix for L in context_lens]
    assert all(n >= 0 for n in own_blocks)
    chunk_blocks = [_cdiv(L, B) for (_, L) in chunks]
    num_blocks = n_prefix + sum(own_blocks) + sum(chunk_blocks) + extra_blocks
    perm = torch.randperm(num_blocks, generator=gen).numpy().astype(np.int64)

    cursor = 0
    prefix_ids, cursor = _assign_blocks(perm, cursor, n_prefix)
    seq_blocks = []
    for n in own_blocks:
        ids, cursor = _assign_blocks(perm, cursor, n)
        seq_blocks.append(np.concatenate([prefix_ids, ids]))
    chunk_ids = []
    for n in chunk_blocks:
        ids, cursor = _assign_blocks(perm, cursor, n)
        chunk_ids.append(ids)

    S = len(context_lens)
    mbs = max([len(b) for b in seq_blocks] + [1])
    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    query = _normal(gen, (S, Hq, D), dtype)
    key_cache = _normal(gen, (num_blocks, Hkv, B, D), dtype)
    value_cache = _normal(gen, (num_blocks, Hkv, B, D), dtype)

    slots = []
    if new_positions is not None:
        for s, pos in enumerate(new_positions):
            if pos is not None:
                slots.append(_slot_of_position(seq_blocks[s], pos, B))
    for c, (n, L) in enumerate(chunks):
        for pos in range(L - n, L):
            slots.append(_slot_of_position(chunk_ids[c], pos, B))
    T = len(slots)
    new_key = _normal(gen, (T, Hkv, D), dtype)
    new_value = _normal(gen, (T, Hkv, D), dtype)

    chunk_kw = {}
    if chunks:
        nq = sum(n for n, _ in chunks)
        cu = np.zeros(len(chunks) + 1, dtype=np.int32)
        cu[1:] = np.cumsum([n for n, _ in chunks])
        chunk_kw = dict(
            chunk_query=_normal(gen, (nq, Hq, D), dtype),
            chunk_cu_query_lens=torch.from_numpy(cu),
            chunk_context_lens=torch.tensor([L for _, L in chunks], dtype=torch.int32),
            chunk_block_tables=_table(chunk_ids, max(chunk_blocks)),
        )
    return PagedCase(
        name=name,
        dtype=dtype,
        num_q_heads=Hq,
        num_kv_heads=Hkv,
        head_dim=D,
        block_size=B,
        num_blocks=num_blocks,
        scale=float(scale if scale is not None else 1.0 / math.sqrt(D)),
        key_cache=key_cache,
        value_cache=value_cache,
        block_tables=_table(seq_blocks, mbs),
        context_lens=torch.tensor(context_lens, dtype=torch.int32),
        query=query,
        new_key=new_key,
        new_value=new_value,
        slot_mapping=torch.tensor(slots, dtype=torch.int64),
        shared_blocks=torch.from_numpy(prefix_ids.astype(np.int32)) if n_prefix else None,
        **chunk_kw,
    )


def _uniform_lens(gen: torch.Generator, n: int, lo: int, hi: int) -> List[int]:
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=gen)]


# --------------------------------------------------------------------------
# The five named workloads.  Sizes follow the pages' scenarios: an 8B-class
# GQA model, 32K-token contexts of a 70B model with 8 KV heads, prompts that
# share a system prefix, and 512-token prefill chunks riding on decode steps.
# --------------------------------------------------------------------------

def tiny_decode(seed: int = 1) -> PagedCase:
    """4 seqs, 4 q = 4 kv heads, d 64, fp32, B 16, lens {1,17,33,100}, 64-block pool."""
    lens = [1, 17, 33, 100]
    used = sum(_cdiv(L, 16) for L in lens)
    return make_case("tiny_decode", seed, "f32", 4, 4, 64, 16, lens,
                     extra_blocks=64 - used, scale=1.0 / 8.0)


def llama8b_decode(seed: int = 2, num_seqs: int = 64) -> PagedCase:
    """Llama-3-8B-shaped layer: 64 seqs, 32 q / 8 kv heads, d 128, bf16, B 16,
    L ~ U{512..4096}, exact-fit pool, one new token per sequence at L-1."""
    gen = torch.Generator().manual_seed(seed)
    lens = _uniform_lens(gen, num_seqs, 512, 4096)
    return make_case("llama8b_decode", seed, "bf16", 32, 8, 128, 16, lens,
                     new_positions=[L - 1 for L in lens], gen=gen)


def long_context_decode(seed: int = 3, num_seqs: int = 8, context_len: int = 32768) -> PagedCase:
    """70B-shaped long context: 8 seqs x 32768 tokens, 64 q / 8 kv heads, d 128,
    bf16, B 32, the whole pool randomly permuted."""
    lens = [context_len] * num_seqs
    return make_case("long_context_decode", seed, "bf16", 64, 8, 128, 32, lens)


def prefix_sharing_decode(seed: int = 4, num_seqs: int = 128) -> PagedCase:
    """128 seqs sharing a 1024-token prefix (64 physical blocks, ref count 128)
    followed by per-sequence suffixes U ~ U{256..2048} on fresh blocks."""
    gen = torch.Generator().manual_seed(seed)
    suffix = _uniform_lens(gen, num_seqs, 256, 2048)
    lens = [1024 + u for u in suffix]
    return make_case("prefix_sharing_decode", seed, "bf16", 32, 8, 128, 16, lens,
                     shared_prefix_tokens=1024, gen=gen)


def mixed_chunked_prefill(seed: int = 5, num_decode: int = 16, chunk_len: int = 512,
                          chunk_prior: int = 2048, num_chunks: int = 2) -> PagedCase:
    """16 decode seqs (L ~ U{1024..4096}) + 2 prefill chunks of 512 queries over
    2048 prior paged tokens; the cache write covers all 16 + 2*512 new tokens."""
    gen = torch.Generator().manual_seed(seed)
    lens = _uniform_lens(gen, num_decode, 1024, 4096)
    chunks = [(chunk_len, chunk_prior + chunk_len)] * num_chunks
    return make_case("mixed_chunked_prefill", seed, "bf16", 32, 8, 128, 16, lens,
                     new_positions=[L - 1 for L in lens], chunks=chunks, gen=gen)


NAMED = {
    "tiny_decode": tiny_decode,
    "llama8b_decode": llama8b_decode,
    "long_context_decode": long_context_decode,
    "prefix_sharing_decode": prefix_sharing_decode,
    "mixed_chunked_prefill": mixed_chunked_prefill,
}


def random_case(seed: int, dtype: str, num_seqs: int, num_q_heads: int, num_kv_heads: int,
                head_dim: int, block_size: int, min_len: int, max_len: int,
                write_new: bool = True, extra_blocks: int = 3,
                chunks: Optional[List[tuple]] = None) -> PagedCase:
    """Small random case for parity sweeps (ragged lengths, spare blocks)."""
    gen = torch.Generator().manual_seed(seed)
    lens = _uniform_lens(gen, num_seqs, min_len, max_len)
    newpos = [L - 1 if (write_new and L > 0) else None for L in lens]
    return make_case(f"random_{seed}", seed, dtype, num_q_heads, num_kv_heads, head_dim,
                     block_size, lens, new_positions=newpos, extra_blocks=extra_blocks,
                     chunks=chunks, gen=gen)


def random_fp8_codes(seed: int, shape, exp_lo: int = 3, exp_hi: int = 9) -> torch.Tensor:
    """Seeded random e4m3 byte codes for FP8 pools: sign and 3 mantissa bits
    uniform, the 4-bit exponent field uniform in [exp_lo, exp_hi] (values of
    magnitude 2^(exp_lo - 7) .. 2^(exp_hi - 6), the spread of N(0, 1) data).
    No NaN code (exponent field 15) is drawn for these defaults.  Only random
    bits: the codes are not a quantisation of anything."""
    gen = torch.Generator().manual_seed(seed)
    sign = torch.randint(0, 2, shape, generator=gen, dtype=torch.int32)
    expo = torch.randint(exp_lo, exp_hi + 1, shape, generator=gen, dtype=torch.int32)
    mant = torch.randint(0, 8, shape, generator=gen, dtype=torch.int32)
    return ((sign << 7) | (expo << 3) | mant).to(torch.uint8)
