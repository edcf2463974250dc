"""Algorithmic byte and flop counts of the paged-attention hot path.

These are the figures a kernel must at least move or compute; throughput and
roofline fractions are these counts divided by measured time.

KV bytes per token follow the sizing formula of "Configuring vLLM and
PagedAttention for High Throughput Enterprise LLM Serving", section "KV Cache
Memory Sizing Formula": 2 (K and V) x layers x kv heads x head dim x bytes per
element.
"""
from __future__ import annotations

from typing import Iterable, Sequence


def kv_bytes_per_token(layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return 2 * layers * num_kv_heads * head_dim * elem_bytes


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def decode_bytes(context_lens: Sequence[int], num_q_heads: int, num_kv_heads: int,
                 head_dim: int, block_size: int, elem_bytes: int,
                 unique_tokens: int | None = None, q_elem_bytes: int | None = None) -> int:
    """K/V of every attended token (once per distinct physical token when
    ``unique_tokens`` is given, as for blocks shared by several sequences),
    plus the query read and the output write, block-table entries and lengths.
    ``elem_bytes`` is that of the cache (1 for FP8); the query and output use
    ``q_elem_bytes`` (default: the same)."""
    S = len(context_lens)
    toks = sum(context_lens) if unique_tokens is None else unique_tokens
    kv = toks * kv_bytes_per_token(1, num_kv_heads, head_dim, elem_bytes)
    qo = 2 * S * num_q_heads * head_dim * (q_elem_bytes or elem_bytes)
    bt = sum(_cdiv(L, block_size) for L in context_lens) * 4 + 4 * S
    return kv + qo + bt


def decode_flops(context_lens: Iterable[int], num_q_heads: int, head_dim: int) -> int:
    return 4 * head_dim * num_q_heads * sum(context_lens)


def cache_write_bytes(num_tokens: int, num_kv_heads: int, head_dim: int, elem_bytes: int,
                      src_elem_bytes: int | None = None) -> int:
    """Read K and V rows of the new tokens (``src_elem_bytes`` each, default
    ``elem_bytes``), write them into the pools (``elem_bytes`` each), read slots."""
    n = num_tokens * num_kv_heads * head_dim * 2
    return n * ((src_elem_bytes or elem_bytes) + elem_bytes) + 8 * num_tokens


def prefill_flops(chunks: Iterable[tuple], num_q_heads: int, head_dim: int) -> int:
    """QK^T and PV over the unmasked (query, key) pairs of causal chunks given
    as (num_queries, context_len incl. the chunk)."""
    pairs = 0
    for n, L in chunks:
        pairs += n * (L - n) + n * (n + 1) // 2
    return 4 * head_dim * num_q_heads * pairs


def prefill_bytes(chunks: Iterable[tuple], num_q_heads: int, num_kv_heads: int,
                  head_dim: int, elem_bytes: int) -> int:
    """Each chunk reads its keys/values once and its queries, writes its outputs."""
    total = 0
    for n, L in chunks:
        total += L * kv_bytes_per_token(1, num_kv_heads, head_dim, elem_bytes)
        total += 2 * n * num_q_heads * head_dim * elem_bytes
    return total
