"""Reference model of the block manager -- TEST INFRASTRUCTURE ONLY.

Only ``tests/`` may use it.  It shares nothing with the library's C++ block
manager and is written to be read against the pages: a pool of fixed-size
physical blocks, a block table per sequence mapping logical to physical
blocks, a reference count per block, blocks taken from a free pool on demand
and returned when a sequence ends ("vLLM High-Performance Inference Engine:
PagedAttention Principles and Deployment Guide", section "PagedAttention
Architecture Deep Dive"; "Configuring vLLM and PagedAttention for High
Throughput Enterprise LLM Serving", section "Architectural Foundations:
PagedAttention & Virtual Memory"), sharing with copy-on-write ("vLLM Guide:
High-Throughput Multi-GPU LLM Serving with PagedAttention", section "What Is
PagedAttention?") and prefix caching of full prompt blocks.

The policy it fixes (the library follows the same one, so that the two can
be compared operation by operation):
  * the free pool is first-in first-out, blocks 0, 1, ... at first;
  * a sequence takes a new block when its last block is full;
  * a write into a shared, partly filled last block takes a new block and
    queues the copy (old, new);
  * with the prefix cache, a full block is indexed under its exact content:
    the block before it in the sequence (with that block's generation: the
    number of times the pool has handed it out) and its own tokens.  A new
    sequence reuses the indexed blocks that match its prompt block by block
    from the start.  A freed indexed block stays findable until the pool
    hands it out again.

No hashing: the index is a dict keyed by the exact content, which is what a
hash index with full verification computes.

Parity pins: tests/test_block_manager.py checks this model against closed
forms (the number of blocks is ceil(L / B); the unused slots of a sequence,
ceil(L / B) * B - L, are fewer than B), invariants (reference counts equal
the number of table entries naming a block; free + referenced = the pool;
a fork shares every block) and the pages' block-table example.
"""
from __future__ import annotations

from collections import deque


class PoolExhausted(RuntimeError):
    pass


class ReferenceBlockManager:
    def __init__(self, num_blocks: int, block_size: int, prefix_cache: bool):
        self.B = block_size
        self.num_blocks = num_blocks
        self.prefix_cache = prefix_cache
        self.ref = [0] * num_blocks
        self.gen = [0] * num_blocks
        self.in_free = [True] * num_blocks
        self.free_q = deque(range(num_blocks))
        self.free_count = num_blocks
        self.key_of = {}        # block -> its key while indexed
        self.index = {}         # key -> block
        self.tables = {}        # seq -> list of blocks
        self.tokens = {}        # seq -> list of token ids
        self.copies = []
        self.hits = 0

    # -- pool ----------------------------------------------------------------
    def _uncache(self, b):
        key = self.key_of.pop(b, None)
        if key is not None and self.index.get(key) == b:
            del self.index[key]

    def _take(self):
        while self.free_q:
            b = self.free_q.popleft()
            if not self.in_free[b]:
                continue  # taken back from the index meanwhile
            self.in_free[b] = False
            self.free_count -= 1
            self._uncache(b)
            self.ref[b] = 1
            self.gen[b] += 1
            return b
        raise PoolExhausted

    def _release(self, b):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.in_free[b] = True
            self.free_count += 1
            self.free_q.append(b)

    def _key(self, parent, toks):
        return (parent, self.gen[parent] if parent >= 0 else 0, tuple(toks))

    def _index_full_block(self, seq, j):
        if not self.prefix_cache:
            return
        table, toks = self.tables[seq], self.tokens[seq]
        b = table[j]
        key = self._key(table[j - 1] if j > 0 else -1, toks[j * self.B:(j + 1) * self.B])
        if b in self.key_of or key in self.index:
            return
        self.index[key] = b
        self.key_of[b] = key

    # -- operations ----------------------------------------------------------
    def add_sequence(self, seq, tokens):
        """Returns (slot per prompt token, -1 where the block came from the
        prefix cache; number of cached tokens)."""
        assert seq not in self.tables
        B, n = self.B, len(tokens)
        nblk = -(-n // B)
        table = []
        if self.prefix_cache:
            # the last prompt token always gets a slot (its query row gives
            # the next token), so at most (n - 1) // B blocks are reused
            for j in range(max(0, n - 1) // B):
                key = self._key(table[-1] if table else -1, tokens[j * B:(j + 1) * B])
                b = self.index.get(key)
                if b is None:
                    break
                table.append(b)
        reused = len(table)
        reclaim = sum(1 for b in table if self.ref[b] == 0)  # cached but free
        if self.free_count - reclaim < nblk - reused:
            raise PoolExhausted
        for b in table:
            if self.ref[b] == 0:
                self.in_free[b] = False
                self.free_count -= 1
            self.ref[b] += 1
        self.hits += reused
        for _ in range(nblk - reused):
            table.append(self._take())
        self.tables[seq] = table
        self.tokens[seq] = list(tokens)
        slots = [-1 if t < reused * B else table[t // B] * B + t % B for t in range(n)]
        for j in range(reused, n // B):
            self._index_full_block(seq, j)
        return slots, reused * B

    def append(self, seq, token):
        B = self.B
        table, toks = self.tables[seq], self.tokens[seq]
        off = len(toks) % B
        if off == 0:
            if self.free_count < 1:
                raise PoolExhausted
            table.append(self._take())
        elif self.ref[table[-1]] > 1:
            if self.free_count < 1:
                raise PoolExhausted
            fresh = self._take()
            self.copies.append((table[-1], fresh))
            self._release(table[-1])
            table[-1] = fresh
        slot = table[-1] * B + off
        toks.append(token)
        if len(toks) % B == 0:
            self._index_full_block(seq, len(toks) // B - 1)
        return slot

    def fork(self, parent, child):
        assert child not in self.tables and parent != child
        self.tables[child] = list(self.tables[parent])
        self.tokens[child] = list(self.tokens[parent])
        for b in self.tables[child]:
            self.ref[b] += 1

    def free(self, seq):
        for b in self.tables.pop(seq):
            self._release(b)
        del self.tokens[seq]

    def take_copies(self):
        c, self.copies = self.copies, []
        return c

    def stats(self):
        return {
            "num_blocks": self.num_blocks,
            "free_blocks": self.free_count,
            "used_blocks": self.num_blocks - self.free_count,
            "shared_blocks": sum(1 for r in self.ref if r > 1),
            "cached_blocks": len(self.key_of),
            "num_seqs": len(self.tables),
            "seq_tokens": sum(len(t) for t in self.tokens.values()),
            "seq_slots": sum(len(t) for t in self.tables.values()) * self.B,
            "prefix_hits": self.hits,
        }
