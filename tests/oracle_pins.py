"""Pins of the CPU oracle against facts that do not come from the oracle.

Each function takes a loaded oracle library (so that the mutation tests can
run the same pins against deliberately broken copies of the oracle) and
raises AssertionError when the oracle disagrees with:

  * the worked block-table examples printed on the pages (tests/golden/),
  * torch's fp64 scaled_dot_product_attention (a library routine) on the same
    keys and values laid out contiguously,
  * closed forms (a 1-token context returns V; constant V; q = 0 gives the
    mean of V; a dominant key returns its V),
  * invariants (relabelling physical blocks; shared vs private prefix blocks;
    softmax rows summing to one),
  * the cache-write contract (slots hit, everything else untouched, bitwise),
  * the block-copy contract (coded blocks land whole; copy-on-write and a swap
    round trip with the table redirected leave attention unchanged).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from paged_kv_cache_262_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _coded_pool(num_blocks, num_kv_heads, block_size, head_dim):
    """fp32 pool whose slot (b, h, o) holds [b, o, h, 1, 0, ...] (exact)."""
    pool = torch.zeros(num_blocks, num_kv_heads, block_size, head_dim, dtype=torch.float32)
    pool[..., 0] = torch.arange(num_blocks, dtype=torch.float32)[:, None, None]
    pool[..., 1] = torch.arange(block_size, dtype=torch.float32)[None, None, :]
    pool[..., 2] = torch.arange(num_kv_heads, dtype=torch.float32)[None, :, None]
    pool[..., 3] = 1.0
    return pool


# ---------------------------------------------------------------- indexing --

def pin_gather_page_examples(lib):
    """Token -> (physical block, offset) exactly as the pages' examples print."""
    for case in _golden("block_table_examples.json")["cases"]:
        B = case["block_size"]
        bt = case["block_table"]
        nb = max(bt) + 1
        pool = _coded_pool(nb, 2, B, 8)
        L = len(bt) * B
        for g in range(2):
            rows = oracle.gather(pool, bt, L, g, lib=lib)
            for tok, blk, off in case["tokens"]:
                assert rows[tok, 0] == blk and rows[tok, 1] == off and rows[tok, 2] == g, \
                    (case["source"], tok, rows[tok, :3])


def pin_decode_one_hot_page_examples(lib):
    """Decode through the pages' tables: a one-hot key selects exactly the
    value stored at the block/offset the example names."""
    for case in _golden("block_table_examples.json")["cases"]:
        B = case["block_size"]
        bt = torch.tensor([case["block_table"]], dtype=torch.int32)
        nb = int(bt.max()) + 1
        D = 16
        for tok, blk, off in case["tokens"]:
            L = tok + 1 + (tok % 3)         # target not always the last key
            L = min(L, bt.shape[1] * B)
            kc = torch.zeros(nb, 1, B, D)
            vc = _coded_pool(nb, 1, B, D)
            kc[blk, 0, off, 0] = 50.0
            q = torch.zeros(1, 1, D)
            q[0, 0, 0] = 50.0
            out = oracle.decode(q, kc, vc, bt, torch.tensor([L], dtype=torch.int32), 1.0,
                                lib=lib)
            assert out[0, 0, 0] == blk and out[0, 0, 1] == off, (case["source"], tok, out[0, 0, :2])


# ------------------------------------------------------- library routines --

def _contig_case(seed, S, Hq, Hkv, D, B, lens, dtype="f32"):
    """Random contiguous K/V per sequence, then placed into a permuted pool."""
    g = torch.Generator().manual_seed(seed)
    Lmax = max(lens)
    K = torch.randn(S, Hkv, Lmax, D, generator=g).to(W.DTYPES[dtype])
    V = torch.randn(S, Hkv, Lmax, D, generator=g).to(W.DTYPES[dtype])
    q = torch.randn(S, Hq, D, generator=g).to(W.DTYPES[dtype])
    nblk = [-(-L // B) for L in lens]
    NB = sum(nblk) + 2
    perm = torch.randperm(NB, generator=g)
    kc = torch.randn(NB, Hkv, B, D, generator=g).to(W.DTYPES[dtype])
    vc = torch.randn(NB, Hkv, B, D, generator=g).to(W.DTYPES[dtype])
    bt = torch.zeros(S, max(nblk), dtype=torch.int32)
    cur = 0
    for s in range(S):
        for b in range(nblk[s]):
            p = int(perm[cur]); cur += 1
            bt[s, b] = p
            n = min(B, lens[s] - b * B)
            kc[p, :, :n, :] = K[s, :, b * B:b * B + n, :]
            vc[p, :, :n, :] = V[s, :, b * B:b * B + n, :]
    return q, K, V, kc, vc, bt, torch.tensor(lens, dtype=torch.int32)


def pin_decode_matches_sdpa(lib):
    """Oracle decode == torch SDPA (fp64, GQA by repeat-interleave) on the
    contiguous K/V the pool was built from."""
    for dtype, (S, Hq, Hkv, D, B, lens) in [
        ("f32", (3, 4, 4, 64, 16, [1, 30, 77])),
        ("bf16", (4, 8, 2, 128, 16, [5, 16, 33, 70])),
        ("bf16", (2, 8, 1, 64, 32, [64, 95])),
    ]:
        q, K, V, kc, vc, bt, L = _contig_case(11, S, Hq, Hkv, D, B, lens, dtype)
        scale = 1.0 / math.sqrt(D)
        out = oracle.decode(q, kc, vc, bt, L, scale, lib=lib)
        for s in range(S):
            n = lens[s]
            ref = F.scaled_dot_product_attention(
                q[s].double()[None, :, None, :], K[s, :, :n].double()[None],
                V[s, :, :n].double()[None], scale=float(np.float32(scale)), enable_gqa=True)
            ref = ref[0, :, 0, :].numpy()
            np.testing.assert_allclose(out[s], ref, rtol=1e-11, atol=1e-12)


def pin_prefill_matches_sdpa(lib):
    """Causal chunk: query i of n sits at position L-n+i and sees keys 0..L-n+i."""
    for dtype, (Hq, Hkv, D, B, chunks) in [
        ("bf16", (8, 2, 64, 16, [(7, 40), (16, 16), (5, 21)])),
        ("f32", (4, 4, 64, 32, [(33, 70)])),
    ]:
        lens = [L for _, L in chunks]
        q_all, K, V, kc, vc, bt, Lt = _contig_case(13, len(chunks), Hq, Hkv, D, B, lens, dtype)
        g = torch.Generator().manual_seed(5)
        nq = sum(n for n, _ in chunks)
        q = torch.randn(nq, Hq, D, generator=g).to(W.DTYPES[dtype])
        cu = torch.tensor([0] + list(np.cumsum([n for n, _ in chunks])), dtype=torch.int32)
        scale = 0.37
        out = oracle.prefill(q, kc, vc, bt, cu, Lt, scale, lib=lib)
        for c, (n, L) in enumerate(chunks):
            qq = q[cu[c]:cu[c + 1]].double().permute(1, 0, 2)[None]
            pos = torch.arange(L - n, L)[:, None]
            mask = torch.arange(L)[None, :] <= pos
            ref = F.scaled_dot_product_attention(qq, K[c, :, :L].double()[None],
                                                 V[c, :, :L].double()[None], attn_mask=mask,
                                                 scale=float(np.float32(scale)), enable_gqa=True)
            ref = ref[0].permute(1, 0, 2).numpy()
            np.testing.assert_allclose(out[cu[c]:cu[c + 1]], ref, rtol=1e-11, atol=1e-12)


def pin_zero_query_gives_mean(lib):
    """q = 0: every weight is 1/L, the output is the plain mean of V (numpy)."""
    q, K, V, kc, vc, bt, L = _contig_case(17, 3, 2, 2, 64, 16, [1, 19, 48])
    q.zero_()
    out = oracle.decode(q, kc, vc, bt, L, 0.125, lib=lib)
    for s, n in enumerate([1, 19, 48]):
        np.testing.assert_allclose(out[s], V[s, :, :n].double().mean(1).numpy(), rtol=1e-13,
                                   atol=1e-14)


# ----------------------------------------------------------- closed forms --

def pin_single_token_returns_value(lib):
    """L = 1: the only weight is exp(0)/exp(0) = 1, so out == v_0 exactly."""
    c = W.tiny_decode()
    out = oracle.decode(c.query, c.key_cache, c.value_cache, c.block_tables, c.context_lens,
                        c.scale, lib=lib)
    assert c.context_lens[0] == 1
    phys = int(c.block_tables[0, 0])
    for h in range(c.num_q_heads):
        g = h // (c.num_q_heads // c.num_kv_heads)
        assert np.array_equal(out[0, h], c.value_cache[phys, g, 0].double().numpy())


def pin_constant_values(lib):
    """V identical for every key: the output is that vector for any weights."""
    c = W.random_case(21, "bf16", 3, 8, 2, 64, 16, 3, 60, write_new=False)
    vrow = torch.randn(c.num_kv_heads, c.head_dim).to(torch.bfloat16)
    vc = vrow[None, :, None, :].expand_as(c.value_cache).contiguous()
    out = oracle.decode(c.query, c.key_cache, vc, c.block_tables, c.context_lens, c.scale,
                        lib=lib)
    G = c.num_q_heads // c.num_kv_heads
    for h in range(c.num_q_heads):
        np.testing.assert_allclose(out[:, h], np.broadcast_to(vrow[h // G].double().numpy(),
                                                               out[:, h].shape), rtol=1e-14)


def pin_dominant_key(lib):
    """One key far above the rest: its weight is 1, the others underflow."""
    c = W.random_case(23, "f32", 2, 4, 4, 64, 16, 20, 50, write_new=False)
    kc = c.key_cache.clone()
    q = c.query.clone()
    q[..., 0] = 0
    for s in range(c.num_seqs):
        L = int(c.context_lens[s])
        t = (7 * s + 3) % L
        phys, off = int(c.block_tables[s, t // 16]), t % 16
        kc[phys, :, off, :] = 0
        kc[phys, :, off, 0] = 1000.0
        q[s, :, :] = 0
        q[s, :, 0] = 1000.0
    out = oracle.decode(q, kc, c.value_cache, c.block_tables, c.context_lens, 1.0, lib=lib)
    for s in range(c.num_seqs):
        L = int(c.context_lens[s])
        t = (7 * s + 3) % L
        phys, off = int(c.block_tables[s, t // 16]), t % 16
        for h in range(c.num_q_heads):
            assert np.array_equal(out[s, h], c.value_cache[phys, h, off].double().numpy())


def pin_row_sums(lib):
    c = W.random_case(29, "bf16", 4, 8, 2, 64, 16, 1, 90, write_new=False)
    out, w = oracle.decode(c.query, c.key_cache, c.value_cache, c.block_tables,
                           c.context_lens, c.scale, return_weights=True, lib=lib)
    for s in range(c.num_seqs):
        L = int(c.context_lens[s])
        np.testing.assert_allclose(w[s, :, :L].sum(-1), 1.0, rtol=0, atol=1e-12)
        assert (w[s, :, L:] == 0).all() and (w[s, :, :L] > 0).all()


def pin_empty_context_gives_zeros(lib):
    c = W.random_case(31, "bf16", 3, 4, 2, 64, 16, 0, 0, write_new=False)
    c.context_lens[1] = 12
    out = oracle.decode(c.query, c.key_cache, c.value_cache, c.block_tables, c.context_lens,
                        c.scale, lib=lib)
    assert (out[0] == 0).all() and (out[2] == 0).all() and np.abs(out[1]).sum() > 0


# ------------------------------------------------------------- invariants --

def _relabel(case, seed):
    """Move every physical block to a new id; tables follow.  Same data."""
    g = torch.Generator().manual_seed(seed)
    NB = case.key_cache.shape[0]
    pi = torch.randperm(NB, generator=g)
    kc = torch.empty_like(case.key_cache)
    vc = torch.empty_like(case.value_cache)
    kc[pi] = case.key_cache
    vc[pi] = case.value_cache
    bt = pi[case.block_tables.long()].to(torch.int32)
    return kc, vc, bt


def pin_block_relabelling_invariance(lib):
    for dtype in ("f32", "bf16"):
        c = W.random_case(37, dtype, 5, 8, 4, 64, 16, 1, 120, write_new=False)
        ref = oracle.decode(c.query, c.key_cache, c.value_cache, c.block_tables,
                            c.context_lens, c.scale, lib=lib)
        kc, vc, bt = _relabel(c, 3)
        out = oracle.decode(c.query, kc, vc, bt, c.context_lens, c.scale, lib=lib)
        assert np.array_equal(ref, out)


def pin_shared_prefix_invariance(lib):
    """Blocks referenced by every table (ref count = number of seqs) give the
    same output as private copies of those blocks."""
    c = W.make_case("p", 41, "bf16", 8, 2, 64, 16, [48 + 5, 48 + 40, 48 + 17],
                    shared_prefix_tokens=48)
    ref = oracle.decode(c.query, c.key_cache, c.value_cache, c.block_tables, c.context_lens,
                        c.scale, lib=lib)
    shared = c.shared_blocks.long()
    assert all(set(shared.tolist()) <= set(c.block_tables[s].tolist()) for s in range(3))
    S = c.num_seqs
    NB = c.key_cache.shape[0]
    kc = torch.cat([c.key_cache] + [c.key_cache[shared]] * S)
    vc = torch.cat([c.value_cache] + [c.value_cache[shared]] * S)
    bt = c.block_tables.clone()
    n = len(shared)
    for s in range(S):
        bt[s, :n] = torch.arange(NB + s * n, NB + (s + 1) * n, dtype=torch.int32)
    out = oracle.decode(c.query, kc, vc, bt, c.context_lens, c.scale, lib=lib)
    assert np.array_equal(ref, out)


def pin_gqa_equals_repeated_kv(lib):
    """Grouped heads equal full multi-head attention with every kv head
    repeated G times (consecutive q heads share a kv head)."""
    c = W.random_case(43, "bf16", 3, 8, 2, 64, 16, 10, 70, write_new=False)
    G = c.num_q_heads // c.num_kv_heads
    ref = oracle.decode(c.query, c.key_cache, c.value_cache, c.block_tables, c.context_lens,
                        c.scale, lib=lib)
    kc = c.key_cache.repeat_interleave(G, dim=1).contiguous()
    vc = c.value_cache.repeat_interleave(G, dim=1).contiguous()
    out = oracle.decode(c.query, kc, vc, c.block_tables, c.context_lens, c.scale, lib=lib)
    assert np.array_equal(ref, out)


def pin_prefill_last_row_is_decode(lib):
    """The last query of a chunk sees every key: it equals a decode step."""
    c = W.random_case(47, "bf16", 1, 8, 2, 64, 16, 1, 1, write_new=False,
                      chunks=[(9, 50), (4, 4)])
    out = oracle.prefill(c.chunk_query, c.key_cache, c.value_cache, c.chunk_block_tables,
                         c.chunk_cu_query_lens, c.chunk_context_lens, c.scale, lib=lib)
    cu = c.chunk_cu_query_lens
    for k in range(c.num_chunks):
        last = int(cu[k + 1]) - 1
        dec = oracle.decode(c.chunk_query[last:last + 1], c.key_cache, c.value_cache,
                            c.chunk_block_tables[k:k + 1], c.chunk_context_lens[k:k + 1],
                            c.scale, lib=lib)
        assert np.array_equal(out[last], dec[0])


# ------------------------------------------------------------- cache write --

def pin_cache_write(lib):
    """Each new token lands in its slot bit for bit; nothing else changes; the
    written token is what a later gather returns at the sequence's last
    position; special bit patterns survive."""
    c = W.random_case(53, "bf16", 4, 8, 2, 64, 16, 3, 70)
    nk, nv = c.new_key.clone(), c.new_value.clone()
    raw = nk.view(torch.int16)
    raw[0, 0, :4] = torch.tensor([0x7FC1, -0x8000, 0x0001, 0x7F80], dtype=torch.int16)
    kc, vc = oracle.reshape_and_cache(nk, nv, c.key_cache, c.value_cache, c.slot_mapping,
                                      lib=lib)
    B = c.block_size
    touched = torch.zeros(c.key_cache.shape[0], B, dtype=torch.bool)
    for t, s in enumerate(c.slot_mapping.tolist()):
        blk, off = s // B, s % B
        touched[blk, off] = True
        assert torch.equal(kc[blk, :, off].view(torch.int16), nk[t].view(torch.int16))
        assert torch.equal(vc[blk, :, off].view(torch.int16), nv[t].view(torch.int16))
    keep = ~touched[:, None, :].expand(-1, c.num_kv_heads, -1)
    assert torch.equal(kc.view(torch.int16)[keep], c.key_cache.view(torch.int16)[keep])
    assert torch.equal(vc.view(torch.int16)[keep], c.value_cache.view(torch.int16)[keep])
    for s in range(c.num_seqs):
        L = int(c.context_lens[s])
        for g in range(c.num_kv_heads):
            rows = oracle.gather(kc, c.block_tables[s], L, g, lib=lib)
            want = nk[s, g].double().numpy()
            np.testing.assert_array_equal(rows[L - 1][~np.isnan(want)], want[~np.isnan(want)])


def pin_cache_write_rejects_bad_slots(lib):
    c = W.random_case(59, "f32", 3, 4, 4, 64, 16, 3, 40)
    slots = c.slot_mapping.clone()
    slots[1] = -1                                   # padding: skipped
    kc, _ = oracle.reshape_and_cache(c.new_key, c.new_value, c.key_cache, c.value_cache,
                                     slots, lib=lib)
    s1 = int(c.slot_mapping[1])
    assert torch.equal(kc[s1 // 16, :, s1 % 16], c.key_cache[s1 // 16, :, s1 % 16])
    bad = c.slot_mapping.clone()
    bad[2] = c.key_cache.shape[0] * 16
    try:
        oracle.reshape_and_cache(c.new_key, c.new_value, c.key_cache, c.value_cache, bad, lib=lib)
        raise AssertionError("out-of-range slot accepted")
    except oracle.OracleError as e:
        assert e.code == 3
    dup = c.slot_mapping.clone()
    dup[2] = dup[0]
    try:
        oracle.reshape_and_cache(c.new_key, c.new_value, c.key_cache, c.value_cache, dup, lib=lib)
        raise AssertionError("duplicate slot accepted")
    except oracle.OracleError as e:
        assert e.code == 4


# -------------------------------------------------------------- block copy --

def _used_blocks(c):
    used = set()
    for s in range(c.num_seqs):
        nb = -(-int(c.context_lens[s]) // c.block_size)
        used.update(int(x) for x in c.block_tables[s, :nb].tolist())
    return used


def pin_copy_blocks_moves_whole_blocks(lib):
    """On coded pools (every element names its block, offset and head), each
    destination block afterwards holds exactly its source block's codes, in K
    and V alike, and every other destination block is unchanged: across pools
    (swap) and inside one pool (copy-on-write)."""
    NB, Hkv, B, D = 12, 2, 16, 64
    kc = _coded_pool(NB, Hkv, B, D)
    vc = kc * 2.0 + 1.0
    # across pools: a smaller destination pool, one source copied twice
    dk0 = torch.full((6, Hkv, B, D), -7.0)
    dv0 = dk0.clone()
    pairs = [(3, 5), (0, 1), (11, 0), (3, 2)]
    dk, dv = oracle.copy_blocks(kc, vc, dk0, dv0, pairs, lib=lib)
    offs = torch.arange(B, dtype=torch.float32)[None, :]
    heads = torch.arange(Hkv, dtype=torch.float32)[:, None]
    for src, dst in pairs:
        assert torch.all(dk[dst, :, :, 0] == src) and torch.all(dk[dst, :, :, 1] == offs)
        assert torch.all(dk[dst, :, :, 2] == heads) and torch.all(dk[dst, :, :, 3] == 1.0)
        assert torch.all(dv[dst, :, :, 0] == 2 * src + 1)
    for d in (3, 4):
        assert torch.all(dk[d] == -7.0) and torch.all(dv[d] == -7.0)
    # inside one pool
    k2, v2 = oracle.copy_blocks(kc, vc, kc, vc, [(1, 9), (4, 10)], lib=lib)
    for src, dst in ((1, 9), (4, 10)):
        assert torch.all(k2[dst, :, :, 0] == src) and torch.all(v2[dst, :, :, 0] == 2 * src + 1)
    for b in set(range(NB)) - {9, 10}:
        assert torch.equal(k2[b], kc[b]) and torch.equal(v2[b], vc[b])


def pin_copy_on_write_keeps_attention(lib):
    """Copying a sequence's blocks to free blocks and pointing its table at the
    copies (copy-on-write before a write) leaves every decode output bit for
    bit unchanged."""
    for dtype in ("f32", "bf16"):
        c = W.random_case(61, dtype, 3, 8, 2, 64, 16, 20, 90, write_new=False, extra_blocks=8)
        ref = oracle.decode(c.query, c.key_cache, c.value_cache, c.block_tables,
                            c.context_lens, c.scale, lib=lib)
        free = sorted(set(range(c.key_cache.shape[0])) - _used_blocks(c))
        nb0 = -(-int(c.context_lens[0]) // c.block_size)
        assert len(free) >= nb0
        pairs = [(int(c.block_tables[0, j]), free[j]) for j in range(nb0)]
        kc, vc = oracle.copy_blocks(c.key_cache, c.value_cache, c.key_cache, c.value_cache,
                                    pairs, lib=lib)
        bt = c.block_tables.clone()
        bt[0, :nb0] = torch.tensor([d for _, d in pairs], dtype=torch.int32)
        out = oracle.decode(c.query, kc, vc, bt, c.context_lens, c.scale, lib=lib)
        assert np.array_equal(ref, out)


def pin_swap_round_trip(lib):
    """Swapping a sequence's blocks out to a host pool and back into other
    free blocks (table redirected) gives the same decode output bit for bit;
    the host pool holds the blocks in swap order."""
    c = W.random_case(67, "bf16", 3, 8, 2, 128, 16, 30, 100, write_new=False, extra_blocks=8)
    ref = oracle.decode(c.query, c.key_cache, c.value_cache, c.block_tables, c.context_lens,
                        c.scale, lib=lib)
    nb1 = -(-int(c.context_lens[1]) // c.block_size)
    own = [int(x) for x in c.block_tables[1, :nb1].tolist()]
    hk0 = torch.zeros((nb1,) + tuple(c.key_cache.shape[1:]), dtype=c.key_cache.dtype)
    hk, hv = oracle.copy_blocks(c.key_cache, c.value_cache, hk0, hk0.clone(),
                                [(b, i) for i, b in enumerate(own)], lib=lib)
    for i, b in enumerate(own):
        assert torch.equal(hk[i].view(torch.int16), c.key_cache[b].view(torch.int16))
        assert torch.equal(hv[i].view(torch.int16), c.value_cache[b].view(torch.int16))
    free = sorted(set(range(c.key_cache.shape[0])) - _used_blocks(c))[:nb1]
    kc, vc = oracle.copy_blocks(hk, hv, c.key_cache, c.value_cache,
                                [(i, f) for i, f in enumerate(free)], lib=lib)
    bt = c.block_tables.clone()
    bt[1, :nb1] = torch.tensor(free, dtype=torch.int32)
    out = oracle.decode(c.query, kc, vc, bt, c.context_lens, c.scale, lib=lib)
    assert np.array_equal(ref, out)


def pin_copy_blocks_rejects(lib):
    kc = _coded_pool(6, 1, 16, 64)
    vc = kc.clone()
    k, v = oracle.copy_blocks(kc, vc, kc, vc, torch.zeros((0, 2), dtype=torch.int64), lib=lib)
    assert torch.equal(k, kc) and torch.equal(v, vc)
    for pairs, code, same in (([(0, 6)], 2, True), ([(-1, 2)], 2, True), ([(0, 2), (1, 2)], 4, True),
                              ([(0, 2), (2, 3)], 6, True), ([(0, 2), (2, 3)], 0, False)):
        dk, dv = (kc, vc) if same else (kc.clone(), vc.clone())
        try:
            oracle.copy_blocks(kc, vc, dk, dv, pairs, lib=lib)
            assert code == 0, f"{pairs} accepted"
        except oracle.OracleError as e:
            assert e.code == code, (pairs, e.code)


# -------------------------------------------------------------- FP8 cache --

def _e4m3_table():
    """The 256 e4m3 values from the format's definition (OCP 8-bit floating
    point, E4M3: exponent bias 7, no infinities, S.1111.111 is NaN)."""
    vals = []
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 7
        if e == 0xF and m == 7:
            vals.append(math.nan)
        elif e == 0:
            vals.append(sign * m * 2.0 ** -9)
        else:
            vals.append(sign * (8 + m) * 2.0 ** (e - 10))
    return vals


def pin_fp8_code_values(lib):
    want = _e4m3_table()
    got = oracle.fp8_decode(torch.arange(256, dtype=torch.uint8), lib=lib)
    for c in range(256):
        assert (math.isnan(want[c]) and math.isnan(got[c])) or want[c] == got[c], c
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6
    assert got[0x38] == 1.0 and math.copysign(1.0, got[0x80]) < 0


def pin_fp8_encode_rounding(lib):
    """Every finite value encodes to its own code; midpoints go to the even
    code; overflow saturates at 448; NaN is 0x7F; the scale divides first."""
    vals = _e4m3_table()
    codes = [c for c in range(256) if not math.isnan(vals[c])]
    enc = oracle.fp8_encode(torch.tensor([vals[c] for c in codes]), lib=lib)
    assert enc.tolist() == codes
    mids = torch.tensor([1.0625, 1.1875, 1.3125, 2.0 ** -9 * 0.5, 2.0 ** -9 * 1.5, 232.0, 464.0])
    want = [0x38, 0x3A, 0x3A, 0x00, 0x02, 0x76, 0x7E]   # ties to the even code
    assert oracle.fp8_encode(mids, lib=lib).tolist() == want
    assert oracle.fp8_encode(-mids, lib=lib).tolist() == [0x80 | w for w in want]
    sat = torch.tensor([449.0, 1000.0, 1e30, math.inf, -math.inf, math.nan])
    assert oracle.fp8_encode(sat, lib=lib).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7F]
    x = torch.randn(500) * 37
    assert torch.equal(oracle.fp8_encode(x, 4.0, lib=lib), oracle.fp8_encode(x * 0.25, lib=lib))
    # the nearest code: no code value lies strictly closer than the chosen one
    y = torch.randn(2000) * 50
    e = oracle.fp8_encode(y, lib=lib)
    dec = oracle.fp8_decode(e, lib=lib)
    finite = np.array([v for v in vals[:0x7F]])
    for yi, di in zip(y.tolist(), dec.tolist()):
        a = min(abs(yi), 448.0)
        assert abs(abs(di) - a) <= np.min(np.abs(finite - a)) + 0.0


def _nearest_e4m3(y):
    """Code of the e4m3 value nearest to y (ties to the even code, saturating at
    448), by a search over the format table; written apart from the oracle."""
    vals = _e4m3_table()
    sign = 0x80 if math.copysign(1.0, y) < 0 else 0
    a = min(abs(y), 448.0)
    best, best_d = None, None
    for c in range(0x7F):
        d = abs(vals[c] - a)
        if best_d is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return sign | best


def pin_fp8_scale_is_one_reciprocal_multiply(lib):
    """The stored code is that of x * fp32(1 / scale), one fp32 multiply by the
    reciprocal (the FP8 reading of the build).  At these two (x, scale) pairs
    the fp32 product and the fp32 quotient x / scale fall on opposite sides
    of the midpoint 7.5 * 2^-9 between codes 0x07 and 0x08, so the two
    readings give different codes; expected codes come from numpy fp32
    arithmetic and the format table."""
    cases = [(0.00439453125, 0.3), (0.02490234375, 1.7)]
    for x, s in cases:
        xf, sf = np.float32(x), np.float32(s)
        want = _nearest_e4m3(float(xf * (np.float32(1.0) / sf)))
        other = _nearest_e4m3(float(xf / sf))
        assert want != other, (x, s)          # the case separates the readings
        assert oracle.fp8_encode(torch.tensor([x, -x]), s, lib=lib).tolist() == [want, 0x80 | want]
        # the cache write (K row and transposed V page) takes the same reading
        key = torch.full((1, 1, 64), x)
        kc0 = torch.zeros((2, 1, 16, 64), dtype=torch.uint8)
        vc0 = torch.zeros((2, 1, 64, 16), dtype=torch.uint8)
        kc, vc = oracle.reshape_and_cache_fp8(key, -key, kc0, vc0, [16 + 3], s, s, lib=lib)
        assert torch.all(kc[1, 0, 3, :] == want) and torch.all(vc[1, 0, :, 3] == (0x80 | want))
    assert [_nearest_e4m3(float(np.float32(x) * (np.float32(1.0) / np.float32(s))))
            for x, s in cases] == [0x08, 0x07]


def pin_fp8_cache_write_layout(lib):
    """K lands at [block][head][offset][d], V transposed at [block][head][d][offset],
    each the code of value / scale; untouched bytes keep their value."""
    NB, Hkv, B, D = 5, 2, 16, 64
    key = torch.zeros(2, Hkv, D)
    val = torch.zeros(2, Hkv, D)
    key[0, 1, 3], val[0, 1, 3] = 1.0, 2.0    # token 0 -> slot 2 * 16 + 5
    key[1, 0, 7], val[1, 0, 60] = -3.0, 0.5  # token 1 -> slot 4 * 16 + 0
    kc0 = torch.full((NB, Hkv, B, D), 0xAA, dtype=torch.uint8)
    vc0 = torch.full((NB, Hkv, D, B), 0xAA, dtype=torch.uint8)
    kc, vc = oracle.reshape_and_cache_fp8(key, val, kc0, vc0, [2 * 16 + 5, 4 * 16], 0.5, 2.0,
                                          lib=lib)
    assert kc[2, 1, 5, 3] == 0x40 and vc[2, 1, 3, 5] == 0x38           # 2.0 and 1.0
    assert kc[4, 0, 0, 7] == 0xCC and vc[4, 0, 60, 0] == 0x28          # -6.0 = -1.5 * 2^2, 0.25
    assert kc[2, 1, 5, 0] == 0 and vc[2, 0, 0, 5] == 0                  # zeros of the rows
    touched_k = torch.zeros_like(kc, dtype=torch.bool)
    touched_k[2, :, 5, :] = True
    touched_k[4, :, 0, :] = True
    touched_v = torch.zeros_like(vc, dtype=torch.bool)
    touched_v[2, :, :, 5] = True
    touched_v[4, :, :, 0] = True
    assert torch.all(kc[~touched_k] == 0xAA) and torch.all(vc[~touched_v] == 0xAA)


def pin_fp8_decode_equals_dequantized_decode(lib):
    """Decode over FP8 pools equals decode over float pools that hold the
    dequantised values (code value x scale, exact in fp32 for these scales)."""
    c = W.random_case(71, "bf16", 4, 8, 2, 64, 16, 1, 90, write_new=False)
    NB, Hkv, B, D = c.key_cache.shape
    ks, vs = 0.25, 0.5
    kc8 = oracle.fp8_encode(c.key_cache.float(), ks, lib=lib)
    vc8 = oracle.fp8_encode(c.value_cache.float(), vs, lib=lib).permute(0, 1, 3, 2).contiguous()
    kf = torch.from_numpy(oracle.fp8_decode(kc8, lib=lib) * ks).float()
    vf = torch.from_numpy(oracle.fp8_decode(vc8, lib=lib) * vs).float().permute(0, 1, 3, 2).contiguous()
    q = c.query.float()
    ref = oracle.decode(q, kf, vf, c.block_tables, c.context_lens, c.scale, lib=lib)
    out = oracle.decode_fp8(q, kc8, vc8, c.block_tables, c.context_lens, c.scale, ks, vs,
                            lib=lib)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def _fp8_prefill_case(lib, ks, vs):
    c = W.random_case(72, "bf16", 2, 8, 2, 64, 16, 20, 60, write_new=False,
                      chunks=[(37, 90), (16, 16), (5, 70)])
    kc8 = oracle.fp8_encode(c.key_cache.float(), ks, lib=lib)
    vc8 = oracle.fp8_encode(c.value_cache.float(), vs, lib=lib).permute(0, 1, 3, 2).contiguous()
    return c, kc8, vc8


def pin_fp8_prefill_equals_dequantized_prefill(lib):
    """Prefill chunks over FP8 pools equal the plain prefill over float pools
    that hold the dequantised values (exact in fp32 for these scales)."""
    ks, vs = 0.25, 0.125
    c, kc8, vc8 = _fp8_prefill_case(lib, ks, vs)
    kf = torch.from_numpy(oracle.fp8_decode(kc8, lib=lib) * ks).float()
    vf = torch.from_numpy(oracle.fp8_decode(vc8, lib=lib) * vs).float().permute(0, 1, 3, 2).contiguous()
    ref = oracle.prefill(c.chunk_query.float(), kf, vf, c.chunk_block_tables,
                         c.chunk_cu_query_lens, c.chunk_context_lens, c.scale, lib=lib)
    out = oracle.prefill_fp8(c.chunk_query, kc8, vc8, c.chunk_block_tables, c.chunk_cu_query_lens,
                             c.chunk_context_lens, c.scale, ks, vs, lib=lib)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def pin_fp8_prefill_last_row_is_decode(lib):
    """The last query of a chunk sees every key of its context: its row equals
    FP8 decode over the same table and length."""
    ks, vs = 0.03, 0.07
    c, kc8, vc8 = _fp8_prefill_case(lib, ks, vs)
    out = oracle.prefill_fp8(c.chunk_query, kc8, vc8, c.chunk_block_tables, c.chunk_cu_query_lens,
                             c.chunk_context_lens, c.scale, ks, vs, lib=lib)
    last = c.chunk_cu_query_lens[1:].long() - 1
    dec = oracle.decode_fp8(c.chunk_query[last], kc8, vc8, c.chunk_block_tables,
                            c.chunk_context_lens, c.scale, ks, vs, lib=lib)
    np.testing.assert_allclose(out[last.numpy()], dec, rtol=1e-12, atol=1e-12)


ALL_PINS = [
    pin_gather_page_examples,
    pin_decode_one_hot_page_examples,
    pin_decode_matches_sdpa,
    pin_prefill_matches_sdpa,
    pin_zero_query_gives_mean,
    pin_single_token_returns_value,
    pin_constant_values,
    pin_dominant_key,
    pin_row_sums,
    pin_empty_context_gives_zeros,
    pin_block_relabelling_invariance,
    pin_shared_prefix_invariance,
    pin_gqa_equals_repeated_kv,
    pin_prefill_last_row_is_decode,
    pin_cache_write,
    pin_cache_write_rejects_bad_slots,
    pin_copy_blocks_moves_whole_blocks,
    pin_copy_on_write_keeps_attention,
    pin_swap_round_trip,
    pin_copy_blocks_rejects,
    pin_fp8_code_values,
    pin_fp8_encode_rounding,
    pin_fp8_scale_is_one_reciprocal_multiply,
    pin_fp8_cache_write_layout,
    pin_fp8_decode_equals_dequantized_decode,
    pin_fp8_prefill_equals_dequantized_prefill,
    pin_fp8_prefill_last_row_is_decode,
]
