"""GPU parity of the FP8 (e4m3) KV cache, through the C ABI.

The quantising cache write must equal the oracle's byte for byte (codes are
integers).  Decode over FP8 pools must be within the bf16 tolerance (1e-2 abs
+ 2e-2 rel) of the oracle's fp64 decode over the same codes: the kernel widens
every code to bf16 exactly, so its only rounding is that of the bf16 path.
Pools for small cases are the oracle's encoding of N(0, 1) data; the full-size
case uses seeded random codes.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_262_amd import binding
from paged_kv_cache_262_amd import workloads as W
from tests.gpu_util import check_close, dev, say

pytestmark = pytest.mark.gpu

NAN_CODE = 0x7F


def fp8_pools(case, ks, vs):
    """Oracle encoding of the case's pools: K [NB, Hkv, B, D], V [NB, Hkv, D, B]."""
    kc8 = oracle.fp8_encode(case.key_cache.float(), ks)
    vc8 = oracle.fp8_encode(case.value_cache.float(), vs).permute(0, 1, 3, 2).contiguous()
    return kc8, vc8


def poison_tails(case, kc8, vc8):
    """NaN codes in every slot past a sequence's context in its last block, and
    in the pool's unused blocks: none of them may reach an output."""
    B = case.block_size
    used = set()
    for s in range(case.num_seqs):
        L = int(case.context_lens[s])
        nblk = -(-L // B)
        row = case.block_tables[s, :nblk].tolist()
        used.update(row)
        if L % B:
            blk = row[-1]
            kc8[blk, :, L % B:, :] = NAN_CODE
            vc8[blk, :, :, L % B:] = NAN_CODE
    for blk in range(kc8.shape[0]):
        if blk not in used:
            kc8[blk] = NAN_CODE
            vc8[blk] = NAN_CODE


def gpu_decode_fp8(case, kc8, vc8, ks, vs, query=None):
    q = dev(case.query if query is None else query)
    out = torch.empty_like(q)
    binding.decode_fp8(out, q, dev(kc8), dev(vc8), dev(case.block_tables),
                       dev(case.context_lens), case.scale, int(case.context_lens.max()), ks, vs)
    torch.cuda.synchronize()
    return out


# ------------------------------------------------------------ cache write ----

def special_rows(x, ks):
    """Plant the encoder's edge cases into new rows x [T, Hkv, D] (in place):
    NaN, +-inf, saturation, zeros of both signs, subnormals, exact ties
    between neighbouring codes (scale is a power of two, so x * (1/scale) is
    exact)."""
    vals = oracle.fp8_decode(torch.arange(0x7F, dtype=torch.uint8))  # finite non-negative
    ties = [(vals[c] + vals[c + 1]) / 2 for c in range(0, 0x7E)]
    sp = [float("nan"), float("inf"), -float("inf"), 1e6, -1e6, 448.0, 464.0, 0.0, -0.0,
          2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11, -(2.0 ** -8)] + ties + [-t for t in ties]
    flat = x.view(-1)
    n = min(len(sp), flat.numel())
    flat[:n] = torch.tensor(sp[:n], dtype=torch.float64).mul(ks).to(x.dtype)


@pytest.mark.parametrize("dtype,D,B", [("bf16", 128, 16), ("bf16", 64, 32), ("f32", 64, 16),
                                       ("f32", 128, 32)])
def test_fp8_cache_write_bitexact(dtype, D, B):
    ks, vs = 0.5, 2.0 ** -3
    c = W.random_case(301, dtype, 6, 8, 4, D, B, 1, 200)
    nk, nv = c.new_key.clone(), c.new_value.clone()
    special_rows(nk, ks)
    special_rows(nv, vs)
    slots = c.slot_mapping.clone()
    slots[-1] = -1                                  # padding token: skipped
    kc8, vc8 = fp8_pools(c, ks, vs)
    say("fp8 cache write", dtype, D, B)
    gk, gv = dev(kc8), dev(vc8)
    binding.reshape_and_cache_fp8(dev(nk), dev(nv), gk, gv, dev(slots), ks, vs)
    torch.cuda.synchronize()
    rk, rv = oracle.reshape_and_cache_fp8(nk, nv, kc8, vc8, slots, ks, vs)
    assert torch.equal(gk.cpu(), rk), "K pool differs"
    assert torch.equal(gv.cpu(), rv), "V pool differs"


def test_fp8_cache_write_many_tokens():
    """Every slot of a 40-block pool rewritten (1,280 tokens, non-power-of-two
    scales): bit-exact."""
    c = W.random_case(302, "bf16", 1, 8, 8, 128, 32, 1, 1, write_new=False, extra_blocks=39)
    gen = torch.Generator().manual_seed(303)
    T = c.num_blocks * 32
    nk = torch.randn(T, 8, 128, generator=gen).to(torch.bfloat16)
    nv = (3 * torch.randn(T, 8, 128, generator=gen)).to(torch.bfloat16)
    slots = torch.randperm(T, generator=gen).to(torch.int64)
    ks, vs = 0.0173, 0.0411
    kc8, vc8 = fp8_pools(c, ks, vs)
    say("fp8 cache write, whole pool", T)
    gk, gv = dev(kc8), dev(vc8)
    binding.reshape_and_cache_fp8(dev(nk), dev(nv), gk, gv, dev(slots), ks, vs)
    torch.cuda.synchronize()
    rk, rv = oracle.reshape_and_cache_fp8(nk, nv, kc8, vc8, slots, ks, vs)
    assert torch.equal(gk.cpu(), rk) and torch.equal(gv.cpu(), rv)


# ---------------------------------------------------------------- decode -----

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B", [16, 32])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_fp8_decode_parity_shapes(D, B, G):
    Hkv = 2
    gen = torch.Generator().manual_seed(2000 + D + B + G)
    lens = [0, 1, B - 1, B, B + 1, 64, 65, 257, 700] + \
        [int(x) for x in torch.randint(1, 1100, (3,), generator=gen)]
    c = W.make_case("fp8 shapes", 8, "bf16", Hkv * G, Hkv, D, B, lens, extra_blocks=2)
    ks, vs = 1.0 / 64, 1.0 / 32
    kc8, vc8 = fp8_pools(c, ks, vs)
    poison_tails(c, kc8, vc8)
    ref = oracle.decode_fp8(c.query, kc8, vc8, c.block_tables, c.context_lens, c.scale, ks, vs)
    say("fp8 decode shapes", D, B, G)
    out = gpu_decode_fp8(c, kc8, vc8, ks, vs)
    check_close(out, ref, "bf16", f"fp8 D{D} B{B} G{G}")
    assert (out[0] == 0).all()                      # empty context gives zeros


def test_fp8_decode_sharp_softmax():
    """Queries scaled by 8: nearly one-hot weights, so a wrong token, a wrong
    scale or an unmasked tail shows at full size."""
    c = W.random_case(304, "bf16", 9, 32, 8, 128, 16, 1, 900, write_new=False)
    ks, vs = 0.03, 0.02
    kc8, vc8 = fp8_pools(c, ks, vs)
    poison_tails(c, kc8, vc8)
    q = (c.query.float() * 8).to(torch.bfloat16)
    ref = oracle.decode_fp8(q, kc8, vc8, c.block_tables, c.context_lens, c.scale, ks, vs)
    say("fp8 decode sharp")
    out = gpu_decode_fp8(c, kc8, vc8, ks, vs, query=q)
    check_close(out, ref, "bf16", "fp8 sharp")


def test_fp8_every_code_widens_exactly():
    """One-token contexts return their V row exactly (the weight is 1): with V
    rows holding all 254 finite codes and a power-of-two v_scale, the output
    is each code's value times the scale, bit for bit in bf16."""
    D, B, Hkv, G = 128, 16, 1, 4
    c = W.make_case("fp8 codes", 9, "bf16", G * Hkv, Hkv, D, B, [1, 1], extra_blocks=0)
    ks, vs = 1.0 / 16, 2.0 ** -5
    kc8, vc8 = fp8_pools(c, ks, vs)
    codes = [x for x in range(256) if x not in (0x7F, 0xFF)] + [0, 0]  # 254 codes, 2 rows
    for s in range(2):
        blk = int(c.block_tables[s, 0])
        vc8[blk, 0, :, 0] = torch.tensor(codes[128 * s:128 * (s + 1)], dtype=torch.uint8)
    ref = oracle.decode_fp8(c.query, kc8, vc8, c.block_tables, c.context_lens, c.scale, ks, vs)
    say("fp8 every code")
    out = gpu_decode_fp8(c, kc8, vc8, ks, vs)
    want = torch.from_numpy(ref).to(torch.bfloat16)
    # value equality: code 0x80 (-0) may come back as +0 from the accumulator
    assert torch.equal(out.cpu().float(), want.float())


def test_fp8_decode_after_gpu_cache_write():
    """The step as a caller runs it: the quantising write of each sequence's new
    token at L - 1, then decode over the written pools."""
    c = W.random_case(305, "bf16", 12, 32, 8, 128, 16, 1, 1500)
    ks, vs = 0.05, 0.04
    kc8, vc8 = fp8_pools(c, ks, vs)
    say("fp8 write then decode")
    gk, gv = dev(kc8), dev(vc8)
    binding.reshape_and_cache_fp8(dev(c.new_key), dev(c.new_value), gk, gv, dev(c.slot_mapping),
                                  ks, vs)
    q = dev(c.query)
    out = torch.empty_like(q)
    binding.decode_fp8(out, q, gk, gv, dev(c.block_tables), dev(c.context_lens), c.scale,
                       int(c.context_lens.max()), ks, vs)
    torch.cuda.synchronize()
    rk, rv = oracle.reshape_and_cache_fp8(c.new_key, c.new_value, kc8, vc8, c.slot_mapping, ks, vs)
    assert torch.equal(gk.cpu(), rk) and torch.equal(gv.cpu(), rv)
    ref = oracle.decode_fp8(c.query, rk, rv, c.block_tables, c.context_lens, c.scale, ks, vs)
    check_close(out, ref, "bf16", "fp8 write + decode")


def test_fp8_decode_llama8b_shape():
    """The Llama-3-8B-shaped batch (64 seqs, 32 q / 8 kv heads, d 128, B 16,
    L ~ U{512..4096}) over seeded random FP8 pools, in the launch the
    benchmark times; every output row checked against the oracle."""
    c = W.llama8b_decode()
    kc8 = W.random_fp8_codes(306, (c.num_blocks, 8, 16, 128))
    vc8 = W.random_fp8_codes(307, (c.num_blocks, 8, 128, 16))
    ks, vs = 1.0 / 8, 1.0 / 4
    say("fp8 decode llama8b shape")
    out = gpu_decode_fp8(c, kc8, vc8, ks, vs)
    ref = oracle.decode_fp8(c.query, kc8, vc8, c.block_tables, c.context_lens, c.scale, ks, vs)
    check_close(out, ref, "bf16", "fp8 llama8b")


def test_fp8_decode_long_context_full_size():
    """The 70B-shaped long-context batch at full size (8 seqs x 32,768 tokens,
    64 q / 8 kv heads, d 128, B 32, the pool permuted) over seeded random FP8
    pools, in the launch the benchmark times; every output element checked
    against the oracle's fp64 decode over the same codes."""
    c = W.long_context_decode()
    NB = c.key_cache.shape[0]
    kc8 = W.random_fp8_codes(311, (NB, 8, 32, 128))
    vc8 = W.random_fp8_codes(312, (NB, 8, 128, 32))
    ks, vs = 1.0 / 16, 1.0 / 8
    say("fp8 decode long context full size")
    out = gpu_decode_fp8(c, kc8, vc8, ks, vs)
    ref = oracle.decode_fp8(c.query, kc8, vc8, c.block_tables, c.context_lens, c.scale, ks, vs)
    check_close(out, ref, "bf16", "fp8 long context")


def test_fp8_decode_prefix_sharing_full_size():
    """The prefix-sharing batch at full size (128 seqs whose tables share one
    1,024-token prefix of 64 physical blocks, suffixes U{256..2048}) over
    seeded random FP8 pools with NaN codes past every context; every output
    element checked against the oracle."""
    c = W.prefix_sharing_decode()
    NB = c.key_cache.shape[0]
    kc8 = W.random_fp8_codes(313, (NB, 8, 16, 128))
    vc8 = W.random_fp8_codes(314, (NB, 8, 128, 16))
    poison_tails(c, kc8, vc8)
    ks, vs = 1.0 / 8, 1.0 / 4
    say("fp8 decode prefix sharing full size")
    out = gpu_decode_fp8(c, kc8, vc8, ks, vs)
    ref = oracle.decode_fp8(c.query, kc8, vc8, c.block_tables, c.context_lens, c.scale, ks, vs)
    check_close(out, ref, "bf16", "fp8 prefix sharing")


# --------------------------------------------------------------- prefill -----

def gpu_prefill_fp8(c, kc8, vc8, ks, vs):
    q = dev(c.chunk_query)
    out = torch.empty_like(q)
    cu = c.chunk_cu_query_lens
    maxq = int((cu[1:] - cu[:-1]).max())
    binding.prefill_chunk_fp8(out, q, dev(kc8), dev(vc8), dev(c.chunk_block_tables), dev(cu),
                              dev(c.chunk_context_lens), c.scale, maxq, ks, vs)
    torch.cuda.synchronize()
    return out


def poison_chunk_tails(c, kc8, vc8):
    """NaN codes past each chunk's context in its last page, and in every page
    no chunk uses."""
    B = c.block_size
    used = set()
    for k in range(c.num_chunks):
        L = int(c.chunk_context_lens[k])
        row = c.chunk_block_tables[k, :-(-L // B)].tolist()
        used.update(row)
        if L % B:
            kc8[row[-1], :, L % B:, :] = NAN_CODE
            vc8[row[-1], :, :, L % B:] = NAN_CODE
    for s in range(c.num_seqs):
        used.update(c.block_tables[s, :-(-int(c.context_lens[s]) // B)].tolist())
    for blk in range(kc8.shape[0]):
        if blk not in used:
            kc8[blk] = NAN_CODE
            vc8[blk] = NAN_CODE


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B", [16, 32])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_fp8_prefill_parity_shapes(D, B, G):
    """Ragged chunks (1 to 200 queries; contexts from one key to several tiles
    of keys, ending inside a block) against the oracle, with NaN codes past
    every context."""
    chunks = [(7, 40), (130, 300), (64, 64), (1, 17), (200, 777)]
    c = W.make_case("pf8", 27 + D + B + G, "bf16", 2 * G, 2, D, B, [5], new_positions=[4],
                    chunks=chunks, extra_blocks=3)
    ks, vs = 1.0 / 64, 1.0 / 32
    kc8, vc8 = fp8_pools(c, ks, vs)
    poison_chunk_tails(c, kc8, vc8)
    say("fp8 prefill shapes", D, B, G)
    out = gpu_prefill_fp8(c, kc8, vc8, ks, vs)
    ref = oracle.prefill_fp8(c.chunk_query, kc8, vc8, c.chunk_block_tables, c.chunk_cu_query_lens,
                             c.chunk_context_lens, c.scale, ks, vs)
    check_close(out, ref, "bf16", f"fp8 prefill D{D} B{B} G{G}")


def test_fp8_prefill_empty_long_and_many_chunks():
    """An empty chunk, a 2,048-query chunk over 6,000 keys, a one-key context
    and 40 small ragged chunks in one launch, NaN codes past every context."""
    chunks = [(3, 10), (0, 50), (2048, 6000), (1, 1)] + \
        [(k % 37 + 1, 100 + 13 * k) for k in range(40)]
    c = W.make_case("pf8 edge", 78, "bf16", 8, 2, 128, 16, [5], new_positions=[4],
                    chunks=chunks, extra_blocks=3)
    ks, vs = 1.0 / 64, 1.0 / 32
    kc8, vc8 = fp8_pools(c, ks, vs)
    poison_chunk_tails(c, kc8, vc8)
    say("fp8 prefill empty, long and many chunks")
    out = gpu_prefill_fp8(c, kc8, vc8, ks, vs)
    ref = oracle.prefill_fp8(c.chunk_query, kc8, vc8, c.chunk_block_tables, c.chunk_cu_query_lens,
                             c.chunk_context_lens, c.scale, ks, vs)
    check_close(out, ref, "bf16", "fp8 prefill edge chunks")


@pytest.mark.parametrize("B", [16, 32])
def test_fp8_prefill_context_beyond_the_table_window(B):
    """A chunk over a 40,000-token context in FP8 pools (seeded random codes):
    at 16-token blocks its tiles read 2,500 pages, more than the 2,048
    block-table entries the FP8 prefill keeps in LDS, so the kernel refills
    that window mid-way (at 32-token blocks it does not: the control case)."""
    c = W.make_case("pf8_long", 191 + B, "bf16", 8, 2, 128, B, [3], new_positions=[2],
                    chunks=[(64, 40000)], extra_blocks=2)
    NB = c.key_cache.shape[0]
    kc8 = W.random_fp8_codes(411 + B, (NB, 2, B, 128))
    vc8 = W.random_fp8_codes(412 + B, (NB, 2, 128, B))
    ks, vs = 1.0 / 16, 1.0 / 8
    say("fp8 prefill long context", B)
    out = gpu_prefill_fp8(c, kc8, vc8, ks, vs)
    ref = oracle.prefill_fp8(c.chunk_query, kc8, vc8, c.chunk_block_tables, c.chunk_cu_query_lens,
                             c.chunk_context_lens, c.scale, ks, vs)
    check_close(out, ref, "bf16", f"fp8 prefill 40K context B{B}")


def test_fp8_prefill_mixed_workload():
    """The mixed chunked-prefill shape (2 chunks of 512 queries over 2,048 prior
    tokens, 32 q / 8 kv heads, d 128, B 16): the chunks' own tokens are written
    by the FP8 cache write first, as a caller would, then prefill.  Every
    output element of every query row is checked against the oracle's fp64
    prefill over the oracle-written pools."""
    c = W.mixed_chunked_prefill()
    ks, vs = 0.05, 0.04
    kc8, vc8 = fp8_pools(c, ks, vs)
    say("fp8 prefill mixed workload")
    gk, gv = dev(kc8), dev(vc8)
    binding.reshape_and_cache_fp8(dev(c.new_key), dev(c.new_value), gk, gv, dev(c.slot_mapping),
                                  ks, vs)
    q = dev(c.chunk_query)
    out = torch.empty_like(q)
    cu = c.chunk_cu_query_lens
    binding.prefill_chunk_fp8(out, q, gk, gv, dev(c.chunk_block_tables), dev(cu),
                              dev(c.chunk_context_lens), c.scale, 512, ks, vs)
    torch.cuda.synchronize()
    rk, rv = oracle.reshape_and_cache_fp8(c.new_key, c.new_value, kc8, vc8, c.slot_mapping, ks, vs)
    assert torch.equal(gk.cpu(), rk) and torch.equal(gv.cpu(), rv)
    ref = oracle.prefill_fp8(c.chunk_query, rk, rv, c.chunk_block_tables, cu,
                             c.chunk_context_lens, c.scale, ks, vs)
    assert out.shape[0] == ref.shape[0] == 1024
    check_close(out, ref, "bf16", "fp8 mixed prefill")


# ------------------------------------------------------------- invariants ----

def _gpu_fp8_decode_bt(c, kc8, vc8, bt, ks, vs):
    q = dev(c.query)
    out = torch.empty_like(q)
    binding.decode_fp8(out, q, dev(kc8), dev(vc8), dev(bt), dev(c.context_lens), c.scale,
                       int(c.context_lens.max()), ks, vs)
    torch.cuda.synchronize()
    return out


def test_fp8_block_relabelling_invariance():
    """Moving every physical block and its table entries gives a bit-identical
    FP8 decode: the arithmetic follows logical positions only."""
    c = W.random_case(308, "bf16", 6, 32, 8, 128, 16, 300, 2000, write_new=False)
    ks, vs = 0.03, 0.05
    kc8, vc8 = fp8_pools(c, ks, vs)
    say("fp8 relabelling invariance")
    a = _gpu_fp8_decode_bt(c, kc8, vc8, c.block_tables, ks, vs)
    pi = torch.randperm(c.num_blocks, generator=torch.Generator().manual_seed(4))
    k2 = torch.empty_like(kc8); k2[pi] = kc8
    v2 = torch.empty_like(vc8); v2[pi] = vc8
    b = _gpu_fp8_decode_bt(c, k2, v2, pi[c.block_tables.long()].to(torch.int32), ks, vs)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_fp8_shared_prefix_invariance():
    """Prefix blocks shared by every table (reference count 12) give the same
    bits as private copies of them, and match the oracle."""
    c = W.prefix_sharing_decode(num_seqs=12)
    ks, vs = 0.04, 0.04
    kc8, vc8 = fp8_pools(c, ks, vs)
    say("fp8 shared prefix invariance")
    a = _gpu_fp8_decode_bt(c, kc8, vc8, c.block_tables, ks, vs)
    shared = c.shared_blocks.long()
    n, NB, S = len(shared), c.num_blocks, c.num_seqs
    k2 = torch.cat([kc8] + [kc8[shared]] * S)
    v2 = torch.cat([vc8] + [vc8[shared]] * S)
    bt = c.block_tables.clone()
    for s in range(S):
        bt[s, :n] = torch.arange(NB + s * n, NB + (s + 1) * n, dtype=torch.int32)
    b = _gpu_fp8_decode_bt(c, k2, v2, bt, ks, vs)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref = oracle.decode_fp8(c.query, kc8, vc8, c.block_tables, c.context_lens, c.scale, ks, vs)
    check_close(a, ref, "bf16", "fp8 prefix vs oracle")


def test_fp8_decode_deterministic():
    c = W.llama8b_decode(num_seqs=16)
    kc8 = W.random_fp8_codes(309, (c.num_blocks, 8, 16, 128))
    vc8 = W.random_fp8_codes(310, (c.num_blocks, 8, 128, 16))
    say("fp8 determinism")
    a = _gpu_fp8_decode_bt(c, kc8, vc8, c.block_tables, 0.125, 0.25)
    b = _gpu_fp8_decode_bt(c, kc8, vc8, c.block_tables, 0.125, 0.25)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_fp8_decode_phases_equal_decode():
    """pa_decode_fp8_partitions then pa_decode_reduce gives pa_decode_fp8's
    output bit for bit, on ragged lengths from empty to many pairs per wave."""
    lens = [0, 1, 15, 16, 17, 300, 4097, 33] + [int(x) for x in torch.randint(
        1, 2000, (24,), generator=torch.Generator().manual_seed(12))]
    c = W.make_case("fp8 phases", 313, "bf16", 16, 4, 128, 16, lens, extra_blocks=2)
    ks, vs = 0.05, 0.05
    kc8, vc8 = fp8_pools(c, ks, vs)
    poison_tails(c, kc8, vc8)
    say("fp8 decode phases")
    a = gpu_decode_fp8(c, kc8, vc8, ks, vs)
    q, gk, gv = dev(c.query), dev(kc8), dev(vc8)
    b = torch.full_like(q, float("nan"))
    maxL = int(c.context_lens.max())
    bt, ln = dev(c.block_tables), dev(c.context_lens)
    ws = binding.make_fp8_workspace(q, gk, maxL)
    binding.decode_fp8_partitions(b, q, gk, gv, bt, ln, c.scale, maxL, ks, vs, ws)
    binding.decode_reduce(b, ln, c.num_kv_heads, c.block_size, c.block_tables.shape[1], maxL, 0,
                          ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref = oracle.decode_fp8(c.query, kc8, vc8, c.block_tables, c.context_lens, c.scale, ks, vs)
    check_close(a, ref, "bf16", "fp8 phases vs oracle")


# ------------------------------------------------ decode with append (fused) --

def _fp8_append_vs_oracle(c, ks, vs, kc8, vc8, split=False):
    """Fused FP8 step on the GPU; the pools must equal the oracle's FP8 cache
    write of each sequence's new token at L - 1, the output the oracle decode
    over them.  Returns (out, gpu pools)."""
    from tests.test_append_gpu import per_sequence_rows
    nk, nv = per_sequence_rows(c)
    gk, gv = dev(kc8), dev(vc8)
    q = dev(c.query)
    out = torch.empty_like(q)
    maxL = max(1, int(c.context_lens.max()))
    bt, lens = dev(c.block_tables), dev(c.context_lens)
    if split:
        ws = binding.make_fp8_workspace(q, gk, maxL)
        binding.decode_fp8_append_partitions(out, q, dev(nk), dev(nv), gk, gv, bt, lens, c.scale,
                                             maxL, ks, vs, ws)
        binding.decode_reduce(out, lens, c.num_kv_heads, c.block_size, c.block_tables.shape[1],
                              maxL, 0, ws)
    else:
        binding.decode_fp8_append(out, q, dev(nk), dev(nv), gk, gv, bt, lens, c.scale, maxL, ks,
                                  vs)
    torch.cuda.synchronize()
    rk, rv = oracle.reshape_and_cache_fp8(c.new_key, c.new_value, kc8, vc8, c.slot_mapping, ks, vs)
    assert torch.equal(gk.cpu(), rk), "K pool"
    assert torch.equal(gv.cpu(), rv), "V pool"
    ref = oracle.decode_fp8(c.query, rk, rv, c.block_tables, c.context_lens, c.scale, ks, vs)
    check_close(out, ref, "bf16", "fp8 append")
    return out


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B", [16, 32])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_fp8_append_parity_shapes(D, B, G):
    Hkv = 2
    gen = torch.Generator().manual_seed(3000 + D + B + G)
    lens = [0, 1, B - 1, B, B + 1, 16, 17, 64, 65, 257, 700] + \
        [int(x) for x in torch.randint(1, 1100, (3,), generator=gen)]
    c = W.make_case("fp8 append", 12, "bf16", Hkv * G, Hkv, D, B, lens,
                    new_positions=[L - 1 if L else None for L in lens], extra_blocks=2)
    ks, vs = 1.0 / 64, 0.021
    kc8, vc8 = fp8_pools(c, ks, vs)
    say("fp8 append shapes", D, B, G)
    out = _fp8_append_vs_oracle(c, ks, vs, kc8, vc8)
    assert (out[0] == 0).all()                      # empty context: zeros, nothing written


def test_fp8_decode_at_max_balanced_batch():
    """8192 sequences, the largest batch the FP8 decode takes."""
    c = W.random_case(312, "bf16", 8192, 8, 2, 128, 16, 1, 40, write_new=False)
    ks, vs = 0.05, 0.05
    kc8, vc8 = fp8_pools(c, ks, vs)
    poison_tails(c, kc8, vc8)
    ref = oracle.decode_fp8(c.query, kc8, vc8, c.block_tables, c.context_lens, c.scale, ks, vs)
    say("fp8 decode 8192 seqs")
    out = gpu_decode_fp8(c, kc8, vc8, ks, vs)
    check_close(out, ref, "bf16", "fp8 8192 seqs")


def test_fp8_append_many_short_sequences():
    """Hundreds of 1..40-token sequences: several new rows per 64-unit chunk."""
    c = W.random_case(311, "bf16", 300, 8, 2, 128, 16, 1, 40, extra_blocks=5)
    ks, vs = 0.05, 0.05
    kc8, vc8 = fp8_pools(c, ks, vs)
    say("fp8 append short sequences")
    _fp8_append_vs_oracle(c, ks, vs, kc8, vc8)


def test_fp8_append_llama8b_matches_unfused_bitwise():
    """The Llama-3-8B-shaped FP8 step: the fused step (one call, and its two
    phases) equals pa_reshape_and_cache_fp8 + pa_decode_fp8 bit for bit."""
    c = W.llama8b_decode()
    kc8 = W.random_fp8_codes(312, (c.num_blocks, 8, 16, 128))
    vc8 = W.random_fp8_codes(313, (c.num_blocks, 8, 128, 16))
    ks, vs = 1.0 / 8, 1.0 / 4
    say("fp8 append llama8b")
    fused = _fp8_append_vs_oracle(c, ks, vs, kc8, vc8)
    split = _fp8_append_vs_oracle(c, ks, vs, kc8, vc8, split=True)
    gk, gv = dev(kc8), dev(vc8)
    binding.reshape_and_cache_fp8(dev(c.new_key), dev(c.new_value), gk, gv, dev(c.slot_mapping),
                                  ks, vs)
    q = dev(c.query)
    ref = torch.empty_like(q)
    binding.decode_fp8(ref, q, gk, gv, dev(c.block_tables), dev(c.context_lens), c.scale,
                       int(c.context_lens.max()), ks, vs)
    torch.cuda.synchronize()
    assert torch.equal(fused.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(split.view(torch.int16), ref.view(torch.int16))


def test_fp8_encoder_every_bf16_pattern():
    """All 65,536 bf16 bit patterns (NaNs, infinities, subnormals, both zeros)
    written through the FP8 cache write: every code equals the oracle's, at a
    power-of-two scale (x / scale exact) and at a general one."""
    T, Hkv, D, B = 64, 8, 128, 16
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    rows = bits.view(torch.bfloat16).reshape(T, Hkv, D)
    rows_v = rows.flip(0).contiguous()               # V gets the patterns in another order
    NB = T // B
    slots = torch.arange(T, dtype=torch.int64)
    for ks, vs in ((1.0, 0.25), (0.0371, 3.3)):
        kc8 = torch.full((NB, Hkv, B, D), 0x55, dtype=torch.uint8)
        vc8 = torch.full((NB, Hkv, D, B), 0x55, dtype=torch.uint8)
        say("fp8 encoder, every bf16 pattern, scales", ks, vs)
        gk, gv = dev(kc8), dev(vc8)
        binding.reshape_and_cache_fp8(dev(rows), dev(rows_v), gk, gv, dev(slots), ks, vs)
        torch.cuda.synchronize()
        rk, rv = oracle.reshape_and_cache_fp8(rows, rows_v, kc8, vc8, slots, ks, vs)
        assert torch.equal(gk.cpu(), rk), "K codes differ"
        assert torch.equal(gv.cpu(), rv), "V codes differ"


@pytest.mark.parametrize("dtype,B", [("bf16", 16), ("bf16", 32), ("f32", 16), ("f32", 32)])
def test_fp8_cache_write_runs_of_consecutive_slots(dtype, B):
    """A chunk's 300 new tokens at consecutive positions starting inside a
    block (groups of 16 that lie in one block take whole-row V stores, the
    others per-token writes), with a padding token and a foreign slot in the
    middle: bit-exact against the oracle."""
    c = W.make_case("fp8 runs", 314, dtype, 8, 4, 128, B, [1], chunks=[(300, 313)],
                    extra_blocks=2)
    slots = c.slot_mapping.clone()
    slots = slots[-300:].clone()                      # the chunk's own positions 13 .. 312
    nk, nv = c.new_key[-300:].contiguous(), c.new_value[-300:].contiguous()
    slots[100] = -1                                   # padding
    slots[200] = int(c.block_tables[0, 0]) * B        # the decode sequence's slot
    ks, vs = 0.05, 1.0 / 16
    kc8, vc8 = fp8_pools(c, ks, vs)
    say("fp8 cache write runs", dtype, B)
    gk, gv = dev(kc8), dev(vc8)
    binding.reshape_and_cache_fp8(dev(nk), dev(nv), gk, gv, dev(slots), ks, vs)
    torch.cuda.synchronize()
    rk, rv = oracle.reshape_and_cache_fp8(nk, nv, kc8, vc8, slots, ks, vs)
    assert torch.equal(gk.cpu(), rk), "K pool differs"
    assert torch.equal(gv.cpu(), rv), "V pool differs"


@pytest.mark.parametrize("dtype,B", [("bf16", 16), ("bf16", 32), ("f32", 16), ("f32", 32)])
def test_fp8_cache_write_whole_row_groups(dtype, B):
    """A chunk's 317 new tokens at positions 16 .. 332, so groups of 16
    consecutive tokens start at 16-aligned slots and take the whole-row path;
    one group has a padding token, one a foreign slot, one two of its slots
    swapped (all three fall back to per-token writes), and the last group is
    partial: bit-exact against the oracle."""
    c = W.make_case("fp8 groups", 315, dtype, 8, 4, 128, B, [1], chunks=[(317, 333)],
                    extra_blocks=2)
    slots = c.slot_mapping[-317:].clone()             # the chunk's own positions 16 .. 332
    nk, nv = c.new_key[-317:].contiguous(), c.new_value[-317:].contiguous()
    assert int(slots[0]) % 16 == 0
    slots[37] = -1                                    # padding inside group 2
    slots[70] = int(c.block_tables[0, 0]) * B         # the decode sequence's slot, group 4
    a, b = int(slots[90]), int(slots[91])             # group 5: two slots swapped
    slots[90], slots[91] = b, a
    ks, vs = 0.05, 1.0 / 16
    kc8, vc8 = fp8_pools(c, ks, vs)
    say("fp8 cache write whole-row groups", dtype, B)
    gk, gv = dev(kc8), dev(vc8)
    binding.reshape_and_cache_fp8(dev(nk), dev(nv), gk, gv, dev(slots), ks, vs)
    torch.cuda.synchronize()
    rk, rv = oracle.reshape_and_cache_fp8(nk, nv, kc8, vc8, slots, ks, vs)
    assert torch.equal(gk.cpu(), rk), "K pool differs"
    assert torch.equal(gv.cpu(), rv), "V pool differs"


def test_fp8_block_manager_drives_decode():
    """The host block manager drives FP8 decode steps: prompts sharing a system
    prefix (reused through the prefix cache), a fork whose first write copies
    the shared partial block (pa_copy_blocks on the FP8 pools), and each step's
    new tokens quantised inside the decode pass (pa_decode_fp8_append).  Every
    step's output must match the oracle over each sequence's logical rows."""
    import random
    from tests.test_block_manager_gpu import B as BB, D as DD, Hkv as HK, Hq as HQ, NB as NBB, kv_rows
    ks, vs = 0.03, 0.03
    rnd = random.Random(6)
    bm = binding.BlockManager(NBB, BB, prefix_cache=True)
    kc = torch.zeros((NBB, HK, BB, DD), dtype=torch.uint8, device="cuda")
    vc = torch.zeros((NBB, HK, DD, BB), dtype=torch.uint8, device="cuda")
    tokens = {}
    system = [rnd.randint(0, 50) for _ in range(2 * BB + 3)]
    for s in range(3):
        prompt = system + [rnd.randint(0, 50) for _ in range(rnd.randint(0, 30))]
        slots, cached = bm.add_sequence(s, prompt)
        tokens[s] = prompt
        keep = [(sl, kv_rows(prompt[:t + 1])) for t, sl in enumerate(slots) if sl >= 0]
        if keep:
            k = torch.stack([r[0] for _, r in keep]).cuda()
            v = torch.stack([r[1] for _, r in keep]).cuda()
            binding.reshape_and_cache_fp8(k, v, kc, vc,
                                          torch.tensor([a for a, _ in keep], dtype=torch.int64).cuda(),
                                          ks, vs)
    for step in range(4):
        if step == 1:
            bm.fork(0, 3)
            tokens[3] = list(tokens[0])
        seqs = sorted(tokens)
        rows = []
        for s in seqs:
            tok = rnd.randint(0, 50)
            tokens[s].append(tok)
            bm.append(s, tok)            # the slot is the table's position L - 1
            rows.append(kv_rows(tokens[s]))
        copies = bm.take_copies()
        if copies:
            binding.copy_blocks(kc, vc, kc, vc, torch.tensor(copies, dtype=torch.int64).cuda())
        tabs = [bm.block_table(s) for s in seqs]
        width = max(len(t) for t, _ in tabs)
        bt = torch.zeros((len(seqs), width), dtype=torch.int32)
        for i, (t, _) in enumerate(tabs):
            bt[i, :len(t)] = torch.tensor(t, dtype=torch.int32)
        lens = torch.tensor([L for _, L in tabs], dtype=torch.int32)
        nk = torch.stack([r[0] for r in rows]).cuda()
        nv = torch.stack([r[1] for r in rows]).cuda()
        q = torch.randn((len(seqs), HQ, DD)).to(torch.bfloat16)
        out = torch.empty((len(seqs), HQ, DD), dtype=torch.bfloat16, device="cuda")
        say("fp8 block manager step", step, "copies", len(copies))
        binding.decode_fp8_append(out, q.cuda(), nk, nv, kc, vc, bt.cuda(), lens.cuda(), DD ** -0.5,
                                  int(lens.max()), ks, vs)
        torch.cuda.synchronize()
        # reference: each sequence's logical rows, encoded by the oracle, laid out contiguously
        maxL = int(lens.max())
        nbl = -(-maxL // BB)
        rk = torch.zeros((len(seqs) * nbl, HK, BB, DD), dtype=torch.bfloat16)
        rv = torch.zeros_like(rk)
        rbt = torch.zeros((len(seqs), nbl), dtype=torch.int32)
        for i, s in enumerate(seqs):
            for t in range(len(tokens[s])):
                k, v = kv_rows(tokens[s][:t + 1])
                rk[i * nbl + t // BB, :, t % BB] = k
                rv[i * nbl + t // BB, :, t % BB] = v
            rbt[i] = torch.arange(i * nbl, (i + 1) * nbl, dtype=torch.int32)
        rk8 = oracle.fp8_encode(rk.float(), ks)
        rv8 = oracle.fp8_encode(rv.float(), vs).permute(0, 1, 3, 2).contiguous()
        ref = oracle.decode_fp8(q, rk8, rv8, rbt, lens, DD ** -0.5, ks, vs)
        check_close(out, ref, "bf16", f"fp8 block manager step {step}")
    bm.close()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fp8_scale_reading_separating_values(dtype):
    """Values whose code differs between x * fp32(1 / scale) (the library's
    reading) and x / scale: 0.00439453125 at scale 0.3 -> 0x08 and
    0.02490234375 at scale 1.7 -> 0x07 (the quotient gives 0x07 and 0x08).
    Written through pa_reshape_and_cache_fp8 and through the fused FP8 decode
    step, bit-exact against the oracle and against those codes."""
    T, Hkv, D, B = 4, 2, 64, 16
    x = torch.tensor([0.00439453125, 0.02490234375])
    for (ks, vs), (xk, xv), (ck, cv) in (((0.3, 1.7), (x[0], x[1]), (0x08, 0x07)),
                                         ((1.7, 0.3), (x[1], x[0]), (0x07, 0x08))):
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        key = torch.full((T, Hkv, D), float(xk)).to(tdt)
        val = torch.full((T, Hkv, D), float(xv)).to(tdt)
        key[1::2] = -key[1::2]
        val[1::2] = -val[1::2]
        kc8 = torch.full((2, Hkv, B, D), 0x55, dtype=torch.uint8)
        vc8 = torch.full((2, Hkv, D, B), 0x55, dtype=torch.uint8)
        slots = torch.tensor([0, 5, 16, 31], dtype=torch.int64)
        say("fp8 scale reading, cache write", dtype, ks, vs)
        gk, gv = dev(kc8), dev(vc8)
        binding.reshape_and_cache_fp8(dev(key), dev(val), gk, gv, dev(slots), ks, vs)
        torch.cuda.synchronize()
        rk, rv = oracle.reshape_and_cache_fp8(key, val, kc8, vc8, slots, ks, vs)
        assert torch.equal(gk.cpu(), rk) and torch.equal(gv.cpu(), rv)
        assert int(rk[0, 0, 0, 0]) == ck and int(rk[0, 0, 5, 0]) == 0x80 | ck
        assert int(rv[1, 1, 3, 0]) == cv and int(rv[1, 1, 3, 15]) == 0x80 | cv
    # the fused write of a decode step takes the same reading
    c = W.make_case("fp8 scale reading", 316, "bf16", 8, 2, 64, 16, [5, 17, 40],
                    new_positions=[4, 16, 39], extra_blocks=1)
    c.new_key[:] = float(x[0])
    c.new_value[:] = float(x[1])
    c.new_key[1] = -c.new_key[1]
    kc8, vc8 = fp8_pools(c, 0.3, 1.7)
    say("fp8 scale reading, fused decode write")
    _fp8_append_vs_oracle(c, 0.3, 1.7, kc8, vc8)
