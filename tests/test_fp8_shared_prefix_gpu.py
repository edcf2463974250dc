"""GPU parity of pa_decode_fp8_shared_prefix, through the C ABI.

The shared-prefix decode over e4m3 pools must give pa_decode_fp8's result
(within the bf16 tolerance of the fp64 oracle, which decodes every sequence's
own table): all head dims, block sizes and head groupings; ragged column
groups; empty suffixes; a sequence shorter than the prefix and a zero-length
one; NaN codes in every pool slot no sequence may read; prefix_blocks 0 (the
plain FP8 decode, bit for bit); a prefix named shorter than the shared
blocks; and the full-size prefix-sharing batch.
"""
import pytest
import torch

import oracle
from paged_kv_cache_262_amd import binding
from paged_kv_cache_262_amd import workloads as W
from tests.gpu_util import check_close, dev, say
from tests.test_fp8_gpu import NAN_CODE, fp8_pools
from tests.test_shared_prefix_gpu import shared_case

pytestmark = pytest.mark.gpu

KS, VS = 1.0 / 64, 1.0 / 32


def poison_codes(c, lens, kc8, vc8):
    """NaN codes in every slot no sequence reads (K [blk, h, token, :],
    V [blk, h, :, token])."""
    B = c.block_size
    reach = {}
    for s in range(c.num_seqs):
        L = int(lens[s])
        for j in range(-(-L // B)):
            blk = int(c.block_tables[s, j])
            reach[blk] = max(reach.get(blk, 0), min(B, L - j * B))
    for blk in range(kc8.shape[0]):
        r = reach.get(blk, 0)
        kc8[blk, :, r:, :] = NAN_CODE
        vc8[blk, :, :, r:] = NAN_CODE


def run(c, lens, kc8, vc8, prefix_blocks=None, workspace=None):
    q = dev(c.query)
    out = torch.empty_like(q)
    if prefix_blocks is None:
        binding.decode_fp8(out, q, dev(kc8), dev(vc8), dev(c.block_tables), dev(lens), c.scale,
                           int(lens.max()), KS, VS)
    else:
        binding.decode_fp8_shared_prefix(out, q, dev(kc8), dev(vc8), dev(c.block_tables),
                                         dev(lens), c.scale, int(lens.max()), prefix_blocks, KS,
                                         VS, workspace=workspace)
    torch.cuda.synchronize()
    return out


def ref(c, lens, kc8, vc8):
    return oracle.decode_fp8(c.query, kc8, vc8, c.block_tables, lens, c.scale, KS, VS)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B", [16, 32])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_fp8_shared_prefix_parity_shapes(D, B, G):
    """Seven sequences over a 3-block prefix, suffixes of 0 to 250 tokens;
    sequence 2 cut to 5 tokens short of the prefix, sequence 5 to length 0."""
    c = shared_case(1700 + D + B + G, D, B, G, 3, [0, 1, 5, 17, 40, 100, 250])
    lens = c.context_lens.clone()
    lens[2] = 3 * B - 5
    lens[5] = 0
    kc8, vc8 = fp8_pools(c, KS, VS)
    poison_codes(c, lens, kc8, vc8)
    say("fp8 shared prefix shapes", D, B, G)
    out = run(c, lens, kc8, vc8, 3)
    check_close(out, ref(c, lens, kc8, vc8), "bf16", f"fp8 shared prefix D{D} B{B} G{G}")


def test_fp8_shared_prefix_only_prefix_and_many_groups():
    """Every sequence exactly the prefix long, 37 sequences, a 40-block prefix."""
    c = shared_case(1731, 128, 16, 4, 40, [0] * 37, Hkv=8)
    kc8, vc8 = fp8_pools(c, KS, VS)
    poison_codes(c, c.context_lens, kc8, vc8)
    say("fp8 shared prefix only")
    out = run(c, c.context_lens, kc8, vc8, 40)
    check_close(out, ref(c, c.context_lens, kc8, vc8), "bf16", "fp8 prefix only")


def test_fp8_shared_prefix_zero_blocks_is_plain_decode():
    """prefix_blocks 0 runs the plain FP8 balanced decode, bit for bit."""
    c = shared_case(1732, 128, 16, 4, 2, [3, 70, 500, 1200, 9], Hkv=8)
    kc8, vc8 = fp8_pools(c, KS, VS)
    say("fp8 shared prefix, zero blocks")
    a = run(c, c.context_lens, kc8, vc8, 0)
    b = run(c, c.context_lens, kc8, vc8)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_fp8_shared_prefix_fewer_blocks_than_shared():
    """A prefix named shorter than the shared blocks: the rest are read per
    sequence by the suffix pass (32-token blocks, G 8)."""
    c = shared_case(1733, 128, 32, 8, 6, [10, 300, 31, 2000], Hkv=8)
    kc8, vc8 = fp8_pools(c, KS, VS)
    poison_codes(c, c.context_lens, kc8, vc8)
    say("fp8 shared prefix, 4 of 6 shared blocks")
    out = run(c, c.context_lens, kc8, vc8, 4)
    check_close(out, ref(c, c.context_lens, kc8, vc8), "bf16", "fp8 partial prefix")


def test_fp8_shared_prefix_full_size_batch():
    """The prefix-sharing batch at full size (128 sequences, a 1,024-token
    prefix, suffixes U{256..2048}, 32 q / 8 kv heads, d 128, B 16) with its
    pools quantised: every output element against the oracle and against
    pa_decode_fp8; and two calls give the same bits."""
    c = W.prefix_sharing_decode()
    kc8, vc8 = fp8_pools(c, KS, VS)
    say("fp8 shared prefix full size")
    ws = binding.make_shared_prefix_workspace(dev(c.query), kc8[:1],
                                              int(c.context_lens.max()), 64)
    out = run(c, c.context_lens, kc8, vc8, 64, workspace=ws)
    r = ref(c, c.context_lens, kc8, vc8)
    check_close(out, r, "bf16", "fp8 shared prefix full size")
    plain = run(c, c.context_lens, kc8, vc8)
    check_close(plain, r, "bf16", "pa_decode_fp8 full size")
    again = run(c, c.context_lens, kc8, vc8, 64, workspace=ws)
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))
