"""GPU parity of the balanced decode's one-wave-per-pair mode, through the C ABI.

A small batch of short contexts (at most 1,024 (sequence, kv head) pairs, no
context longer than 8 units of 16 tokens) runs with one wave per pair: every
pair is finished by its own wave in the decode launch and no reduce runs.
Checked against the fp64 oracle: fp32, bf16 and FP8 pools; head dims 64 and
128; 16- and 32-token blocks; every head grouping; empty sequences (zero
rows, which the reduce writes in the equal split); the decode with its new
tokens written inside the pass; the two-call API, whose reduce call must
leave the output as the decode wrote it; and the batches on both sides of the
1,024-pair bound, where the equal split takes over.
"""
import pytest
import torch

import oracle
from paged_kv_cache_262_amd import binding
from paged_kv_cache_262_amd import workloads as W
from tests.gpu_util import check_close, dev, oracle_decode, say
from tests.test_append_gpu import check_case
from tests.test_fp8_gpu import fp8_pools, gpu_decode_fp8

pytestmark = pytest.mark.gpu

LENS = [0, 1, 5, 16, 17, 64, 100, 127, 128, 0, 33]


def decode_two_calls(c, kc, vc):
    q, bt, lens = dev(c.query), dev(c.block_tables), dev(c.context_lens)
    maxL = max(1, int(c.context_lens.max()))
    out = torch.full_like(q, float("nan"))
    ws = binding.make_workspace(q, kc, maxL)
    binding.decode_partitions(out, q, kc, vc, bt, lens, c.scale, maxL, 0, ws)
    torch.cuda.synchronize()
    after_decode = out.clone()
    binding.decode_reduce(out, lens, c.num_kv_heads, c.block_size, c.block_tables.shape[1], maxL,
                          0, ws)
    torch.cuda.synchronize()
    return after_decode, out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B", [16, 32])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_one_wave_per_pair_shapes(dtype, D, B, G):
    """Eleven sequences of 0 to 128 tokens (two empty): the decode launch alone
    writes every row (zeros for the empty sequences), and the reduce call
    changes nothing."""
    c = W.make_case("pairs", 1100 + D + B + G, dtype, 2 * G, 2, D, B, LENS, extra_blocks=3)
    kc, vc = dev(c.key_cache), dev(c.value_cache)
    say("one wave per pair", dtype, D, B, G)
    after_decode, out = decode_two_calls(c, kc, vc)
    assert torch.equal(after_decode.view(torch.int16 if dtype == "bf16" else torch.int32),
                       out.view(torch.int16 if dtype == "bf16" else torch.int32))
    ref = oracle_decode(c, c.key_cache, c.value_cache)
    check_close(out, ref, dtype, f"pairs {dtype} D{D} B{B} G{G}")
    for s, L in enumerate(LENS):
        if L == 0:
            assert torch.count_nonzero(out[s]) == 0, f"row of empty sequence {s}"
    one = torch.empty_like(out)
    binding.decode(one, dev(c.query), kc, vc, dev(c.block_tables), dev(c.context_lens), c.scale,
                   max(LENS))
    nocopy = torch.empty_like(out)
    binding.decode_no_alloc(nocopy, dev(c.query), kc, vc, dev(c.block_tables),
                            dev(c.context_lens), c.scale, max(LENS))
    torch.cuda.synchronize()
    view = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(one.view(view), out.view(view)), "pa_decode against the two calls"
    assert torch.equal(nocopy.view(view), out.view(view)), "pa_decode_no_alloc"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_wave_per_pair_append(dtype):
    """The new token of each sequence written inside the pass: pools equal to
    the oracle's cache write bit for bit, output to the oracle's decode, and
    the fused call equal to the unfused pair bit for bit."""
    lens = [1, 2, 16, 17, 50, 128, 99, 64]
    c = W.make_case("pairs append", 1201, dtype, 8, 4, 128, 16, lens,
                    new_positions=[L - 1 for L in lens], extra_blocks=3)
    fused = check_case(c, f"pairs append {dtype}")
    check_case(c, f"pairs append {dtype} two calls", split=True)
    kc, vc = dev(c.key_cache), dev(c.value_cache)
    binding.reshape_and_cache(dev(c.new_key), dev(c.new_value), kc, vc, dev(c.slot_mapping))
    unfused = torch.empty_like(fused)
    binding.decode(unfused, dev(c.query), kc, vc, dev(c.block_tables), dev(c.context_lens),
                   c.scale, max(lens))
    torch.cuda.synchronize()
    view = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(fused.view(view), unfused.view(view)), "fused against unfused"


def test_one_wave_per_pair_fp8():
    c = W.make_case("pairs fp8", 1301, "bf16", 8, 2, 128, 16, LENS, extra_blocks=3)
    ks, vs = 1.0 / 64, 1.0 / 32
    kc8, vc8 = fp8_pools(c, ks, vs)
    say("one wave per pair, fp8")
    out = gpu_decode_fp8(c, kc8, vc8, ks, vs)
    ref = oracle.decode_fp8(c.query, kc8, vc8, c.block_tables, c.context_lens, c.scale, ks, vs)
    check_close(out, ref, "bf16", "pairs fp8")


@pytest.mark.parametrize("S", [128, 129])
def test_pair_bound(S):
    """128 sequences x 8 kv heads = 1,024 pairs (one wave each) and 129 x 8 =
    1,032 (over the bound: the equal split and its reduce), contexts of 1 to
    128 tokens."""
    c = W.random_case(1400 + S, "bf16", S, 32, 8, 128, 16, 1, 128, write_new=False)
    kc, vc = dev(c.key_cache), dev(c.value_cache)
    say("pair bound", S)
    after_decode, out = decode_two_calls(c, kc, vc)
    if S * 8 <= 1024:
        assert torch.equal(after_decode.view(torch.int16), out.view(torch.int16))
    check_close(out, oracle_decode(c, c.key_cache, c.value_cache), "bf16", f"pair bound S{S}")
