"""pa_decode_no_alloc: the decode with the library's static per-GPU workspace.

Through the C ABI: two calls in a row, the second on a smaller batch, each
equal bit for bit to pa_decode with a caller-allocated workspace (same plan,
same kernels) and within the bf16 tolerance of the fp64 oracle; the fixed
partition path too; a batch whose workspace exceeds the static array is
rejected before anything runs.
"""
import pytest
import torch

from paged_kv_cache_262_amd import binding
from paged_kv_cache_262_amd import workloads as W
from tests.gpu_util import check_close, dev, oracle_decode, say

pytestmark = pytest.mark.gpu


def _both(c, P=0):
    kc, vc = dev(c.key_cache), dev(c.value_cache)
    q, bt, lens = dev(c.query), dev(c.block_tables), dev(c.context_lens)
    maxL = int(c.context_lens.max())
    ref = torch.empty_like(q)
    binding.decode(ref, q, kc, vc, bt, lens, c.scale, maxL, partition_size=P)
    out = torch.full_like(q, float("nan"))
    binding.decode_no_alloc(out, q, kc, vc, bt, lens, c.scale, maxL, partition_size=P)
    torch.cuda.synchronize()
    return out, ref


def test_no_alloc_equals_decode_two_calls_then_smaller():
    big = W.random_case(901, "bf16", 64, 32, 8, 128, 16, 1, 3000, write_new=False)
    small = W.random_case(902, "bf16", 5, 8, 2, 128, 16, 1, 700, write_new=False)
    for name, c in (("64 seqs x 32/8 heads", big), ("5 seqs x 8/2 heads", small)):
        say("no-alloc decode,", name)
        out, ref = _both(c)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), name
        check_close(out, oracle_decode(c, c.key_cache, c.value_cache), "bf16", name)


def test_no_alloc_fixed_partitions_and_f32():
    c = W.random_case(903, "f32", 6, 8, 8, 64, 16, 1, 900, write_new=False)
    say("no-alloc decode, f32, partitions of 128")
    out, ref = _both(c, P=128)
    assert torch.equal(out, ref)
    check_close(out, oracle_decode(c, c.key_cache, c.value_cache), "f32", "f32 P=128")


def test_no_alloc_rejects_a_batch_beyond_the_scratch():
    cap = binding.decode_no_alloc_max_workspace()
    assert cap == 32 << 20
    # 8192 sequences x 2 kv heads x group 4 need about 34.6 MiB of records
    need = binding.decode_workspace_bytes(8192, 8, 2, 128, 16, 40, 0)
    assert need > cap
    q = torch.zeros((8192, 8, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((4, 2, 16, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((8192, 3), dtype=torch.int32, device="cuda")
    lens = torch.ones(8192, dtype=torch.int32, device="cuda")
    out = torch.zeros_like(q)
    say("no-alloc decode, oversized batch rejected")
    with pytest.raises(binding.PAError) as e:
        binding.decode_no_alloc(out, q, kc, kc, bt, lens, 0.1, 40)
    assert e.value.status == binding.PA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (out == 0).all()
