"""The decode kernels' cache policy, through the C ABI.

Units whose block the previous or the next sequence of the batch holds at the
same table position are loaded with the default cache policy (other waves
read them again), all others non-temporally.  The policy is an immediate of
the load instruction, so a wave splits its run of units wherever the flag
changes, and a split inside one (sequence, kv head) pair carries the running
softmax state across.  That split must not change a bit of the output.

Each case gives neighbouring sequences an irregular set of common blocks
(about half of the positions, so single shared blocks, alternating blocks
and longer stretches all occur inside the pairs), decodes, then gives every
sequence private copies of all its blocks (the same contents, nothing shared,
so no split) and requires identical bits; both are also checked against the
fp64 oracle.  Contexts are long (about 16K tokens) so that every wave's share
of the units spans many flag changes.
"""
import pytest
import torch

import oracle
from paged_kv_cache_262_amd import workloads as W
from tests.gpu_util import check_close, dev, gpu_decode, oracle_decode, say
from tests.test_fp8_gpu import fp8_pools, gpu_decode_fp8

pytestmark = pytest.mark.gpu

LENS = [16001, 15360, 16384, 12345]


def shared_tables(c, seed):
    """Sequence s + 1 takes sequence s's block at about half of the positions
    both hold (chains through several sequences included)."""
    g = torch.Generator().manual_seed(seed)
    bt = c.block_tables.clone()
    B = c.block_size
    nblk = [-(-int(L) // B) for L in c.context_lens]
    for s in range(c.num_seqs - 1):
        n = min(nblk[s], nblk[s + 1])
        take = torch.rand(n, generator=g) < 0.5
        bt[s + 1, :n] = torch.where(take, bt[s, :n], bt[s + 1, :n])
    return bt, nblk


def private_copies(pools, bt, nblk):
    """Pools extended by one private copy of every block each sequence uses,
    and tables that point at those copies (dim 0 of each pool is the block)."""
    NB = pools[0].shape[0]
    rows = torch.cat([bt[s, :n].long() for s, n in enumerate(nblk)])
    out = [torch.cat([p, p[rows]]) for p in pools]
    bt2 = bt.clone()
    k = NB
    for s, n in enumerate(nblk):
        bt2[s, :n] = torch.arange(k, k + n, dtype=torch.int32)
        k += n
    return out, bt2


@pytest.mark.parametrize("dtype,Hq,Hkv,B", [("bf16", 32, 8, 16), ("bf16", 32, 4, 32),
                                            ("f32", 8, 4, 16)])
def test_neighbour_sharing_does_not_change_bits(dtype, Hq, Hkv, B):
    c = W.make_case("policy", 1501 + B + Hkv, dtype, Hq, Hkv, 128, B, LENS, extra_blocks=3)
    bt, nblk = shared_tables(c, 7 + B)
    shared = sum(int((bt[s + 1, :min(nblk[s], nblk[s + 1])] ==
                      bt[s, :min(nblk[s], nblk[s + 1])]).sum()) for s in range(c.num_seqs - 1))
    assert shared > 100
    (kc2, vc2), bt2 = private_copies((c.key_cache, c.value_cache), bt, nblk)
    say("cache policy: shared tables", dtype, Hq, Hkv, B)
    a = gpu_decode(c, dev(c.key_cache), dev(c.value_cache), block_tables=bt)
    say("cache policy: private copies", dtype, Hq, Hkv, B)
    b = gpu_decode(c, dev(kc2), dev(vc2), block_tables=bt2)
    torch.cuda.synchronize()
    view = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(a.view(view), b.view(view)), "shared blocks changed the output bits"
    check_close(a, oracle_decode(c, c.key_cache, c.value_cache, block_tables=bt), dtype,
                f"policy {dtype} B{B}")


@pytest.mark.parametrize("B", [16, 32])
def test_neighbour_sharing_does_not_change_bits_fp8(B):
    c = W.make_case("policy fp8", 1601 + B, "bf16", 32, 8, 128, B, LENS, extra_blocks=3)
    ks, vs = 1.0 / 64, 1.0 / 32
    kc8, vc8 = fp8_pools(c, ks, vs)
    bt, nblk = shared_tables(c, 11 + B)
    (kc2, vc2), bt2 = private_copies((kc8, vc8), bt, nblk)
    c.block_tables = bt
    say("cache policy fp8: shared tables", B)
    a = gpu_decode_fp8(c, kc8, vc8, ks, vs)
    c.block_tables = bt2
    say("cache policy fp8: private copies", B)
    b = gpu_decode_fp8(c, kc2, vc2, ks, vs)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "shared blocks changed the bits"
    ref = oracle.decode_fp8(c.query, kc8, vc8, bt, c.context_lens, c.scale, ks, vs)
    check_close(a, ref, "bf16", f"policy fp8 B{B}")
