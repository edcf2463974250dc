"""Decode and prefill steps captured into a HIP graph (torch.cuda.CUDAGraph on
the current stream, which the binding passes to the C ABI).

Callers that capture their serving step need the library's calls to be
capturable: no allocation, no synchronisation and no host work that depends
on device data inside the call.  Each case warms the call up outside capture
(first-call set-up such as the shared-prefix side stream and the static
workspace address happens there), captures one step, then replays it several
times.  Between replays new queries are written into the captured input
buffer, the same call runs eagerly on a separate output, and other GPU work
runs; every replay must equal its eager twin bit for bit (both run the same
kernels on the same inputs, and the kernels are deterministic).
"""
import pytest
import torch

from paged_kv_cache_262_amd import binding
from paged_kv_cache_262_amd import workloads as W
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _capture(step):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def _replays_equal_eager(name, q, out, step_into, seed):
    """step_into(o) runs the step writing o; captured with o = out."""
    g = _capture(lambda: step_into(out))
    gen = torch.Generator().manual_seed(seed)
    noise = torch.empty(1 << 20, device=q.device)
    for r in range(REPLAYS):
        q.copy_(torch.randn(q.shape, generator=gen).to(q.dtype).to(q.device))
        ref = torch.empty_like(out)
        step_into(ref)
        noise.normal_()  # other work on the stream between eager call and replay
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"{name}: replay {r}"
        assert torch.isfinite(out).all(), f"{name}: replay {r}"


@pytest.mark.parametrize("entry", ["no_alloc", "caller_workspace"])
def test_decode_step_graph(entry):
    c = W.random_case(941, "bf16", 24, 32, 8, 128, 16, 1, 2500, write_new=False)
    kc, vc = dev(c.key_cache), dev(c.value_cache)
    q, bt, lens = dev(c.query), dev(c.block_tables), dev(c.context_lens)
    maxL = int(c.context_lens.max())
    out = torch.empty_like(q)
    ws = binding.make_workspace(q, kc, maxL)
    say("graph: decode", entry)

    def step_into(o):
        if entry == "no_alloc":
            binding.decode_no_alloc(o, q, kc, vc, bt, lens, c.scale, maxL)
        else:
            binding.decode(o, q, kc, vc, bt, lens, c.scale, maxL, workspace=ws)

    _replays_equal_eager(f"decode {entry}", q, out, step_into, 51)


def test_shared_prefix_decode_graph():
    """The prefix pass runs on the library's side stream: capture follows the
    fork and join events into the graph."""
    P, B = 4 * 16, 16
    c = W.make_case("graph shared prefix", 942, "bf16", 8, 2, 128, B,
                    [P + u for u in (0, 3, 40, 130, 250, 17, 90)], shared_prefix_tokens=P,
                    extra_blocks=3)
    kc, vc = dev(c.key_cache), dev(c.value_cache)
    q, bt, lens = dev(c.query), dev(c.block_tables), dev(c.context_lens)
    maxL = int(c.context_lens.max())
    out = torch.empty_like(q)
    ws = binding.make_shared_prefix_workspace(q, kc, maxL, 4)
    say("graph: shared-prefix decode")

    def step_into(o):
        binding.decode_shared_prefix(o, q, kc, vc, bt, lens, c.scale, maxL, 4, workspace=ws)

    _replays_equal_eager("shared-prefix decode", q, out, step_into, 52)


def test_fp8_shared_prefix_decode_graph():
    """The same with e4m3 pools (pa_decode_fp8_shared_prefix)."""
    from tests.test_fp8_gpu import fp8_pools
    P, B = 4 * 16, 16
    c = W.make_case("graph fp8 shared prefix", 944, "bf16", 8, 2, 128, B,
                    [P + u for u in (0, 3, 40, 130, 250, 17, 90)], shared_prefix_tokens=P,
                    extra_blocks=3)
    kc8, vc8 = fp8_pools(c, 1.0 / 64, 1.0 / 32)
    kc, vc = dev(kc8), dev(vc8)
    q, bt, lens = dev(c.query), dev(c.block_tables), dev(c.context_lens)
    maxL = int(c.context_lens.max())
    out = torch.empty_like(q)
    ws = binding.make_shared_prefix_workspace(q, kc, maxL, 4)
    say("graph: fp8 shared-prefix decode")

    def step_into(o):
        binding.decode_fp8_shared_prefix(o, q, kc, vc, bt, lens, c.scale, maxL, 4, 1.0 / 64,
                                         1.0 / 32, workspace=ws)

    _replays_equal_eager("fp8 shared-prefix decode", q, out, step_into, 54)


def test_prefill_chunk_graph():
    c = W.make_case("graph prefill", 943, "bf16", 8, 2, 128, 16, [5], new_positions=[4],
                    chunks=[(100, 700), (37, 37), (256, 1300)], extra_blocks=3)
    kc, vc = dev(c.key_cache), dev(c.value_cache)
    q = dev(c.chunk_query)
    out = torch.empty_like(q)
    bt, cu, cl = dev(c.chunk_block_tables), dev(c.chunk_cu_query_lens), dev(c.chunk_context_lens)
    maxq = int((c.chunk_cu_query_lens[1:] - c.chunk_cu_query_lens[:-1]).max())
    say("graph: prefill chunk")

    def step_into(o):
        binding.prefill_chunk(o, q, kc, vc, bt, cu, cl, c.scale, maxq)

    _replays_equal_eager("prefill chunk", q, out, step_into, 53)
