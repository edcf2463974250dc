#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

A step is one pass of the hot path over one batch: the cache write of the
step's new K/V tokens, decode attention over every sequence's paged context
(split-K partial results, then their merge), plus the prefill chunks when the
workload has them (pa_prefill_chunk).  When the new tokens are one per
sequence at its last position (a plain decode step) the cache write runs inside
the decode pass (pa_decode_append_partitions + pa_decode_reduce); otherwise it
is its own launch (pa_reshape_and_cache).  The default workload is the
Llama-3-8B-shaped decode layer: 64 sequences, 32 q / 8 kv heads, head_dim 128,
bf16, 16-token blocks, contexts uniform in [512, 4096], one new token per
sequence.

Inputs are synthetic (seeded) and already resident in HBM when timing starts.
Steps alternate between independent replicas of the pools so that the 256 MB
last-level cache cannot serve a step from the previous one.

Prints ONE JSON line (rank 0).  The value is the effective decode KV
bandwidth: algorithmic KV bytes of the step / step time.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from paged_kv_cache_262_amd import accounting as acct  # noqa: E402
from paged_kv_cache_262_amd import binding  # noqa: E402
from paged_kv_cache_262_amd import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, vendor figure
METRIC = "paged-attn decode KV GB/s (% of HBM peak) + seq-tokens/s, 8B GQA shape"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, choices=sorted(W.NAMED),
                    help="time only this workload (default: the Llama-3-8B-shaped decode as "
                         "the headline, then every other workload and the ceilings)")
    ap.add_argument("--no-extra", action="store_true",
                    help="default run: only the headline workload")
    ap.add_argument("--partition-size", type=int, default=0,
                    help="0: balanced split over waves (default); >0: fixed partitions")
    ap.add_argument("--replicas", type=int, default=2)
    ap.add_argument("--device-warmup-ms", type=float, default=50.0,
                    help="before the --warmup steps, run the same steps untimed for this long "
                         "(wall time), so that the timed steps see the clocks of a device that "
                         "has been busy; 0 turns it off")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="the oracle baseline repeats its full-workload run until this much "
                         "time has passed")
    ap.add_argument("--cpu-max-seconds", type=float, default=30.0,
                    help="cap on the whole oracle baseline (all threads, then one thread)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this size (counter calibration)")
    ap.add_argument("--op", default="attention",
                    choices=["attention", "copy_on_write", "swap_out", "swap_in",
                             "block_manager"],
                    help="attention: the hot-path step (default); the others time "
                         "pa_copy_blocks on the workload's pool")
    ap.add_argument("--copy-seqs", type=int, default=8,
                    help="sequences whose blocks a copy op moves")
    ap.add_argument("--no-shared-prefix", action="store_true",
                    help="prefix-sharing workload: the plain decode instead of "
                         "pa_decode_shared_prefix / pa_decode_fp8_shared_prefix (whose step "
                         "also reports the plain one)")
    ap.add_argument("--fused-writes", action="store_true",
                    help="chunked-prefill workloads (bf16): write the new tokens inside the "
                         "decode pass (pa_decode_append) and the prefill pass "
                         "(pa_prefill_chunk_append) instead of one pa_reshape_and_cache launch, "
                         "which is faster on MI355X; both step times are reported")
    ap.add_argument("--streams", type=int, default=1, choices=[1, 2],
                    help="chunked-prefill workloads: 2 runs decode and prefill on two streams "
                         "of equal priority (and also times the serial step)")
    ap.add_argument("--kv", default="native", choices=["native", "fp8"],
                    help="native: pools in the workload's dtype (default); fp8: e4m3 pools "
                         "written by pa_reshape_and_cache_fp8, decode by pa_decode_fp8")
    return ap.parse_args()


# Sources each kernel is built from; the traffic figures in
# profiles/hbm_traffic.txt are only reported while these are unchanged.
KERNEL_SOURCES = {
    "reshape_and_cache_kernel": ["reshape_and_cache.hip", "pa_common.h", "pa_internal.h"],
    "reshape_and_cache_fp8_kernel": ["reshape_and_cache.hip", "pa_common.h", "pa_internal.h"],
    "decode_stream_mma_kernel": ["decode.hip", "pa_common.h", "pa_internal.h", "pa_prefix.h"],
    "decode_stream_fp8_kernel": ["decode.hip", "pa_common.h", "pa_internal.h", "pa_prefix.h"],
    "decode_stream_kernel": ["decode.hip", "pa_common.h", "pa_internal.h", "pa_prefix.h"],
    "decode_stream_reduce_kernel": ["decode.hip", "pa_common.h", "pa_internal.h", "pa_prefix.h"],
    "decode_partition_kernel": ["decode.hip", "pa_common.h", "pa_internal.h", "pa_prefix.h"],
    "decode_prefix_mma_kernel": ["decode.hip", "pa_common.h", "pa_internal.h", "pa_prefix.h"],
    "prefill_chunk_kernel": ["prefill.hip", "pa_common.h", "pa_internal.h", "pa_prefill_append.h"],
    "prefill_chunk_fp8_kernel": ["prefill.hip", "pa_common.h", "pa_internal.h",
                                 "pa_prefill_append.h"],
    "copy_blocks_kernel": ["copy_blocks.hip", "pa_common.h", "pa_internal.h"],
}


def _source_digest(kernel: str):
    if kernel not in KERNEL_SOURCES:
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "paged_kv_cache_262_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _profile_value(table: str, kernel: str, workload: str):
    """Column 4 of the row (kernel, workload, hash of the kernel's current
    sources) of a table under profiles/, or None when no row matches."""
    path = os.path.join(ROOT, "profiles", table)
    digest = _source_digest(kernel)
    if digest is None or not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            parts = line.split()
            if (len(parts) >= 4 and not line.startswith("#")
                    and parts[:3] == [kernel, workload, digest]):
                return float(parts[3])
    return None


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    (scaled by a copy of known size), or None if not measured on these sources."""
    v = _profile_value("hbm_traffic.txt", kernel, workload)
    return None if v is None else int(v)


def profiled_duration_ns(kernel: str, workload: str):
    """Average launch duration from a rocprofv3 kernel trace of this workload
    on the current sources, or None."""
    return _profile_value("kernel_times.txt", kernel, workload)


def fused_append(case) -> bool:
    """A decode-only step whose new tokens are one per sequence, each at position
    L - 1 of its sequence: the cache write then runs inside the decode pass
    (pa_decode_append) instead of as its own launch."""
    if case.num_chunks or case.slot_mapping.numel() != case.num_seqs:
        return False
    B = case.block_size
    lens = case.context_lens.tolist()
    if min(lens) <= 0:
        return False
    bt = case.block_tables
    want = [int(bt[s, (L - 1) // B]) * B + (L - 1) % B for s, L in enumerate(lens)]
    return want == case.slot_mapping.tolist()


def split_mixed(case) -> bool:
    """A chunked-prefill step whose first num_seqs new tokens are one per
    decode sequence at position L - 1 (the rest are the chunks' own tokens):
    the decode tokens can then be written inside the decode pass and the
    chunk tokens by a cache write on the prefill's stream."""
    if not case.num_chunks or case.slot_mapping.numel() < case.num_seqs:
        return False
    B = case.block_size
    lens = case.context_lens.tolist()
    if min(lens) <= 0:
        return False
    bt = case.block_tables
    want = [int(bt[s, (L - 1) // B]) * B + (L - 1) % B for s, L in enumerate(lens)]
    return want == case.slot_mapping[:case.num_seqs].tolist()


# Per-pool scales of the FP8 benchmark pools: N(0, 1) data over 1/32 spans
# +-14 before saturation.
FP8_K_SCALE = FP8_V_SCALE = 1.0 / 32


def fp8_pools_on_device(case, dev):
    """FP8 pools (K [NB, Hkv, B, D], V [NB, Hkv, D, B] uint8) holding the
    workload's pools, quantised by the library's own cache write: every slot
    of the pool is written once."""
    NB, Hkv, B, D = case.key_cache.shape
    kc8 = torch.zeros((NB, Hkv, B, D), dtype=torch.uint8, device=dev)
    vc8 = torch.zeros((NB, Hkv, D, B), dtype=torch.uint8, device=dev)
    step = max(1, (1 << 28) // (2 * Hkv * B * D * case.key_cache.element_size()))
    for b0 in range(0, NB, step):
        b1 = min(NB, b0 + step)
        rows_k = case.key_cache[b0:b1].permute(0, 2, 1, 3).reshape(-1, Hkv, D).to(dev)
        rows_v = case.value_cache[b0:b1].permute(0, 2, 1, 3).reshape(-1, Hkv, D).to(dev)
        slots = torch.arange(b0 * B, b1 * B, dtype=torch.int64, device=dev)
        binding.reshape_and_cache_fp8(rows_k, rows_v, kc8, vc8, slots, FP8_K_SCALE, FP8_V_SCALE)
    torch.cuda.synchronize()
    return kc8, vc8


class Replica:
    """One device copy of a workload."""

    def __init__(self, case, dev, fp8=False):
        if fp8:
            self.kc, self.vc = fp8_pools_on_device(case, dev)
        else:
            self.kc = case.key_cache.to(dev)
            self.vc = case.value_cache.to(dev)
        self.q = case.query.to(dev)
        self.bt = case.block_tables.to(dev)
        self.lens = case.context_lens.to(dev)
        self.nk = case.new_key.to(dev)
        self.nv = case.new_value.to(dev)
        self.slots = case.slot_mapping.to(dev)
        self.out = torch.empty_like(self.q)
        S = case.num_seqs
        if fused_append(case) or split_mixed(case):
            self.nk_seq = case.new_key[:S].contiguous().to(dev)
            self.nv_seq = case.new_value[:S].contiguous().to(dev)
        if split_mixed(case):
            self.nk_chunk = case.new_key[S:].contiguous().to(dev)
            self.nv_chunk = case.new_value[S:].contiguous().to(dev)
            self.slots_chunk = case.slot_mapping[S:].contiguous().to(dev)
        if case.num_chunks:
            self.cq = case.chunk_query.to(dev)
            self.cbt = case.chunk_block_tables.to(dev)
            self.ccu = case.chunk_cu_query_lens.to(dev)
            self.clens = case.chunk_context_lens.to(dev)
            self.cout = torch.empty_like(self.cq)


METRICS = {
    "llama8b_decode": METRIC,
    "tiny_decode": "paged-attn decode KV GB/s + seq-tokens/s, tiny fp32 shape (4 seqs, d 64)",
    "long_context_decode": "paged-attn decode KV GB/s (% of HBM peak) + seq-tokens/s, "
                           "70B-shaped GQA, 8 seqs x 32K",
    "prefix_sharing_decode": "paged-attn decode unique-KV GB/s (% of HBM peak), 128 seqs "
                             "sharing a 1024-token prefix",
    "mixed_chunked_prefill": "mixed chunked-prefill step: decode KV GB/s + prefill TFLOP/s "
                             "(% of bf16 MFMA peak)",
}
# The other workloads the default run measures after the headline one.
# (workload, FP8 pools, options of measure(), suffix of the entry's key); the
# entries with options time the alternative entry points on the same batch.
EXTRA_WORKLOADS = [("tiny_decode", False, {}, ""), ("long_context_decode", False, {}, ""),
                   ("prefix_sharing_decode", False, {}, ""),
                   ("mixed_chunked_prefill", False, {}, ""),
                   ("mixed_chunked_prefill", False, {"fuse_writes": True}, "_fused_writes"),
                   ("llama8b_decode", True, {}, ""), ("long_context_decode", True, {}, ""),
                   ("prefix_sharing_decode", True, {}, ""),
                   ("mixed_chunked_prefill", True, {}, "")]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested). Sharding is described in the design notes.",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    binding.load()
    dev = torch.device("cuda:0")
    full_run = args.workload is None
    name = args.workload or "llama8b_decode"
    case = W.NAMED[name]()
    if args.op == "block_manager":
        return run_block_manager(args, case)
    if args.op != "attention":
        return run_copy(args, case, dev)
    fp8 = args.kv == "fp8"
    if fp8 and (case.dtype != "bf16" or args.partition_size):
        print("--kv fp8 runs bf16 workloads with the balanced split", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib, dev)
    result, reps = measure(case, dev, fp8, args.partition_size, args.steps, args.warmup,
                           args.replicas, args.streams, not args.no_shared_prefix,
                           args.fused_writes, args.device_warmup_ms)
    del reps
    torch.cuda.empty_cache()
    ceilings = None
    if full_run and not args.no_extra:
        result["workloads"] = {}
        for wname, wfp8, opts, tag in EXTRA_WORKLOADS:
            wcase = case if wname == name else W.NAMED[wname]()
            r, wreps = measure(wcase, dev, wfp8, 0, args.steps, args.warmup, args.replicas,
                               device_warmup_ms=args.device_warmup_ms, **opts)
            del wreps
            torch.cuda.empty_cache()
            result["workloads"][wname + ("_fp8" if wfp8 else "") + tag] = summary(r)
        ceilings = measure_ceilings(dev, result["roofline"]["algorithmic_bytes_per_launch"])
        result["ceilings"] = ceilings
        attach_attainable(result, ceilings)
        for r in result["workloads"].values():
            attach_attainable(r, ceilings)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, fp8, args.cpu_seconds,
                                              args.cpu_max_seconds, result["_kv_bytes"])
    result.pop("_kv_bytes", None)
    print(json.dumps(result), flush=True)


def copy_probe(mib, dev):
    """One plain device copy of known size (the counter calibration)."""
    n = mib * (1 << 20) // 4
    a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(f"copy probe: {mib} MiB read + {mib} MiB written", file=sys.stderr, flush=True)


def measure(case, dev, fp8, P, steps, warmup, replicas, streams=1, shared_prefix=True,
            fuse_writes=False, device_warmup_ms=50.0):
    """Times `steps` steps of the hot path on one workload (after `warmup`
    untimed ones), then the same steps again with an event around each kernel
    for the per-kernel breakdown.  Returns (result dict, device replicas)."""
    S, Hq, Hkv, D, B = (case.num_seqs, case.num_q_heads, case.num_kv_heads, case.head_dim,
                        case.block_size)
    label = case.name + (" (FP8 e4m3 KV cache)" if fp8 else "")
    print(f"workload {label}: setting up", file=sys.stderr, flush=True)
    eb = 1 if fp8 else case.key_cache.element_size()  # bytes per cached element
    lens = case.context_lens.tolist()
    maxL = case.max_context_len
    reps = [Replica(case, dev, fp8) for _ in range(max(1, replicas))]
    ws = binding.make_workspace(reps[0].q, reps[0].kc, maxL, P)
    stream = torch.cuda.current_stream()
    # The prefix-sharing batch: pa_decode_shared_prefix (pa_decode_fp8_shared_prefix
    # over FP8 pools), which reads the shared blocks once per tile of sequences
    # instead of once per sequence (its prefix pass runs on a second stream
    # beside the suffix pass).
    pb = case.shared_blocks.numel() if case.shared_blocks is not None else 0
    sp = bool(shared_prefix and pb and case.dtype == "bf16" and P == 0)
    sp_name = "pa_decode_fp8_shared_prefix" if fp8 else "pa_decode_shared_prefix"
    ws_sp = binding.make_shared_prefix_workspace(reps[0].q, reps[0].kc, maxL, pb) if sp else None

    # Algorithmic work per step.
    unique = None
    if case.shared_blocks is not None:
        n_sh = case.shared_blocks.numel() * B
        unique = n_sh + sum(L - n_sh for L in lens)
    dec_bytes = acct.decode_bytes(lens, Hq, Hkv, D, B, eb, unique_tokens=unique,
                                  q_elem_bytes=case.query.element_size())
    kv_bytes = (sum(lens) if unique is None else unique) * acct.kv_bytes_per_token(1, Hkv, D, eb)
    T = case.slot_mapping.numel()
    cw_bytes = acct.cache_write_bytes(T, Hkv, D, eb, src_elem_bytes=case.new_key.element_size())
    chunks = []
    if case.num_chunks:
        cu = case.chunk_cu_query_lens.tolist()
        chunks = [(cu[i + 1] - cu[i], int(case.chunk_context_lens[i]))
                  for i in range(case.num_chunks)]
    pf_flops = acct.prefill_flops(chunks, Hq, D) if chunks else 0
    maxq = max((n for n, _ in chunks), default=0)

    ev = {k: [] for k in ("cw0", "cw1", "dp0", "dp1", "dr1", "pf0", "pf1")}
    fused = fused_append(case)
    # A bf16 chunked-prefill step whose decode tokens sit at L - 1: the decode
    # tokens are written inside the decode pass (pa_decode_append) and the
    # chunk tokens inside the prefill pass (pa_prefill_chunk_append).
    mixed_fused = bool(fuse_writes and chunks and split_mixed(case) and not fp8 and P == 0)
    # Events of the per-kernel pass, created before it starts.
    pool = [torch.cuda.Event(enable_timing=True) for _ in range(5 * steps)]

    def mark(key):
        e = pool.pop()
        e.record(stream)
        ev[key].append(e)
        return e

    def step(i, record):
        r = reps[i % len(reps)]
        if record:
            mark("cw0")
        if T and fp8 and not fused:
            binding.reshape_and_cache_fp8(r.nk, r.nv, r.kc, r.vc, r.slots, FP8_K_SCALE,
                                          FP8_V_SCALE, stream=stream)
        elif T and not fused and not mixed_fused:
            binding.reshape_and_cache(r.nk, r.nv, r.kc, r.vc, r.slots, stream=stream)
        if record:
            ev["dp0"].append(mark("cw1"))
        if sp and fp8:  # prefix pass, suffix pass and reduce in one call
            binding.decode_fp8_shared_prefix(r.out, r.q, r.kc, r.vc, r.bt, r.lens, case.scale,
                                             maxL, pb, FP8_K_SCALE, FP8_V_SCALE,
                                             workspace=ws_sp, stream=stream)
            if record:
                mark("dp1")
                mark("dr1")
            return
        if sp:
            binding.decode_shared_prefix(r.out, r.q, r.kc, r.vc, r.bt, r.lens, case.scale, maxL,
                                         pb, workspace=ws_sp, stream=stream)
            if record:
                mark("dp1")
                mark("dr1")
            return
        if fp8 and fused:
            binding.decode_fp8_append_partitions(r.out, r.q, r.nk_seq, r.nv_seq, r.kc, r.vc, r.bt,
                                                 r.lens, case.scale, maxL, FP8_K_SCALE,
                                                 FP8_V_SCALE, ws, stream=stream)
        elif fp8:
            binding.decode_fp8_partitions(r.out, r.q, r.kc, r.vc, r.bt, r.lens, case.scale, maxL,
                                          FP8_K_SCALE, FP8_V_SCALE, ws, stream=stream)
        elif fused or mixed_fused:
            binding.decode_append_partitions(r.out, r.q, r.nk_seq, r.nv_seq, r.kc, r.vc, r.bt,
                                             r.lens, case.scale, maxL, P, ws, stream=stream)
        else:
            binding.decode_partitions(r.out, r.q, r.kc, r.vc, r.bt, r.lens, case.scale, maxL, P,
                                      ws, stream=stream)
        if record:
            mark("dp1")
        binding.decode_reduce(r.out, r.lens, Hkv, B, case.max_blocks_per_seq, maxL, P, ws,
                              stream=stream)
        if record:
            e = mark("dr1")
        if chunks:
            if record:
                ev["pf0"].append(e)
            if fp8:
                binding.prefill_chunk_fp8(r.cout, r.cq, r.kc, r.vc, r.cbt, r.ccu, r.clens,
                                          case.scale, maxq, FP8_K_SCALE, FP8_V_SCALE,
                                          stream=stream)
            elif mixed_fused:
                binding.prefill_chunk_append(r.cout, r.cq, r.nk_chunk, r.nv_chunk, r.kc, r.vc,
                                             r.cbt, r.ccu, r.clens, case.scale, maxq,
                                             stream=stream)
            else:
                binding.prefill_chunk(r.cout, r.cq, r.kc, r.vc, r.cbt, r.ccu, r.clens, case.scale,
                                      maxq, stream=stream)
            if record:
                mark("pf1")

    # streams == 2: a chunked-prefill step whose decode tokens can be written
    # inside the decode pass runs as two streams of equal priority: decode
    # (with those writes) and its reduce on the current stream; the cache
    # write of the chunk tokens and the prefill on a second one.  The two meet
    # at the end of every step.  (The kernels cannot share a CU, so this is
    # slower than the serial step; it is kept to measure that.)
    overlap = streams == 2 and bool(chunks) and split_mixed(case)
    side = torch.cuda.Stream(device=dev) if overlap else None
    forks = [torch.cuda.Event() for _ in range(2)]
    joins = [torch.cuda.Event() for _ in range(2)]

    def overlapped_step(i):
        r = reps[i % len(reps)]
        fork, join = forks[i % 2], joins[i % 2]
        fork.record(stream)
        side.wait_event(fork)
        if fp8:
            binding.decode_fp8_append_partitions(r.out, r.q, r.nk_seq, r.nv_seq, r.kc, r.vc, r.bt,
                                                 r.lens, case.scale, maxL, FP8_K_SCALE,
                                                 FP8_V_SCALE, ws, stream=stream)
            binding.reshape_and_cache_fp8(r.nk_chunk, r.nv_chunk, r.kc, r.vc, r.slots_chunk,
                                          FP8_K_SCALE, FP8_V_SCALE, stream=side)
            binding.prefill_chunk_fp8(r.cout, r.cq, r.kc, r.vc, r.cbt, r.ccu, r.clens,
                                      case.scale, maxq, FP8_K_SCALE, FP8_V_SCALE, stream=side)
        else:
            binding.decode_append_partitions(r.out, r.q, r.nk_seq, r.nv_seq, r.kc, r.vc, r.bt,
                                             r.lens, case.scale, maxL, P, ws, stream=stream)
            binding.reshape_and_cache(r.nk_chunk, r.nv_chunk, r.kc, r.vc, r.slots_chunk,
                                      stream=side)
            binding.prefill_chunk(r.cout, r.cq, r.kc, r.vc, r.cbt, r.ccu, r.clens, case.scale,
                                  maxq, stream=side)
        join.record(side)
        binding.decode_reduce(r.out, r.lens, Hkv, B, case.max_blocks_per_seq, maxL, P, ws,
                              stream=stream)
        stream.wait_event(join)

    def timed(fn, n):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0 = torch.cuda.Event(enable_timing=True); e0.record(stream)
        for i in range(n):
            fn(i)
        e1 = torch.cuda.Event(enable_timing=True); e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, time.perf_counter() - t0

    run_step = overlapped_step if overlap else (lambda i: step(i, False))
    # The garbage collector is off from here on: a collection that stalls the
    # host long enough to drain the queue would show up inside one interval.
    # It runs once before the warm-up, not between warm-up and timing: a host
    # pause of some milliseconds there lets the GPU clocks drop, and the first
    # timed steps then ran 2-6% slower than the same steps timed again.
    gc.collect()
    gc.disable()
    # Device warm-up: the same steps, untimed, for device_warmup_ms of wall
    # time (the host waits for the device every 16 steps, so the time is the
    # device's).  An idle device raises its clocks over the first tens of
    # milliseconds of sustained work; measured on this part, the first 200
    # steps timed after a 20-step warm-up ran 1.5% (8B decode) to 6% (mixed
    # step) slower than the same steps timed again, and 400 more untimed
    # steps removed the difference.
    n_dev = 0
    t_end = time.perf_counter() + device_warmup_ms / 1e3
    while time.perf_counter() < t_end:
        run_step(n_dev)
        if overlap:
            step(n_dev, False)
        n_dev += 1
        if n_dev % 16 == 0:
            torch.cuda.synchronize()
    for i in range(warmup):
        run_step(i)
        if overlap:
            step(i, False)
    torch.cuda.synchronize()
    print(f"warmup done ({n_dev} device warm-up steps, then {warmup} steps)", file=sys.stderr,
          flush=True)

    # The timed steps carry no events between kernels; a second pass of the
    # same steps records one event around each kernel for the breakdown.
    ms_step, wall = timed(run_step, steps)
    print(f"timed {steps} steps: {ms_step:.4f} ms/step (wall {wall:.3f} s)", file=sys.stderr,
          flush=True)
    serial_ms = timed(lambda i: step(i, False), steps)[0] if overlap else None
    separate_ms = None
    if mixed_fused:  # the same step with one cache-write launch, for comparison
        mixed_fused = False
        for i in range(warmup):
            step(i, False)
        separate_ms = timed(lambda i: step(i, False), steps)[0]
        mixed_fused = True
    plain_ms = None
    if sp:  # the same batch through the plain balanced decode, for comparison
        sp = False
        for i in range(warmup):
            step(i, False)
        plain_ms = timed(lambda i: step(i, False), steps)[0]
        sp = True
    for i in range(steps):
        step(i, True)
    torch.cuda.synchronize()
    gc.enable()
    print("per-kernel pass done", file=sys.stderr, flush=True)

    medians = {}

    def avg_ms(a, b):
        xs = sorted(x.elapsed_time(y) for x, y in zip(ev[a], ev[b]))
        if not xs:
            return None
        medians[a + b] = xs[len(xs) // 2]
        return sum(xs) / len(xs)

    t_cw = avg_ms("cw0", "cw1") if T and not fused and not mixed_fused else None
    t_dp = avg_ms("dp0", "dp1")
    # The reduce call launches nothing when the decode gives each (sequence,
    # kv head) pair one wave (small batches of short contexts).
    has_reduce = binding.decode_needs_reduce(S, Hq, Hkv, D, B, maxL, P)
    t_dr = avg_ms("dp1", "dr1") if not sp and has_reduce else None  # sp: inside the one call
    t_pf = avg_ms("pf0", "pf1") if chunks else None

    value = kv_bytes / (ms_step * 1e-3) / 1e9
    # Key of the profile rows (kernel traces, HBM bytes) for this measurement:
    # the step with the writes inside the passes runs other kernel variants.
    wl = case.name + ("_fp8" if fp8 else "") + ("_fused" if mixed_fused else "")
    # bf16 uses the matrix-core variant of the balanced split.
    dp_kernel = ("decode_stream_fp8_kernel" if fp8 else
                 "decode_partition_kernel" if P != 0 or S > 8192 else
                 "decode_stream_mma_kernel" if case.dtype == "bf16" else "decode_stream_kernel")
    # The fused step's decode kernel also moves the new tokens' rows.
    dp_bytes = dec_bytes + (cw_bytes if fused else 0)
    if mixed_fused:  # the decode tokens' rows (S of the T new rows)
        dp_bytes = dec_bytes + acct.cache_write_bytes(S, Hkv, D, eb,
                                                      src_elem_bytes=case.new_key.element_size())
    if sp:  # one call: prefix pass + suffix pass + reduce
        dp_kernel = sp_name
    result = {
        "metric": METRICS[case.name] + (", FP8 e4m3 KV cache" if fp8 else ""),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "device_warmup": {"ms": device_warmup_ms, "steps": n_dev},
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 kv, bf16 q" if fp8 else case.dtype,
        "data": "synthetic",
        "config": {
            "workload": label,
            "num_seqs": S, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
            "block_size": B, "context_tokens": sum(lens), "new_tokens": T,
            "split": "balanced" if P == 0 else f"partitions of {P} tokens",
            "decode": (f"{sp_name} (prefix pass, suffix pass, reduce)" if sp
                       else "pa_decode_partitions + pa_decode_reduce"),
            "cache_write": ("decode tokens inside the decode pass (pa_decode_append), chunk "
                            "tokens inside the prefill pass (pa_prefill_chunk_append)"
                            if mixed_fused else
                            "fused into the decode pass (pa_decode_fp8_append)" if fused and fp8
                            else "fused into the decode pass (pa_decode_append)" if fused
                            else "pa_reshape_and_cache_fp8" if T and fp8
                            else "pa_reshape_and_cache" if T else "none"),
            "replicas": len(reps),
            "prefill_chunks": chunks,
            "streams": ("2 of equal priority: decode with its tokens' cache write + reduce; "
                        "the chunk tokens' cache write + prefill" if overlap else "1"),
        },
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "seq_tokens_per_s": round(sum(lens) / (ms_step * 1e-3), 1),
        "new_tokens_per_s": round(S / (ms_step * 1e-3), 1),
        "serial_ms_per_step": _r(serial_ms),
        "plain_decode_ms_per_step": _r(plain_ms),
        "separate_cache_write_ms_per_step": _r(separate_ms),
        "kernels_ms": {"reshape_and_cache": "fused" if (fused or mixed_fused) else _r(t_cw),
                       ("decode_shared_prefix" if sp else "decode_partition"): _r(t_dp),
                       "decode_reduce": _r(t_dr) if (sp or has_reduce) else "none",
                       "prefill_chunk": _r(t_pf)},
        "roofline": roofline(dp_kernel, wl, "hbm", dp_bytes, t_dp, HBM_PEAK_GBS,
                             medians["dp0dp1"]),
        "_kv_bytes": kv_bytes,
    }
    if chunks:
        pf_kernel = "prefill_chunk_fp8_kernel" if fp8 else "prefill_chunk_kernel"  # (append variant when fused)
        pr = roofline(pf_kernel, wl, "mfma", pf_flops, t_pf, BF16_MFMA_PEAK_TFLOPS,
                      medians["pf0pf1"])
        pr["query_tokens_per_s"] = round(sum(n for n, _ in chunks) / (t_pf * 1e-3), 1)
        result["prefill_roofline"] = pr
    if t_cw is not None:
        cw_kernel = "reshape_and_cache_fp8_kernel" if fp8 else "reshape_and_cache_kernel"
        cw = roofline(cw_kernel, wl, "hbm", cw_bytes, t_cw, HBM_PEAK_GBS, medians["cw0cw1"])
        cw["GB/s"] = cw["achieved"]
        result["cache_write"] = cw
    return result, reps


def _r(x, nd=5):
    return None if x is None else round(x, nd)


def roofline(kernel, workload, bound, work, ms, peak, median_ms):
    """Roofline entry of one kernel: `work` algorithmic bytes (hbm) or flops
    (mfma) per launch over its event-timed average `ms`; beside it the same
    work over the rocprofv3 kernel-trace average committed for these sources,
    when there is one."""
    scale = 1e9 if bound == "hbm" else 1e12
    achieved = work / (ms * 1e-3) / scale
    r = {"kernel": kernel, "bound": bound, "achieved": round(achieved, 1), "peak": peak,
         "unit": "GB/s" if bound == "hbm" else "TFLOP/s", "frac": round(achieved / peak, 4),
         "timer": "HIP events around each launch on its stream",
         "traffic": measured_traffic(kernel, workload),
         ("algorithmic_bytes_per_launch" if bound == "hbm"
          else "algorithmic_flops_per_launch"): work,
         "event_us": round(ms * 1e3, 2), "event_median_us": round(median_ms * 1e3, 2)}
    prof_ns = profiled_duration_ns(kernel, workload)
    if prof_ns is not None:
        a = work / (prof_ns * 1e-9) / scale
        r["rocprof_us"] = round(prof_ns / 1e3, 2)
        r["rocprof_frac"] = round(a / peak, 4)
    else:
        r["rocprof_us"] = r["rocprof_frac"] = None
    return r


def summary(r):
    """The per-workload entry of the default run's line."""
    keys = ("metric", "value", "unit", "ms_per_step", "serial_ms_per_step",
            "plain_decode_ms_per_step", "separate_cache_write_ms_per_step", "hbm_frac",
            "seq_tokens_per_s", "kernels_ms", "roofline", "prefill_roofline", "cache_write")
    out = {k: r[k] for k in keys if k in r}
    out["step_us"] = round(r["ms_per_step"] * 1e3, 2)
    out["workload"] = r["config"]["workload"]
    return out


def measure_ceilings(dev, decode_bytes):
    """Attainable ceilings measured next to the kernels: a streaming read of
    2 x 1 GiB and of two buffers of the 8B decode's algorithmic size
    (alternated, so the last-level cache cannot serve one read from the
    previous one), and the bf16 matrix-core probe."""
    stream = torch.cuda.current_stream()
    sink = binding.probe_sink(dev)

    def time_reads(nbytes, launches):
        nbytes = -(-nbytes // 16) * 16
        bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(2)]
        for i in range(4):
            binding.probe_stream_read(bufs[i % 2], sink, stream=stream)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True); e0.record(stream)
        for i in range(launches):
            binding.probe_stream_read(bufs[i % 2], sink, stream=stream)
        e1 = torch.cuda.Event(enable_timing=True); e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / launches
        del bufs
        return nbytes, ms

    nb, ms = time_reads(1 << 30, 20)
    big = nb / (ms * 1e-3) / 1e9
    nb2, ms2 = time_reads(decode_bytes, 40)
    fit = nb2 / (ms2 * 1e-3) / 1e9
    torch.cuda.empty_cache()

    # About 1 ms per launch; 20 launches bring the clock up before the 10 timed.
    iters = 5000
    for _ in range(20):
        binding.probe_mfma_bf16(sink, iters, stream=stream)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True); e0.record(stream)
    flops = 0.0
    for _ in range(10):
        flops += binding.probe_mfma_bf16(sink, iters, stream=stream)
    e1 = torch.cuda.Event(enable_timing=True); e1.record(stream)
    torch.cuda.synchronize()
    tf = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    print(f"ceilings: read {big:.0f} GB/s (1 GiB), {fit:.0f} GB/s ({nb2} B); "
          f"bf16 MFMA {tf:.0f} TFLOP/s", file=sys.stderr, flush=True)
    return {
        "stream_read": {"op": "pa_probe_stream_read", "GB/s": round(big, 1),
                        "frac_of_peak": round(big / HBM_PEAK_GBS, 4), "bytes": nb,
                        "peak": HBM_PEAK_GBS},
        "stream_read_decode_size": {"op": "pa_probe_stream_read", "GB/s": round(fit, 1),
                                    "bytes": nb2, "us": round(ms2 * 1e3, 2),
                                    "frac_of_peak": round(fit / HBM_PEAK_GBS, 4)},
        "mfma_bf16": {"op": "pa_probe_mfma_bf16", "TFLOP/s": round(tf, 1),
                      "frac_of_peak": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                      "peak": BF16_MFMA_PEAK_TFLOPS},
    }


def attach_attainable(r, ceilings):
    """Each roofline's achieved rate as a fraction of the measured ceiling."""
    for key in ("roofline", "cache_write"):
        if r.get(key):
            r[key]["frac_of_attainable"] = round(
                r[key]["achieved"] / ceilings["stream_read"]["GB/s"], 4)
    if r.get("prefill_roofline"):
        r["prefill_roofline"]["frac_of_attainable"] = round(
            r["prefill_roofline"]["achieved"] / ceilings["mfma_bf16"]["TFLOP/s"], 4)


def run_block_manager(args, case):
    """The host block manager (pa_bm_*) on the workload's batch: each sequence is
    added with a prompt of its context length (the prefix-sharing workload's
    shared prefix is the same tokens, found by the prefix cache), then every
    step appends one token to every sequence, takes the copy-on-write pairs and
    exports every block table.  Reports the host time per step, the prefix
    cache's reuse and the internal fragmentation against its closed form."""
    import random
    rnd = random.Random(0)
    B = case.block_size
    lens = case.context_lens.tolist()
    shared = (case.shared_blocks.numel() * B) if case.shared_blocks is not None else 0
    system = [rnd.randint(0, 31999) for _ in range(shared)]
    prompts = [system + [rnd.randint(0, 31999) for _ in range(L - shared)] for L in lens]
    nb_needed = sum(-(-(L + args.steps + args.warmup) // B) for L in lens) + 8
    bm = binding.BlockManager(nb_needed, B, prefix_cache=True)
    t0 = time.perf_counter()
    for s, p in enumerate(prompts):
        bm.add_sequence(s, p)
    t_add = time.perf_counter() - t0
    after_add = bm.stats()

    ids = list(range(len(prompts)))
    toks = [7] * len(prompts)
    width = max(-(-(L + args.steps + args.warmup) // B) for L in lens)

    def step():
        bm.append_batch(ids, toks)
        bm.take_copies()
        bm.block_tables(ids, width)
    for _ in range(args.warmup):
        step()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    per = (time.perf_counter() - t0) / args.steps
    st = bm.stats()
    frag = 1.0 - st["seq_tokens"] / st["seq_slots"]
    closed = sum(-(-(L + args.steps + args.warmup) // B) * B - (L + args.steps + args.warmup)
                 for L in lens) / st["seq_slots"]
    result = {
        "metric": "block manager host time per decode step (append + tables)",
        "value": round(per * 1e6, 2), "unit": "us", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(per * 1e3, 5), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "int", "data": "synthetic",
        "config": {"workload": f"{case.name} batch on the host block manager",
                   "num_seqs": len(lens), "block_size": B, "pool_blocks": nb_needed},
        "add_all_sequences_ms": round(t_add * 1e3, 3),
        "prefix_hits_blocks": after_add["prefix_hits"],
        "shared_blocks_after_add": after_add["shared_blocks"],
        "internal_fragmentation": round(frag, 6),
        "fragmentation_closed_form": round(closed, 6),
        "roofline": None,
    }
    if not args.no_cpu_baseline:
        from oracle.block_manager import ReferenceBlockManager
        ref = ReferenceBlockManager(nb_needed, B, True)
        for s, p in enumerate(prompts):
            ref.add_sequence(s, p)
        t0 = time.perf_counter()
        n = args.steps + args.warmup  # the pool holds exactly this many appends
        for _ in range(n):
            for s in range(len(prompts)):
                ref.append(s, 7)
            ref.take_copies()
            for s in range(len(prompts)):
                list(ref.tables[s])
        result["cpu_baseline"] = {"value": round((time.perf_counter() - t0) / n * 1e6, 2),
                                  "unit": "us", "cores": 1, "kind": "oracle",
                                  "sample": f"the Python reference model, {n} steps"}
    bm.close()
    print(json.dumps(result), flush=True)


PCIE_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction: the host link of the swap
COPY_SETS = 4


def run_copy(args, case, dev):
    """pa_copy_blocks on the workload's pool: the blocks of --copy-seqs
    sequences are copied to fresh blocks of the same device pool
    (copy_on_write), to a pinned host pool (swap_out) or from it back into
    fresh device blocks (swap_in).  One launch per step; the steps rotate over
    COPY_SETS disjoint groups of sequences, so that the sources of a launch
    are not in the last-level cache from the launch before."""
    B = case.block_size
    lens = case.context_lens.tolist()
    k = args.copy_seqs
    nsets = max(1, min(COPY_SETS, len(lens) // k))
    srcs = []
    for j in range(nsets):
        ids = range(j * k, (j + 1) * k)
        srcs.append(torch.cat([case.block_tables[s, :-(-int(lens[s]) // B)] for s in ids])
                    .to(torch.int64))
    ns = [x.numel() for x in srcs]
    NB = case.key_cache.shape[0]
    kc = torch.cat([case.key_cache, torch.zeros_like(case.key_cache[:1]).expand(sum(ns), -1, -1, -1)]).to(dev)
    vc = torch.cat([case.value_cache, torch.zeros_like(case.value_cache[:1]).expand(sum(ns), -1, -1, -1)]).to(dev)
    firsts = [NB + sum(ns[:j]) for j in range(nsets)]
    fresh = [torch.arange(f, f + n, dtype=torch.int64) for f, n in zip(firsts, ns)]
    block_bytes = case.key_cache[0].numel() * case.key_cache.element_size()
    shape = tuple(case.key_cache.shape[1:])
    calls = []  # (src k, src v, dst k, dst v, mapping) per set
    for j in range(nsets):
        n = ns[j]
        if args.op == "copy_on_write":
            calls.append((kc, vc, kc, vc, torch.stack([srcs[j], fresh[j]], 1)))
            continue
        hk = torch.zeros((n,) + shape, dtype=case.key_cache.dtype, pin_memory=True)
        hv = torch.zeros_like(hk).pin_memory()
        slots = torch.arange(n, dtype=torch.int64)
        if args.op == "swap_out":
            calls.append((kc, vc, hk, hv, torch.stack([srcs[j], slots], 1)))
        else:
            binding.copy_blocks(kc, vc, hk, hv, torch.stack([srcs[j], slots], 1).contiguous().to(dev))
            calls.append((hk, hv, kc, vc, torch.stack([slots, fresh[j]], 1)))
    calls = [(a, b, c, d, m.contiguous().to(dev)) for a, b, c, d, m in calls]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        binding.copy_blocks(*calls[i % nsets], stream=stream)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True); e0.record(stream)
    for i in range(args.steps):
        binding.copy_blocks(*calls[i % nsets], stream=stream)
    e1 = torch.cuda.Event(enable_timing=True); e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # The same launches with an event on each side, for the kernel's own time
    # (back to back, host launch time can leave gaps between short launches).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record(stream)
        binding.copy_blocks(*calls[i % nsets], stream=stream)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    # K and V blocks, each read once and written once
    moved_i = [2 * ns[i % nsets] * block_bytes for i in range(args.steps)]
    moved = sum(moved_i) // args.steps
    gbs = moved / (ms * 1e-3) / 1e9
    k_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    k_gbs = moved / (k_ms * 1e-3) / 1e9
    if args.op == "copy_on_write":
        roof = {"bound": "hbm", "achieved": round(2 * k_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(2 * k_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                "algorithmic_bytes_per_launch": 2 * moved, "kernel": "copy_blocks_kernel",
                "timer": "HIP events around each launch on its stream",
                "event_us": round(k_ms * 1e3, 2)}
    else:
        roof = {"bound": "pcie", "achieved": round(k_gbs, 1), "peak": PCIE_PEAK_GBS,
                "unit": "GB/s", "frac": round(k_gbs / PCIE_PEAK_GBS, 4), "traffic": None,
                "algorithmic_bytes_per_launch": moved, "kernel": "copy_blocks_kernel",
                "timer": "HIP events around each launch on its stream",
                "event_us": round(k_ms * 1e3, 2)}
    # the runtime's copy of contiguous buffers of the same size, rotated the same way
    nb = moved // 2
    if args.op == "copy_on_write":
        bufs = [(torch.empty(nb, dtype=torch.uint8, device=dev),
                 torch.empty(nb, dtype=torch.uint8, device=dev)) for _ in range(nsets)]
    elif args.op == "swap_out":
        bufs = [(torch.empty(nb, dtype=torch.uint8, pin_memory=True),
                 torch.empty(nb, dtype=torch.uint8, device=dev)) for _ in range(nsets)]
    else:
        bufs = [(torch.empty(nb, dtype=torch.uint8, device=dev),
                 torch.empty(nb, dtype=torch.uint8, pin_memory=True)) for _ in range(nsets)]
    for i in range(nsets):
        bufs[i][0].copy_(bufs[i][1], non_blocking=True)
    torch.cuda.synchronize()
    f0 = torch.cuda.Event(enable_timing=True); f0.record(stream)
    for i in range(20):
        bufs[i % nsets][0].copy_(bufs[i % nsets][1], non_blocking=True)
    f1 = torch.cuda.Event(enable_timing=True); f1.record(stream)
    torch.cuda.synchronize()
    ref = round(nb * (1 if args.op != "copy_on_write" else 2) /
                (f0.elapsed_time(f1) / 20 * 1e-3) / 1e9, 1)
    result = {
        "metric": f"pa_copy_blocks {args.op} GB/s", "value": round(gbs, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": case.dtype, "data": "synthetic",
        "config": {"workload": f"{args.op} of {k} {case.name} sequences, rotating over "
                               f"{nsets} groups",
                   "blocks_per_group": ns, "block_bytes": block_bytes,
                   "bytes_moved_per_launch": moved},
        "roofline": roof,
        ("contiguous_copy_traffic_GBs" if args.op == "copy_on_write"
         else "contiguous_copy_engine_GBs"): ref,
    }
    if not args.no_cpu_baseline:
        import oracle
        n = ns[0]
        m = torch.stack([srcs[0], torch.arange(n, dtype=torch.int64)], 1)
        dst = torch.zeros((n,) + shape, dtype=case.key_cache.dtype)
        runs, t = 0, 0.0
        while t < 2.0 or runs == 0:
            t0 = time.perf_counter()
            oracle.copy_blocks(case.key_cache, case.value_cache, dst, dst.clone(), m)
            t += time.perf_counter() - t0
            runs += 1
        result["cpu_baseline"] = {"value": round(2 * n * block_bytes / (t / runs) / 1e9, 3),
                                  "unit": "GB/s", "cores": 1, "kind": "oracle",
                                  "sample": f"the first group's {n} blocks copied on the host, "
                                            f"{runs} runs"}
    print(json.dumps(result), flush=True)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _omp():
    """The OpenMP runtime the oracle library is linked against."""
    import ctypes
    try:
        return ctypes.CDLL("libgomp.so.1")
    except OSError:
        return None


def cpu_baseline(case, fp8, min_seconds, max_seconds, kv_bytes):
    """The fp64 oracle (test infrastructure, as it stands) on the same step:
    the cache write of the new tokens, decode over every sequence and, for the
    chunked-prefill workload, the prefill chunks.  First on all of this host's
    threads, repeated until min_seconds have passed; then on one thread over a
    sample of the sequences, scaled by the sample's share of the KV bytes.
    Neither part runs past max_seconds in total."""
    import oracle
    t_begin = time.perf_counter()
    omp = _omp()
    threads = omp.omp_get_max_threads() if omp else int(os.environ.get("OMP_NUM_THREADS", 1))
    if fp8:
        # Seeded random e4m3 codes (NaN codes excluded) in the pool shapes: the
        # oracle's time does not depend on the values, and encoding the whole
        # pools with its table search would take minutes.  Untimed.
        g = torch.Generator().manual_seed(0)
        NB, Hkv_, B_, D_ = case.key_cache.shape
        kc0 = torch.randint(0, 256, (NB, Hkv_, B_, D_), dtype=torch.uint8, generator=g)
        vc0 = torch.randint(0, 256, (NB, Hkv_, D_, B_), dtype=torch.uint8, generator=g)
        for t in (kc0, vc0):
            t[(t & 0x7F) == 0x7F] -= 1

        def dec(q, bt, lens):
            return oracle.decode_fp8(q, kc, vc, bt, lens, case.scale, FP8_K_SCALE, FP8_V_SCALE)
    else:
        kc0, vc0 = case.key_cache, case.value_cache

        def dec(q, bt, lens):
            return oracle.decode(q, kc, vc, bt, lens, case.scale)
    kc, vc = kc0, vc0

    def full_step():
        nonlocal kc, vc
        if case.slot_mapping.numel():
            if fp8:
                kc, vc = oracle.reshape_and_cache_fp8(case.new_key, case.new_value, kc0, vc0,
                                                      case.slot_mapping, FP8_K_SCALE, FP8_V_SCALE)
            else:
                kc, vc = oracle.reshape_and_cache(case.new_key, case.new_value, kc0, vc0,
                                                  case.slot_mapping)
        dec(case.query, case.block_tables, case.context_lens)
        if case.num_chunks:
            args = (case.chunk_query, kc, vc, case.chunk_block_tables, case.chunk_cu_query_lens,
                    case.chunk_context_lens, case.scale)
            if fp8:
                oracle.prefill_fp8(*args, FP8_K_SCALE, FP8_V_SCALE)
            else:
                oracle.prefill(*args)

    budget = max_seconds * 0.6
    runs, t = 0, 0.0
    while runs == 0 or (t < min_seconds and t + t / runs < budget):
        t0 = time.perf_counter()
        full_step()
        t += time.perf_counter() - t0
        runs += 1
    per = t / runs
    what = "cache write + decode" + (" + prefill chunks" if case.num_chunks else "")
    out = {"value": round(kv_bytes / per / 1e9, 3), "unit": "GB/s", "cores": threads,
           "kind": "oracle", "cpu_model": _cpu_model(),
           "sample": f"full {case.name} step ({what}; all {case.num_seqs} seqs x "
                     f"{case.num_q_heads} q heads, fp64{', FP8 pools of random codes' if fp8 else ''}), "
                     f"{runs} runs, {per * 1e3:.1f} ms per run on {threads} threads"}
    # One thread, on the first sequences: as many as fit the remaining time
    # at the measured rate (a thread is at most `threads` times slower).
    left = max(0.5, max_seconds - (time.perf_counter() - t_begin))
    lens = case.context_lens.tolist()
    n = 1
    est = per * threads / max(1, sum(lens))  # seconds per context token on one thread
    while n < len(lens) and est * sum(lens[:n + 1]) < min(left * 0.8, min_seconds):
        n += 1
    if omp is not None:
        omp.omp_set_num_threads(1)
    try:
        t0 = time.perf_counter()
        dec(case.query[:n].contiguous(), case.block_tables[:n].contiguous(),
            case.context_lens[:n].contiguous())
        t1 = time.perf_counter() - t0
    finally:
        if omp is not None:
            omp.omp_set_num_threads(threads)
    Hkv, D = case.num_kv_heads, case.head_dim
    eb = 1 if fp8 else case.key_cache.element_size()
    sample_bytes = sum(lens[:n]) * acct.kv_bytes_per_token(1, Hkv, D, eb)
    out["one_thread"] = {"value": round(sample_bytes / t1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                         "sample": f"decode of the first {n} of {len(lens)} sequences "
                                   f"({sum(lens[:n])} context tokens), {t1:.2f} s",
                         "enforced": omp is not None}
    out["seconds"] = round(time.perf_counter() - t_begin, 2)
    return out


if __name__ == "__main__":
    main()
