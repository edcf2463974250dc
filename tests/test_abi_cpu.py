"""The C ABI library without a GPU: it loads, exports every declared symbol,
and rejects bad arguments on the host before anything is launched."""
import ctypes
import os
import re

import pytest

from paged_kv_cache_262_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = range(5)
# Fake device addresses: never dereferenced, every call below fails its host
# checks before any launch.
A = 0x10000
A2 = 0x20000


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        from paged_kv_cache_262_amd import build
        build.build()
    return binding.load()


def test_every_declared_symbol_is_exported(lib):
    syms = declared_symbols()
    assert len(syms) >= 10
    for s in syms:
        assert hasattr(lib, s), s
        assert s in binding.SIGNATURES, f"binding lacks {s}"


def test_status_strings_and_version(lib):
    assert lib.pa_abi_version() == 1
    names = [lib.pa_status_string(i).decode() for i in range(6)]
    assert names == ["PA_OK", "PA_ERR_INVALID_ARG", "PA_ERR_UNSUPPORTED", "PA_ERR_WORKSPACE",
                     "PA_ERR_HIP", "PA_ERR_POOL_EXHAUSTED"]


def test_auto_partition_and_workspace(lib):
    P = lib.pa_decode_auto_partition_size(64, 8, 4096, 16)
    assert P % 16 == 0 and 64 <= P <= 1024
    # fixed partitions: (max, sum, output) per (seq, q head, partition)
    np_ = -(-4096 // 512)
    need = lib.pa_decode_workspace_bytes(64, 32, 8, 128, 16, 4096, 512)
    assert need >= 64 * 32 * np_ * (128 + 2) * 4
    # balanced split: one record per (seq, kv head) plus one per wave (1024 waves),
    # G heads each, and the unit scan
    need = lib.pa_decode_workspace_bytes(64, 32, 8, 128, 16, 4096, 0)
    assert need >= (64 * 8 + 1024) * 4 * (128 + 2) * 4 + 65 * 4
    # one partition needs no real workspace
    assert lib.pa_decode_workspace_bytes(4, 4, 4, 64, 16, 100, 128) == 256


def test_decode_needs_reduce(lib):
    """One wave per (sequence, kv head) pair, so no second launch, for at most
    1,024 pairs with no context above 8 units of 16 tokens; the equal split
    and the fixed partitions always reduce."""
    f = lib.pa_decode_needs_reduce
    assert f(4, 4, 4, 64, 16, 100, 0) == 0
    assert f(64, 32, 8, 128, 16, 4096, 0) == 1        # 8B decode batch
    assert f(0, 32, 8, 128, 16, 4096, 0) == 0         # nothing to do
    assert f(4, 4, 4, 64, 16, 100, 128) == 1          # fixed partitions
    assert f(128, 32, 8, 128, 16, 128, 0) == 0        # 1,024 pairs of 8 units
    assert f(129, 32, 8, 128, 16, 128, 0) == 1        # 1,032 pairs
    assert f(128, 32, 8, 128, 16, 129, 0) == 1        # 9 units
    assert f(4, 6, 4, 64, 16, 100, 0) == 1            # invalid sizes
    assert f(-1, 4, 4, 64, 16, 100, 0) == 1


def _decode(lib, **kw):
    a = dict(out=A, query=A, kc=A, vc=A, bt=A, lens=A, S=4, Hq=8, Hkv=2, D=128, B=16, mbs=8,
             NB=32, maxL=100, P=0, scale=0.1, dtype=1, ws=A2, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.pa_decode(a["out"], a["query"], a["kc"], a["vc"], a["bt"], a["lens"], a["S"],
                         a["Hq"], a["Hkv"], a["D"], a["B"], a["mbs"], a["NB"], a["maxL"], a["P"],
                         a["scale"], a["dtype"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=6, Hkv=4), INVALID),            # Hq not a multiple of Hkv
    (dict(Hq=0), INVALID),
    (dict(D=96), UNSUPPORTED),
    (dict(B=8), UNSUPPORTED),
    (dict(Hq=32, Hkv=2), UNSUPPORTED),       # group 16 not built
    (dict(dtype=7), UNSUPPORTED),
    (dict(query=0), INVALID),                # NULL
    (dict(kc=A + 4), INVALID),               # misaligned
    (dict(maxL=8 * 16 + 1), INVALID),        # beyond table capacity
    (dict(P=24), INVALID),                   # not a multiple of the block size
    (dict(scale=float("nan")), INVALID),
    (dict(ws=0, maxL=100, P=64), WORKSPACE),
    (dict(wsb=16, maxL=100, P=64), WORKSPACE),
    (dict(NB=0), INVALID),
    (dict(S=-1), INVALID),
])
def test_decode_rejects(lib, kw, status):
    assert _decode(lib, **kw) == status
    assert lib.pa_last_error().decode()


def test_reshape_rejects(lib):
    f = lib.pa_reshape_and_cache
    assert f(A, A, A, A, A, -1, 8, 128, 16, 10, 1, None) == INVALID
    assert f(A, A, A, A, A, 4, 8, 100, 16, 10, 1, None) == UNSUPPORTED
    assert f(0, A, A, A, A, 4, 8, 128, 16, 10, 1, None) == INVALID
    assert f(A, A, A, A, A + 4, 4, 8, 128, 16, 10, 1, None) == INVALID  # slots misaligned
    assert f(A, A, A, A, A, 4, 8, 128, 16, 0, 1, None) == INVALID
    assert f(0, 0, 0, 0, 0, 0, 8, 128, 16, 10, 1, None) == OK  # nothing to do


def test_prefill_rejects(lib):
    f = lib.pa_prefill_chunk
    args = [A, A, A, A, A, A, A, 2, 512, 32, 8, 128, 16, 160, 1000, 0.1]
    assert f(*args, 0, None) == UNSUPPORTED          # fp32 prefill
    bad = list(args); bad[9] = 7                       # 32 % 7
    assert f(*bad, 1, None) == INVALID
    bad = list(args); bad[1] = 0
    assert f(*bad, 1, None) == INVALID
    bad = list(args); bad[8] = -1                      # max_query_len
    assert f(*bad, 1, None) == INVALID
    for sc in (0.0, -0.1, float("inf"), float("nan")):  # the scale must be positive, finite
        bad = list(args); bad[15] = sc
        assert f(*bad, 1, None) == INVALID, sc
        assert "scale" in lib.pa_last_error().decode()


def test_binding_refuses_cpu_tensors(lib):
    import torch
    q = torch.zeros(2, 4, 64)
    with pytest.raises(ValueError):
        binding.reshape_and_cache(q, q, torch.zeros(4, 4, 16, 64), torch.zeros(4, 4, 16, 64),
                                  torch.zeros(2, dtype=torch.int64))


def test_fp8_reshape_rejects(lib):
    f = lib.pa_reshape_and_cache_fp8
    ok = [A, A, A, A, A, 4, 8, 128, 16, 10, 1]
    assert f(*ok, 0.0, 1.0, None) == INVALID                  # scale must be positive
    assert f(*ok, 1.0, float("inf"), None) == INVALID
    assert f(*ok, 1.0, float("nan"), None) == INVALID
    bad = list(ok); bad[10] = 2                                # new rows as FP8: not supported
    assert f(*bad, 1.0, 1.0, None) == UNSUPPORTED
    bad = list(ok); bad[7] = 96
    assert f(*bad, 1.0, 1.0, None) == UNSUPPORTED
    bad = list(ok); bad[2] = A + 4                             # misaligned pool
    assert f(*bad, 1.0, 1.0, None) == INVALID
    assert f(0, 0, 0, 0, 0, 0, 8, 128, 16, 10, 1, 1.0, 1.0, None) == OK


def _decode_fp8(lib, **kw):
    a = dict(out=A, query=A, kc=A, vc=A, bt=A, lens=A, S=4, Hq=8, Hkv=2, D=128, B=16, mbs=8,
             NB=32, maxL=100, scale=0.1, ks=1.0, vs=1.0, ws=A2, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.pa_decode_fp8(a["out"], a["query"], a["kc"], a["vc"], a["bt"], a["lens"], a["S"],
                             a["Hq"], a["Hkv"], a["D"], a["B"], a["mbs"], a["NB"], a["maxL"],
                             a["scale"], a["ks"], a["vs"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(ks=0.0), INVALID),
    (dict(vs=-1.0), INVALID),
    (dict(ks=float("nan")), INVALID),
    (dict(S=8193), UNSUPPORTED),             # beyond the balanced split
    (dict(Hq=32, Hkv=2), UNSUPPORTED),       # group 16 not built
    (dict(D=96), UNSUPPORTED),
    (dict(query=0), INVALID),
    (dict(vc=A + 4), INVALID),
    (dict(maxL=8 * 16 + 1), INVALID),
    (dict(wsb=16), WORKSPACE),
    (dict(ws=0), WORKSPACE),
])
def test_decode_fp8_rejects(lib, kw, status):
    assert _decode_fp8(lib, **kw) == status
    assert lib.pa_last_error().decode()


def test_fp8_prefill_rejects(lib):
    f = lib.pa_prefill_chunk_fp8
    args = [A, A, A, A, A, A, A, 2, 512, 32, 8, 128, 16, 160, 1000, 0.1]
    assert f(*args, 0.0, 1.0, None) == INVALID                     # scale must be positive
    assert f(*args, 1.0, float("nan"), None) == INVALID
    for sc in (0.0, -0.1):                                          # so must the attention scale
        bad = list(args); bad[15] = sc
        assert f(*bad, 1.0, 1.0, None) == INVALID, sc
    bad = list(args); bad[9] = 7                                    # 32 % 7
    assert f(*bad, 1.0, 1.0, None) == INVALID
    bad = list(args); bad[11] = 96
    assert f(*bad, 1.0, 1.0, None) == UNSUPPORTED
    bad = list(args); bad[3] = A + 4                                # misaligned V pool
    assert f(*bad, 1.0, 1.0, None) == INVALID
    bad = list(args); bad[7] = 0                                    # no chunks: nothing to do
    assert f(*bad, 1.0, 1.0, None) == OK


def test_no_alloc_decode_rejects_on_the_host(lib):
    """pa_decode_no_alloc checks its arguments, and the size of the workspace
    the plan needs against its static array, before any device call."""
    f = lib.pa_decode_no_alloc
    assert lib.pa_decode_no_alloc_max_workspace() == 32 << 20
    args = [A, A, A, A, A, A, 8192, 8, 2, 128, 16, 3, 4, 40, 0, 0.1, 1, None]
    assert f(*args) == WORKSPACE                      # ~34.6 MiB of records
    assert "static scratch" in lib.pa_last_error().decode()
    bad = list(args); bad[6] = 64; bad[1] = 0         # NULL query
    assert f(*bad) == INVALID
    bad = list(args); bad[6] = 64; bad[9] = 96        # head_dim not built
    assert f(*bad) == UNSUPPORTED
    bad = list(args); bad[6] = 0                      # no sequences: nothing to do
    assert f(*bad) == OK


def test_probes_reject_bad_arguments_on_the_host(lib):
    # checked before any device call
    assert lib.pa_probe_sink_words() >= 4096 * 256
    assert lib.pa_probe_stream_read(None, 16, None, None) == 1
    assert lib.pa_probe_stream_read(None, 0, None, None) == 1
    assert lib.pa_probe_stream_read(None, 24, None, None) == 1
    assert b"multiple of 16" in lib.pa_last_error()
    assert lib.pa_probe_mfma_bf16(None, 0, None, None) == 1
    assert b"iters" in lib.pa_last_error()
    assert lib.pa_probe_mfma_bf16(None, 5, None, None) == 1


def test_shared_prefix_rejects_on_the_host(lib):
    """Argument checks of pa_decode_shared_prefix that run before any device call."""
    f = lib.pa_decode_shared_prefix
    f.restype = ctypes.c_int32
    f.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int32] * 6 + [ctypes.c_int64, ctypes.c_int32,
                  ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t,
                  ctypes.c_void_p]
    args = lambda S=4, mbs=10, maxL=100, pb=2, ws=None, D=128, G=4: (
        None, None, None, None, None, None, S, 8 * G, 8, D, 16, mbs, 100, maxL, pb, 0.1, ws, 0,
        None)
    assert f(*args(pb=-1)) == 1 and b"prefix_blocks" in lib.pa_last_error()
    assert f(*args(pb=11)) == 1
    assert f(*args(S=8193)) == 2
    assert f(*args(maxL=161)) == 1
    assert f(*args(D=96)) == 2
    assert f(*args()) == 3 and b"workspace" in lib.pa_last_error()
    assert f(*args(S=0)) == 0  # nothing to do


def test_fp8_shared_prefix_rejects_on_the_host(lib):
    """pa_decode_fp8_shared_prefix: the shared-prefix checks, and the pools'
    scales, before any device call."""
    f = lib.pa_decode_fp8_shared_prefix
    args = lambda S=4, mbs=10, maxL=100, pb=2, ws=None, D=128, G=4, ks=0.5, vs=0.25: (
        None, None, None, None, None, None, S, 8 * G, 8, D, 16, mbs, 100, maxL, pb, 0.1, ks, vs,
        ws, 0, None)
    assert f(*args(ks=0.0)) == 1 and b"k_scale" in lib.pa_last_error()
    assert f(*args(vs=float("inf"))) == 1
    assert f(*args(ks=float("nan"))) == 1
    assert f(*args(pb=-1)) == 1 and b"prefix_blocks" in lib.pa_last_error()
    assert f(*args(S=8193)) == 2
    assert f(*args(D=96)) == 2
    assert f(*args()) == 3 and b"workspace" in lib.pa_last_error()
    assert f(*args(S=0)) == 0  # nothing to do


def test_shared_prefix_workspace_covers_suffix_and_prefix_records(lib):
    w = lib.pa_decode_shared_prefix_workspace_bytes
    w.restype = ctypes.c_size_t
    w.argtypes = [ctypes.c_int32] * 7
    d = lib.pa_decode_workspace_bytes
    d.restype = ctypes.c_size_t
    d.argtypes = [ctypes.c_int32] * 7
    # no prefix: exactly the balanced decode's workspace
    assert w(128, 32, 8, 128, 16, 3072, 0) == d(128, 32, 8, 128, 16, 3072, 0)
    # 128 seqs, 64-block prefix: the suffix split (max 2048 tokens past the
    # prefix) plus 4 prefix records of 130 floats per (sequence, q head)
    base = d(128, 32, 8, 128, 16, 3072 - 1024, 0)
    assert w(128, 32, 8, 128, 16, 3072, 64) == base + 128 * 32 * 4 * 128 * 4 + 128 * 32 * 4 * 8
