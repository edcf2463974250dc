"""MI355X-native paged KV-cache attention (PagedAttention).

The compute lives in ``libpa.so`` (hand-written HIP kernels for gfx950 behind a
plain C ABI, declared in ``include/pa.h``).  This package is the thin Python
binding over it: argument marshalling from torch tensors to pointers and the
caller's current HIP stream.  Nothing here computes attention; if the shared
library is missing every entry point raises.
"""
from .binding import (  # noqa: F401
    BlockManager,
    PAError,
    copy_blocks,
    decode,
    decode_append,
    decode_append_partitions,
    decode_partitions,
    decode_reduce,
    decode_workspace_bytes,
    library_path,
    prefill_chunk,
    reshape_and_cache,
)
