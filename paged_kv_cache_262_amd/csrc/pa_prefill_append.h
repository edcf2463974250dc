// Launcher of the prefill pass that also writes the chunks' own K/V rows
// (prefill.hip), called by the C ABI layer after it has validated every
// host-side argument.
#pragma once

#include "pa_internal.h"

namespace pa {

// a as for launch_prefill_chunk (bf16 pools); new_key / new_value
// [Tq][Hkv][D] bf16 hold the K/V rows of the chunks' tokens, row i of chunk
// c at position context_lens[c] - n_c + i.
hipError_t launch_prefill_chunk_append(const PrefillArgs &a, const void *new_key,
                                       const void *new_value, hipStream_t stream);

}  // namespace pa
