// Launchers of the shared-prefix decode (decode.hip), called by the C ABI
// layer after it has validated every host-side argument.
#pragma once

#include "pa_internal.h"

namespace pa {

// The prefix: tokens [0, prefix_tokens) of every sequence, in the pages
// listed by prefix_table[0 .. prefix_tokens / B).  Records: x_o [S * Hq][ksplit][D]
// and x_ml [S * Hq][ksplit][2] (max in log2 units, sum).
struct PrefixArgs {
    const int32_t *prefix_table;
    int prefix_tokens;
    int ksplit;  // 1 .. kPrefixMaxSplits
    float *x_o, *x_ml;
};

constexpr int kPrefixMaxSplits = 8;

// Prefix splits for a batch: about one wave per SIMD, each with at least one
// unit of the prefix.
int prefix_splits(int num_seqs, int num_q_heads, int num_kv_heads, int prefix_tokens);

// a describes the suffix pass: block_tables advanced past the prefix pages,
// max_context_len reduced by the prefix, balanced split over the waves, bf16.
hipError_t launch_decode_prefix(const DecodeArgs &a, const PrefixArgs &p, hipStream_t stream);
// The balanced split over the tokens past the prefix, every pair written as
// records; then the reduce with the prefix records.
hipError_t launch_decode_suffix(const DecodeArgs &a, int len_skip, hipStream_t stream);
hipError_t launch_decode_reduce_prefix(const DecodeArgs &a, const PrefixArgs &p,
                                       hipStream_t stream);

}  // namespace pa
