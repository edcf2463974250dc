// Launchers of the gfx950 kernels, called by the C ABI layer after it has
// validated every host-side argument.  Each returns the HIP launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

hipError_t launch_reshape_and_cache(const void *key, const void *value, void *key_cache,
                                    void *value_cache, const int64_t *slot_mapping,
                                    int num_tokens, int num_kv_heads, int head_dim,
                                    int block_size, int64_t num_blocks, int elem_bytes,
                                    hipStream_t stream);

// Writes the new token of each sequence s (rows key[s], value[s], [S][Hkv][D])
// into the slot of position context_lens[s] - 1; sequences whose length is 0
// or above max_tokens, or whose block-table entry is outside the pool, are
// skipped.
// Cache write into e4m3 pools: element x of a new row is stored as the
// e4m3 code of x * inv_scale (fp32 multiply, round to nearest even,
// saturating at +-448, NaN -> 0x7F); K at [blk][h][off][d], V at
// [blk][h][d][off].  elem_bytes (4 or 2) is that of the new rows.
hipError_t launch_reshape_and_cache_fp8(const void *key, const void *value, void *key_cache,
                                        void *value_cache, const int64_t *slot_mapping,
                                        int num_tokens, int num_kv_heads, int head_dim,
                                        int block_size, int64_t num_blocks, int elem_bytes,
                                        float k_inv_scale, float v_inv_scale, hipStream_t stream);

hipError_t launch_append_rows(const void *key, const void *value, void *key_cache,
                              void *value_cache, const int32_t *block_tables,
                              const int32_t *context_lens, int num_seqs, int num_kv_heads,
                              int head_dim, int block_size, int max_blocks_per_seq,
                              int64_t num_blocks, int max_tokens, int elem_bytes,
                              hipStream_t stream);

// Largest batch the balanced (stream) decode split handles: its workgroups
// scan the per-sequence unit counts in LDS.  Larger batches use fixed
// partitions.
constexpr int kStreamMaxSeqs = 8192;
// Waves the balanced split spreads the work over: one per SIMD of MI355X's
// 256 CUs.  With two waves per SIMD the older one wins most of the memory
// issue slots and the younger one finishes far later, so the kernel ends on a
// long tail; one wave per SIMD with the same loads in flight ends sooner.  A
// constant, so results do not depend on the device.
#ifndef PA_STREAM_WAVES
#define PA_STREAM_WAVES 1024
#endif
constexpr int kStreamWaves = PA_STREAM_WAVES;

struct DecodeArgs {
    void *out;
    const void *query, *key_cache, *value_cache;
    const int32_t *block_tables, *context_lens;
    int num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq;
    int64_t num_blocks;
    int max_context_len, partition_size, num_partitions;
    int stream_waves;  // > 0: balanced split over this many waves; 0: fixed partitions
    // Nonzero (with stream_waves == S * Hkv): one wave per (sequence, kv head)
    // pair instead of the equal split, so every pair is finished by its own
    // wave and no reduce runs.  Chosen for small batches of short contexts,
    // where the equal split would cut every pair into single units.
    int pairs;
    float scale;
    int dtype;  // 0 f32, 1 bf16
    // Workspace.  Fixed partitions: ws_o [S][Hq][num_partitions][D] and ws_ml
    // [S][Hq][num_partitions][2] (max in log2 units, sum).  Balanced split:
    // records r = pair + wave, ws_o [S*Hkv + waves][G][D], ws_ml [..][G][2],
    // ws_scan [S + 1] (units per sequence, exclusive scan).
    float *ws_o;
    float *ws_ml;
    int *ws_scan;
    // Non-null: the step's new token of each sequence ([S][Hkv][D]) is written
    // at position context_lens[s] - 1 and attended to (decode with append).
    const void *new_key, *new_value;
    // Nonzero: the pools hold e4m3 codes (K [NB][Hkv][B][D], V [NB][Hkv][D][B])
    // of value / k_scale and value / v_scale; query and output are bf16.
    int kv_fp8;
    float k_scale, v_scale;
};

// Copies block mapping[2i] of the source pools to block mapping[2i + 1] of the
// destination pools (block_bytes each, K and V); pairs with an id outside its
// pool are skipped.  The pointers are device addresses (device memory, or
// the device view of pinned host memory).
hipError_t launch_copy_blocks(const void *src_key, const void *src_value, void *dst_key,
                              void *dst_value, const int64_t *mapping, int num_pairs,
                              int64_t src_num_blocks, int64_t dst_num_blocks, int64_t block_bytes,
                              hipStream_t stream);

// Returns hipErrorNotSupported when no kernel is built for the shape.
hipError_t launch_decode_partitions(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_reduce(const DecodeArgs &a, hipStream_t stream);
bool decode_shape_supported(int dtype, int head_dim, int block_size, int group);

struct PrefillArgs {
    void *out;
    const void *query, *key_cache, *value_cache;
    const int32_t *block_tables, *cu_query_lens, *context_lens;
    int num_chunks, max_query_len, num_q_heads, num_kv_heads, head_dim, block_size,
        max_blocks_per_seq;
    int64_t num_blocks;
    float scale;
    // Nonzero: e4m3 pools (K [NB][Hkv][B][D], V [NB][Hkv][D][B]) of value /
    // k_scale and value / v_scale; query and output are bf16.
    int kv_fp8;
    float k_scale, v_scale;
};

hipError_t launch_prefill_chunk(const PrefillArgs &a, hipStream_t stream);
bool prefill_shape_supported(int head_dim, int block_size, int group);

}  // namespace pa
