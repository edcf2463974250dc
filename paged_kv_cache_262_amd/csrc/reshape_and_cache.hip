// Cache write: scatter the K/V rows of new tokens into their physical slots.
//
// Blocks are taken from the pool on demand as sequences grow, so a new
// token's slot can be anywhere in the pool ("Configuring vLLM and
// PagedAttention for High Throughput Enterprise LLM Serving", section
// "Architectural Foundations: PagedAttention & Virtual Memory").  The copy is
// bitwise: 16-byte vector moves, no conversion.
//
// One workgroup per new token.  Its threads cover the token's kv heads x
// 16-byte chunks of both K and V, so every global access is a contiguous
// 16-byte piece of a head row (head_dim * elem bytes = 128..512 bytes).
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint4 *__restrict__ key, const uint4 *__restrict__ value, uint4 *__restrict__ key_cache,
    uint4 *__restrict__ value_cache, const int64_t *__restrict__ slot_mapping, int num_kv_heads,
    int block_size, int chunks_per_row, int64_t num_slots) {
    const int t = blockIdx.x;
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) return;  // padding (or a caller error)
    const int64_t blk = slot / block_size;
    const int off = (int)(slot - blk * block_size);
    const int per_tensor = num_kv_heads * chunks_per_row;
    for (int i = threadIdx.x; i < 2 * per_tensor; i += blockDim.x) {
        const bool is_v = i >= per_tensor;
        const int j = is_v ? i - per_tensor : i;
        const int h = j / chunks_per_row;
        const int c = j - h * chunks_per_row;
        const int64_t src = ((int64_t)t * num_kv_heads + h) * chunks_per_row + c;
        const int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * chunks_per_row + c;
        if (is_v)
            value_cache[dst] = value[src];
        else
            key_cache[dst] = key[src];
    }
}

hipError_t launch_reshape_and_cache(const void *key, const void *value, void *key_cache,
                                    void *value_cache, const int64_t *slot_mapping,
                                    int num_tokens, int num_kv_heads, int head_dim,
                                    int block_size, int64_t num_blocks, int elem_bytes,
                                    hipStream_t stream) {
    const int chunks = head_dim * elem_bytes / 16;
    const int per_token = 2 * num_kv_heads * chunks;
    int threads = per_token >= 256 ? 256 : ((per_token + 63) / 64) * 64;
    hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(num_tokens), dim3(threads), 0, stream,
                       (const uint4 *)key, (const uint4 *)value, (uint4 *)key_cache,
                       (uint4 *)value_cache, slot_mapping, num_kv_heads, block_size, chunks,
                       num_blocks * block_size);
    return hipGetLastError();
}

// The new token of sequence s goes to position context_lens[s] - 1, whose slot
// is block_tables[s][(L - 1) / B] at offset (L - 1) % B.  One workgroup per
// sequence.
__global__ __launch_bounds__(256) void append_rows_kernel(
    const uint4 *__restrict__ key, const uint4 *__restrict__ value, uint4 *__restrict__ key_cache,
    uint4 *__restrict__ value_cache, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, int num_kv_heads, int block_size,
    int max_blocks_per_seq, int64_t num_blocks, int max_tokens, int chunks_per_row) {
    const int s = blockIdx.x;
    const int L = context_lens[s];
    if (L <= 0 || L > max_tokens) return;
    const int pos = L - 1;
    const int64_t blk = block_tables[(int64_t)s * max_blocks_per_seq + pos / block_size];
    if (blk < 0 || blk >= num_blocks) return;  // a caller error: nothing is written
    const int off = pos % block_size;
    const int per_tensor = num_kv_heads * chunks_per_row;
    for (int i = threadIdx.x; i < 2 * per_tensor; i += blockDim.x) {
        const bool is_v = i >= per_tensor;
        const int j = is_v ? i - per_tensor : i;
        const int h = j / chunks_per_row;
        const int c = j - h * chunks_per_row;
        const int64_t src = ((int64_t)s * num_kv_heads + h) * chunks_per_row + c;
        const int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * chunks_per_row + c;
        if (is_v)
            value_cache[dst] = value[src];
        else
            key_cache[dst] = key[src];
    }
}

hipError_t launch_append_rows(const void *key, const void *value, void *key_cache,
                              void *value_cache, const int32_t *block_tables,
                              const int32_t *context_lens, int num_seqs, int num_kv_heads,
                              int head_dim, int block_size, int max_blocks_per_seq,
                              int64_t num_blocks, int max_tokens, int elem_bytes,
                              hipStream_t stream) {
    if (num_seqs == 0) return hipSuccess;
    const int chunks = head_dim * elem_bytes / 16;
    const int per_seq = 2 * num_kv_heads * chunks;
    const int threads = per_seq >= 256 ? 256 : ((per_seq + 63) / 64) * 64;
    hipLaunchKernelGGL(append_rows_kernel, dim3(num_seqs), dim3(threads), 0, stream,
                       (const uint4 *)key, (const uint4 *)value, (uint4 *)key_cache,
                       (uint4 *)value_cache, block_tables, context_lens, num_kv_heads,
                       block_size, max_blocks_per_seq, num_blocks, max_tokens, chunks);
    return hipGetLastError();
}

}  // namespace pa
