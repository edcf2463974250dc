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

}  // namespace pa
