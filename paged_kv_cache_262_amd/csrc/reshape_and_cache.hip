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

// ---- FP8 (e4m3) cache write ---------------------------------------------------
//
// Quantised KV cache ("vLLM Guide: High-Throughput Multi-GPU LLM Serving with
// PagedAttention", the quantisation support among the engine's pillars and
// its FP8 engine example): each element is kept as an 8-bit e4m3 code (sign,
// 4 exponent bits with bias 7, 3 mantissa bits; no infinities; S.1111.111 is
// NaN; largest finite 448, smallest subnormal 2^-9) of x / scale, one fp32
// scale per pool.  The pages fix no rounding: x / scale is taken as one fp32
// multiply by 1 / scale (computed on the host), then rounded to the nearest
// e4m3 value, ties to the even code, saturating at +-448; NaN gives 0x7F.

template <typename T>
__device__ __forceinline__ void load4(const T *p, float (&x)[4]) {
    if constexpr (sizeof(T) == 4) {
        const float4 v = *(const float4 *)p;
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    } else {
        const uint2 v = *(const uint2 *)p;
        x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    }
}

template <typename T>
__device__ __forceinline__ float load1(const T *p) {
    if constexpr (sizeof(T) == 4)
        return *p;
    else
        return __uint_as_float((uint32_t)*(const uint16_t *)p << 16);
}

// One workgroup per (group of kFp8Group consecutive new tokens, kv head).
// When the group's slots are kFp8Group consecutive slots starting at a
// multiple of kFp8Group (a chunk's tokens filling that part of a block), the
// group's V codes of one dim form one 16-byte segment of a transposed V page
// row, written whole, and its K rows are contiguous, so every store of the
// workgroup covers whole 16-byte pieces.  Otherwise each token of the group is
// written on its own: a thread takes 4 consecutive dims, one 4-byte store into
// the K row and four byte stores down the dims of the V page (each lands in
// its own row of the page).
constexpr int kFp8Group = 16;

template <typename T>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const T *__restrict__ key, const T *__restrict__ value, uint8_t *__restrict__ key_cache,
    uint8_t *__restrict__ value_cache, const int64_t *__restrict__ slot_mapping, int num_tokens,
    int num_kv_heads, int head_dim, int block_size, int64_t num_slots, float k_inv,
    float v_inv) {
    __shared__ int64_t sl[kFp8Group];
    const int t0 = blockIdx.x * kFp8Group, h = blockIdx.y;
    const int nt = min(kFp8Group, num_tokens - t0);
    if (threadIdx.x < kFp8Group) sl[threadIdx.x] = threadIdx.x < nt ? slot_mapping[t0 + threadIdx.x] : -1;
    __syncthreads();
    const int64_t s0 = sl[0];
    bool full = nt == kFp8Group && s0 >= 0 && s0 + kFp8Group <= num_slots && s0 % kFp8Group == 0;
#pragma unroll
    for (int i = 1; i < kFp8Group; ++i) full = full && sl[i] == s0 + i;
    const int D = head_dim, B = block_size;
    if (full) {
        // The group lies in one block (block size is a multiple of 16), at
        // offsets off0 .. off0 + 15.  Lanes 4d .. 4d + 3 encode the 16 codes
        // of V row d (4 tokens each) and store them as one contiguous 16-byte
        // piece; consecutive lanes cover consecutive 4-byte pieces of the
        // group's K rows, which are contiguous in the page.
        const int64_t blk = s0 / B;
        const int off0 = (int)(s0 - blk * B);
        const int64_t page = (blk * num_kv_heads + h) * (int64_t)B * D;
        const int64_t row0 = (int64_t)t0 * num_kv_heads + h;  // row of token t0, head h
        for (int j = threadIdx.x; j < 4 * D; j += blockDim.x) {
            const int d = j >> 2, q = j & 3;
            uint32_t w = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = load1(value + (row0 + (int64_t)(4 * q + e) * num_kv_heads) * D + d);
                w |= e4m3_code(x * v_inv) << (8 * e);
            }
            *(uint32_t *)(value_cache + page + (int64_t)d * B + off0 + 4 * q) = w;
        }
        const int quads = D / 4;
        for (int j = threadIdx.x; j < kFp8Group * quads; j += blockDim.x) {
            const int i = j / quads, d0 = (j - i * quads) * 4;
            float k[4];
            load4(key + (row0 + (int64_t)i * num_kv_heads) * D + d0, k);
            uint32_t w = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) w |= e4m3_code(k[e] * k_inv) << (8 * e);
            *(uint32_t *)(key_cache + page + (int64_t)(off0 + i) * D + d0) = w;
        }
        return;
    }
    const int quads = D / 4;
    for (int j = threadIdx.x; j < nt * quads; j += blockDim.x) {
        const int i = j / quads, d0 = (j - i * quads) * 4;
        const int64_t slot = sl[i];
        if (slot < 0 || slot >= num_slots) continue;  // padding (or a caller error)
        const int64_t blk = slot / B;
        const int off = (int)(slot - blk * B);
        const int64_t src = ((int64_t)(t0 + i) * num_kv_heads + h) * D + d0;
        const int64_t page = (blk * num_kv_heads + h) * (int64_t)B * D;
        float k[4], v[4];
        load4(key + src, k);
        load4(value + src, v);
        uint32_t kw = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) kw |= e4m3_code(k[e] * k_inv) << (8 * e);
        *(uint32_t *)(key_cache + page + (int64_t)off * D + d0) = kw;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            value_cache[page + (int64_t)(d0 + e) * B + off] = (uint8_t)e4m3_code(v[e] * v_inv);
    }
}

hipError_t launch_reshape_and_cache_fp8(const void *key, const void *value, void *key_cache,
                                        void *value_cache, const int64_t *slot_mapping,
                                        int num_tokens, int num_kv_heads, int head_dim,
                                        int block_size, int64_t num_blocks, int elem_bytes,
                                        float k_inv_scale, float v_inv_scale, hipStream_t stream) {
    if (num_tokens == 0) return hipSuccess;
    const dim3 grid((unsigned)((num_tokens + kFp8Group - 1) / kFp8Group), (unsigned)num_kv_heads);
    if (elem_bytes == 4)
        hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<float>, grid, dim3(256), 0, stream,
                           (const float *)key, (const float *)value, (uint8_t *)key_cache,
                           (uint8_t *)value_cache, slot_mapping, num_tokens, num_kv_heads,
                           head_dim, block_size, num_blocks * block_size, k_inv_scale,
                           v_inv_scale);
    else
        hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<bf16_t>, grid, dim3(256), 0, stream,
                           (const bf16_t *)key, (const bf16_t *)value, (uint8_t *)key_cache,
                           (uint8_t *)value_cache, slot_mapping, num_tokens, num_kv_heads,
                           head_dim, block_size, num_blocks * block_size, k_inv_scale,
                           v_inv_scale);
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
