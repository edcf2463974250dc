// Whole-block copies between KV pools.
//
// Physical blocks shared by several sequences are copied before one of them
// writes into its own copy ("vLLM Guide: High-Throughput Multi-GPU LLM Serving
// with PagedAttention", section "What Is PagedAttention?": copy-on-write
// sharing), and under memory pressure the pages of a paused request move to
// host memory over PCIe and later back ("Configuring vLLM and PagedAttention
// for High Throughput Enterprise LLM Serving", section "Quick Answers", the
// question on KV-cache offloading).  Both are the same gather: block
// mapping[2i] of the source pools goes to block mapping[2i + 1] of the
// destination pools, K and V, bit for bit.  The pools may be device memory
// or pinned host memory mapped into the device's address space; the blocks
// of a paused request are scattered over the pool, so one launch moves them
// all instead of one copy command per block.
//
// One workgroup per (pair, tensor, 16 KiB part of a block).  Each thread moves
// four 16-byte chunks, all loads before the stores, so a wave keeps 4 KiB in
// flight (the latency of a host-memory read is several microseconds).
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
constexpr int kCopyPart = kCopyThreads * kCopyUnroll;  // 16-byte chunks per workgroup

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    const uint4 *__restrict__ src_key, const uint4 *__restrict__ src_value,
    uint4 *__restrict__ dst_key, uint4 *__restrict__ dst_value,
    const int64_t *__restrict__ mapping, int64_t src_num_blocks, int64_t dst_num_blocks,
    int64_t chunks_per_block) {
    const int64_t pair = blockIdx.x;
    const int64_t s = mapping[2 * pair], d = mapping[2 * pair + 1];
    if (s < 0 || s >= src_num_blocks || d < 0 || d >= dst_num_blocks) return;  // caller error
    const uint4 *src = (blockIdx.y ? src_value : src_key) + s * chunks_per_block;
    uint4 *dst = (blockIdx.y ? dst_value : dst_key) + d * chunks_per_block;
    const int64_t base = (int64_t)blockIdx.z * kCopyPart + threadIdx.x;
    uint4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kCopyThreads;
        if (i < chunks_per_block) v[u] = src[i];
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kCopyThreads;
        if (i < chunks_per_block) dst[i] = v[u];
    }
}

hipError_t launch_copy_blocks(const void *src_key, const void *src_value, void *dst_key,
                              void *dst_value, const int64_t *mapping, int num_pairs,
                              int64_t src_num_blocks, int64_t dst_num_blocks, int64_t block_bytes,
                              hipStream_t stream) {
    const int64_t chunks = block_bytes / 16;
    const dim3 grid((unsigned)num_pairs, 2, (unsigned)((chunks + kCopyPart - 1) / kCopyPart));
    hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kCopyThreads), 0, stream,
                       (const uint4 *)src_key, (const uint4 *)src_value, (uint4 *)dst_key,
                       (uint4 *)dst_value, mapping, src_num_blocks, dst_num_blocks, chunks);
    return hipGetLastError();
}

}  // namespace pa
