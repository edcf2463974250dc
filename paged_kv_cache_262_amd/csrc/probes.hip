// Measurement probes: the attainable ceilings the kernels are compared with.
//
// pa_probe_stream_read reads a device buffer once with 16-byte loads and as
// much in flight as the chip takes (the same load width the decode kernels
// use), so bytes / time is the HBM read rate a streaming kernel can reach on
// this part.  pa_probe_mfma_bf16 keeps every SIMD issuing independent
// 32x32x16 bf16 matrix products on register operands, so flops / time is the
// dense bf16 matrix rate the clock sustains under that load (the clock ramps
// up under sustained matrix work, so a caller runs it for some milliseconds
// before timing it).  Neither touches
// the attention data; the bench times them next to the hot path.
#include <stdint.h>

#include "pa_probes.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;  // 16-byte loads in flight per thread

// Workgroup b reads chunks b, b + grid, b + 2 grid, ... of kReadThreads *
// kReadUnroll * 16 bytes (all loads of a chunk issued before any is used);
// a partial last chunk is read lane by lane.  Each thread folds what it read
// into one word so the loads are not removed, and writes it to sink.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4 *__restrict__ src,
                                                                   size_t n16, uint32_t *sink) {
    constexpr size_t chunk = (size_t)kReadThreads * kReadUnroll;
    const size_t nchunks = n16 / chunk;
    u32x4 acc = {0, 0, 0, 0};
    for (size_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const u32x4 *p = src + c * chunk + threadIdx.x;
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int i = 0; i < kReadUnroll; ++i) v[i] = __builtin_nontemporal_load(p + i * kReadThreads);
#pragma unroll
        for (int i = 0; i < kReadUnroll; ++i) acc ^= v[i];
    }
    for (size_t i = nchunks * chunk + (size_t)blockIdx.x * kReadThreads + threadIdx.x; i < n16;
         i += (size_t)gridDim.x * kReadThreads)
        acc ^= src[i];
    sink[(size_t)blockIdx.x * kReadThreads + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

constexpr int kMfmaThreads = 256;  // one wave per SIMD per workgroup
constexpr int kMfmaChains = 4;     // independent accumulators per wave

// Each wave runs iters rounds of kMfmaChains independent 32x32x16 bf16
// products on operands held in registers and writes one word per lane.
__global__ __launch_bounds__(kMfmaThreads) void mfma_peak_kernel(int iters, float *sink) {
    bf16x8_v a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (threadIdx.x + i));
        b[i] = (__bf16)(0.002f * (blockIdx.x + i));
    }
    f32x16 acc[kMfmaChains] = {};
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int c = 0; c < kMfmaChains; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) s += acc[c][0] + acc[c][15];
    sink[(size_t)blockIdx.x * kMfmaThreads + threadIdx.x] = s;
}

}  // namespace

int probe_read_grid() { return 4096; }

hipError_t launch_probe_stream_read(const void *buf, size_t bytes, void *sink, hipStream_t stream) {
    hipLaunchKernelGGL(stream_read_kernel, dim3(probe_read_grid()), dim3(kReadThreads), 0, stream,
                       (const u32x4 *)buf, bytes / 16, (uint32_t *)sink);
    return hipGetLastError();
}

// Four workgroups per CU: four waves per SIMD keep the matrix pipe fed.
int probe_mfma_grid() { return 1024; }

hipError_t launch_probe_mfma_bf16(void *sink, int iters, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_peak_kernel, dim3(probe_mfma_grid()), dim3(kMfmaThreads), 0, stream,
                       iters, (float *)sink);
    return hipGetLastError();
}

double probe_mfma_flops(int iters) {
    return (double)probe_mfma_grid() * (kMfmaThreads / 64) * iters * kMfmaChains * 32.0 * 32.0 *
           16.0 * 2.0;
}

}  // namespace pa
