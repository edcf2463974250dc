// Launchers of the ceiling probes (probes.hip), called by the C ABI layer
// after it has validated the arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace pa {

// stream_read reads bytes (a multiple of 16) of buf once and writes
// probe_read_grid() * 256 words to sink; mfma_bf16 writes probe_mfma_grid() *
// 256 floats to sink and performs probe_mfma_flops(iters) flops of bf16
// matrix products.
int probe_read_grid();
hipError_t launch_probe_stream_read(const void *buf, size_t bytes, void *sink, hipStream_t stream);
int probe_mfma_grid();
hipError_t launch_probe_mfma_bf16(void *sink, int iters, hipStream_t stream);
double probe_mfma_flops(int iters);

}  // namespace pa
