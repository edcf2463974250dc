// Prefill chunk attention (bf16 MFMA) -- placeholder until the kernel lands.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

bool prefill_shape_supported(int, int, int) { return false; }

hipError_t launch_prefill_chunk(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pa
