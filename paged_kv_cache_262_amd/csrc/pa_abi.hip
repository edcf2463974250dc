// C ABI of libpa.so (include/pa.h): host-side argument checks, launch
// geometry and error reporting.  No allocation, no synchronisation.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "pa.h"
#include "pa_internal.h"
#include "pa_prefill_append.h"
#include "pa_prefix.h"
#include "pa_probes.h"

namespace {

thread_local char g_error[512] = "";

pa_status fail(pa_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
    return st;
}

pa_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return PA_OK;
    if (e == hipErrorNotSupported) return fail(PA_ERR_UNSUPPORTED, "%s: shape not built", what);
    return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr size_t kMinWorkspace = 256;
constexpr int kMinPartition = 64;
constexpr int kMaxPartition = 4096;  // 64 units of 16 tokens per wave, 4 waves

#define CHECK_PTR(p, a)                                                             \
    do {                                                                            \
        if (!(p)) return fail(PA_ERR_INVALID_ARG, "%s is NULL", #p);                \
        if (!aligned((p), (a)))                                                     \
            return fail(PA_ERR_INVALID_ARG, "%s is not %d-byte aligned", #p, (int)(a)); \
    } while (0)

pa_status check_common(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t dtype) {
    if (num_q_heads <= 0 || num_kv_heads <= 0)
        return fail(PA_ERR_INVALID_ARG, "head counts must be positive (%d, %d)", num_q_heads,
                    num_kv_heads);
    if (num_q_heads % num_kv_heads)
        return fail(PA_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d",
                    num_q_heads, num_kv_heads);
    if (num_kv_heads > 65535) return fail(PA_ERR_INVALID_ARG, "num_kv_heads too large");
    if (dtype != PA_F32 && dtype != PA_BF16)
        return fail(PA_ERR_UNSUPPORTED, "dtype %d not supported", dtype);
    if (!pa::decode_shape_supported(dtype, head_dim, block_size, num_q_heads / num_kv_heads))
        return fail(PA_ERR_UNSUPPORTED, "head_dim %d, block_size %d, group %d not supported",
                    head_dim, block_size, num_q_heads / num_kv_heads);
    return PA_OK;
}

int32_t resolve_partition(int32_t partition_size, int32_t num_seqs, int32_t num_kv_heads,
                          int32_t max_context_len, int32_t block_size) {
    if (partition_size > 0) return partition_size;
    return pa_decode_auto_partition_size(num_seqs, num_kv_heads, max_context_len, block_size);
}

// Decode work split: balanced over waves (partition_size 0, batches up to
// kStreamMaxSeqs) or fixed partitions.
// Balanced split: one wave per (sequence, kv head) pair instead of the equal
// split when the pairs fit in one round of waves and no context is longer than
// this many 16-token units, so that a small batch of short contexts is one
// launch (the equal split would cut every pair into single units and need the
// reduce).
constexpr int64_t kPairModeUnits = 8;

struct DecodePlan {
    bool stream;
    bool pairs;      // balanced split with one wave per pair
    int waves;       // balanced split
    int32_t P;       // fixed partitions
    int64_t np;
    size_t o_bytes, ml_bytes, scan_bytes;
    size_t total() const { return o_bytes + ml_bytes + scan_bytes; }
};

DecodePlan plan_decode(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t max_context_len,
                       int32_t partition_size, bool allow_pairs = true) {
    DecodePlan p{};
    const int64_t S = num_seqs > 0 ? num_seqs : 0;
    p.stream = partition_size == 0 && S <= pa::kStreamMaxSeqs;
    if (p.stream) {
        const int64_t per_pair = cdiv64(max_context_len > 0 ? max_context_len : 0, 16);
        const int64_t npairs = S * num_kv_heads;
        const int64_t units = npairs * per_pair;
        p.pairs = allow_pairs && npairs > 0 && npairs <= pa::kStreamWaves &&
                  per_pair <= kPairModeUnits;
        p.waves = p.pairs ? (int)npairs
                          : (int)(units < pa::kStreamWaves ? (units > 0 ? units : 1)
                                                           : pa::kStreamWaves);
        const int64_t G = num_q_heads / num_kv_heads;
        const int64_t recs = (S * num_kv_heads + p.waves) * G;
        p.o_bytes = align256((size_t)recs * head_dim * 4);
        p.ml_bytes = align256((size_t)recs * 2 * 4);
        p.scan_bytes = align256((size_t)(S + 1) * 4);
        return p;
    }
    p.P = resolve_partition(partition_size, num_seqs, num_kv_heads, max_context_len, block_size);
    p.np = cdiv64(max_context_len, p.P);
    if (p.np > 1) {
        const size_t rows = (size_t)S * num_q_heads * p.np;
        p.o_bytes = align256(rows * head_dim * 4);
        p.ml_bytes = align256(rows * 2 * 4);
    }
    return p;
}

struct DecodeSetup {
    pa::DecodeArgs a;
    size_t need;
};

pa_status setup_decode(DecodeSetup &st, void *out, const void *query, const void *key_cache,
                       const void *value_cache, const int32_t *block_tables,
                       const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
                       int32_t partition_size, float scale, int32_t dtype, void *workspace,
                       size_t workspace_bytes, bool needs_inputs, bool allow_pairs = true) {
    pa_status s = check_common(num_q_heads, num_kv_heads, head_dim, block_size, dtype);
    if (s != PA_OK) return s;
    if (num_seqs < 0 || num_seqs > 65535)
        return fail(PA_ERR_INVALID_ARG, "num_seqs %d out of range [0, 65535]", num_seqs);
    if (max_blocks_per_seq <= 0) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq <= 0");
    if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
        return fail(PA_ERR_INVALID_ARG, "max_context_len %d outside [0, %lld]", max_context_len,
                    (long long)max_blocks_per_seq * block_size);
    if (partition_size < 0 || (partition_size > 0 && (partition_size % block_size ||
                                                       partition_size % 16 ||
                                                       partition_size > kMaxPartition)))
        return fail(PA_ERR_INVALID_ARG,
                    "partition_size %d must be 0 or a multiple of block_size and 16 up to %d",
                    partition_size, kMaxPartition);
    if (num_seqs > 0) {
        CHECK_PTR(out, 16);
        CHECK_PTR(context_lens, 4);
        if (needs_inputs) {
            CHECK_PTR(query, 16);
            CHECK_PTR(key_cache, 16);
            CHECK_PTR(value_cache, 16);
            CHECK_PTR(block_tables, 4);
            if (num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "num_blocks <= 0");
            if (!isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale is not finite");
        }
    }
    const DecodePlan plan = plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                        block_size, max_context_len, partition_size, allow_pairs);
    const size_t need = plan.total() > kMinWorkspace ? plan.total() : kMinWorkspace;
    const bool uses_ws = num_seqs > 0 && (plan.stream || plan.np > 1);
    if (uses_ws) {
        if (!workspace) return fail(PA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
        if (!aligned(workspace, 256))
            return fail(PA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
        if (workspace_bytes < plan.total())
            return fail(PA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes,
                        plan.total());
    }
    pa::DecodeArgs &a = st.a;
    a.out = out;
    a.query = query;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.block_size = block_size;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_blocks = num_blocks;
    a.max_context_len = max_context_len;
    a.partition_size = plan.stream ? 0 : plan.P;
    a.num_partitions = plan.stream ? 0 : (int)plan.np;
    a.stream_waves = plan.stream ? plan.waves : 0;
    a.pairs = plan.stream && plan.pairs;
    a.scale = scale;
    a.dtype = dtype;
    a.new_key = nullptr;
    a.new_value = nullptr;
    a.kv_fp8 = 0;
    a.k_scale = 1.0f;
    a.v_scale = 1.0f;
    char *ws = (char *)workspace;
    a.ws_o = uses_ws ? (float *)ws : nullptr;
    a.ws_ml = uses_ws ? (float *)(ws + plan.o_bytes) : nullptr;
    a.ws_scan = (uses_ws && plan.stream) ? (int *)(ws + plan.o_bytes + plan.ml_bytes) : nullptr;
    st.need = need;
    return PA_OK;
}

// The device address of p when the device can access it: device memory
// (itself) or pinned host memory (its mapped view).  Pageable host memory, or
// a pointer HIP does not know, gives false.  hipPointerGetAttributes is a
// host-side query; its error, if any, is cleared so that it does not surface
// at a later call.
bool device_view(const void *p, const void **dev) {
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) {
        *dev = p;
        return true;
    }
    if (a.type == hipMemoryTypeHost && a.devicePointer && a.hostPointer) {
        *dev = (const char *)a.devicePointer + ((const char *)p - (const char *)a.hostPointer);
        return true;
    }
    return false;
}

// ---- PA_DEBUG=1: device-resident tables checked on the host ----------------
// Copies the tables an entry point reads (after the work already queued on
// the stream) and checks the preconditions the kernels assume; a violation
// returns PA_ERR_INVALID_ARG before any launch.  Synchronises the stream.

bool debug_checks() {
    const char *e = getenv("PA_DEBUG");
    return e && e[0] && strcmp(e, "0") != 0;
}

template <typename T>
pa_status fetch(std::vector<T> &dst, const void *src, size_t n, hipStream_t stream,
                const char *what) {
    dst.resize(n);
    if (n == 0) return PA_OK;
    hipError_t e = hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "PA_DEBUG: reading %s: %s", what, hipGetErrorString(e));
    return PA_OK;
}

// Table rows: every entry a sequence of length L reads, [0, ceil(L / B)),
// must name a block of the pool.
pa_status check_table_rows(const std::vector<int32_t> &bt, const std::vector<int32_t> &lens,
                           int32_t max_blocks, int32_t block_size, int64_t num_blocks,
                           const char *what) {
    for (size_t s = 0; s < lens.size(); ++s) {
        const int64_t nb = (lens[s] + (int64_t)block_size - 1) / block_size;
        for (int64_t j = 0; j < nb; ++j) {
            const int32_t b = bt[s * (size_t)max_blocks + (size_t)j];
            if (b < 0 || b >= num_blocks)
                return fail(PA_ERR_INVALID_ARG, "PA_DEBUG: %s[%zu][%lld] = %d outside [0, %lld)",
                            what, s, (long long)j, b, (long long)num_blocks);
        }
    }
    return PA_OK;
}

pa_status debug_decode(const pa::DecodeArgs &a, hipStream_t stream) {
    if (a.num_seqs <= 0) return PA_OK;
    std::vector<int32_t> lens, bt;
    pa_status s = fetch(lens, a.context_lens, (size_t)a.num_seqs, stream, "context_lens");
    if (s != PA_OK) return s;
    for (int32_t i = 0; i < a.num_seqs; ++i)
        if (lens[i] < 0 || lens[i] > a.max_context_len)
            return fail(PA_ERR_INVALID_ARG, "PA_DEBUG: context_lens[%d] = %d outside [0, %d]", i,
                        lens[i], a.max_context_len);
    s = fetch(bt, a.block_tables, (size_t)a.num_seqs * a.max_blocks_per_seq, stream,
              "block_tables");
    if (s != PA_OK) return s;
    return check_table_rows(bt, lens, a.max_blocks_per_seq, a.block_size, a.num_blocks,
                            "block_tables");
}

// Shared-prefix decode: the full-table checks of debug_decode, and the first
// prefix_blocks entries of every row equal to those of row 0.
pa_status debug_shared_prefix(const int32_t *block_tables, const int32_t *context_lens,
                              int32_t num_seqs, int32_t max_blocks, int32_t block_size,
                              int64_t num_blocks, int32_t max_context_len, int32_t prefix_blocks,
                              hipStream_t stream) {
    if (num_seqs <= 0) return PA_OK;
    std::vector<int32_t> lens, bt;
    pa_status s = fetch(lens, context_lens, (size_t)num_seqs, stream, "context_lens");
    if (s != PA_OK) return s;
    for (int32_t i = 0; i < num_seqs; ++i)
        if (lens[i] < 0 || lens[i] > max_context_len)
            return fail(PA_ERR_INVALID_ARG, "PA_DEBUG: context_lens[%d] = %d outside [0, %d]", i,
                        lens[i], max_context_len);
    s = fetch(bt, block_tables, (size_t)num_seqs * max_blocks, stream, "block_tables");
    if (s != PA_OK) return s;
    s = check_table_rows(bt, lens, max_blocks, block_size, num_blocks, "block_tables");
    if (s != PA_OK) return s;
    for (int32_t j = 0; j < prefix_blocks; ++j)
        if (bt[j] < 0 || (int64_t)bt[j] >= num_blocks)
            return fail(PA_ERR_INVALID_ARG, "PA_DEBUG: prefix block %d = %d outside the pool", j,
                        bt[j]);
    for (int32_t i = 1; i < num_seqs; ++i)
        for (int32_t j = 0; j < prefix_blocks; ++j)
            if (bt[(size_t)i * max_blocks + j] != bt[j])
                return fail(PA_ERR_INVALID_ARG,
                            "PA_DEBUG: block_tables[%d][%d] = %d differs from the shared prefix "
                            "block %d",
                            i, j, bt[(size_t)i * max_blocks + j], bt[j]);
    return PA_OK;
}

pa_status debug_slots(const int64_t *slot_mapping, int32_t num_tokens, int64_t num_slots,
                      hipStream_t stream) {
    std::vector<int64_t> slots;
    pa_status s = fetch(slots, slot_mapping, (size_t)num_tokens, stream, "slot_mapping");
    if (s != PA_OK) return s;
    std::vector<int64_t> used;
    for (int32_t t = 0; t < num_tokens; ++t) {
        if (slots[t] < 0) continue;  // padding
        if (slots[t] >= num_slots)
            return fail(PA_ERR_INVALID_ARG, "PA_DEBUG: slot_mapping[%d] = %lld outside [0, %lld)",
                        t, (long long)slots[t], (long long)num_slots);
        used.push_back(slots[t]);
    }
    std::sort(used.begin(), used.end());
    for (size_t i = 1; i < used.size(); ++i)
        if (used[i] == used[i - 1])
            return fail(PA_ERR_INVALID_ARG, "PA_DEBUG: slot %lld written twice",
                        (long long)used[i]);
    return PA_OK;
}

pa_status debug_prefill(const int32_t *cu_query_lens, const int32_t *context_lens,
                        const int32_t *block_tables, int32_t num_chunks, int32_t max_query_len,
                        int32_t max_blocks, int32_t block_size, int64_t num_blocks,
                        hipStream_t stream) {
    std::vector<int32_t> cu, lens, bt;
    pa_status s = fetch(cu, cu_query_lens, (size_t)num_chunks + 1, stream, "cu_query_lens");
    if (s == PA_OK) s = fetch(lens, context_lens, (size_t)num_chunks, stream, "context_lens");
    if (s == PA_OK)
        s = fetch(bt, block_tables, (size_t)num_chunks * max_blocks, stream, "block_tables");
    if (s != PA_OK) return s;
    if (cu[0] != 0) return fail(PA_ERR_INVALID_ARG, "PA_DEBUG: cu_query_lens[0] = %d, not 0", cu[0]);
    for (int32_t c = 0; c < num_chunks; ++c) {
        const int32_t n = cu[c + 1] - cu[c];
        if (n < 0 || n > max_query_len)
            return fail(PA_ERR_INVALID_ARG, "PA_DEBUG: chunk %d has %d queries (max_query_len %d)",
                        c, n, max_query_len);
        if (n > lens[c] || (int64_t)lens[c] > (int64_t)max_blocks * block_size)
            return fail(PA_ERR_INVALID_ARG,
                        "PA_DEBUG: chunk %d: %d queries over context_lens %d (table holds %lld)",
                        c, n, lens[c], (long long)max_blocks * block_size);
    }
    return check_table_rows(bt, lens, max_blocks, block_size, num_blocks, "block_tables");
}

pa_status debug_copy(const void *mapping, int32_t num_pairs, int64_t src_num_blocks,
                     int64_t dst_num_blocks, bool same_pool, hipStream_t stream) {
    std::vector<int64_t> m;
    pa_status s = fetch(m, mapping, (size_t)num_pairs * 2, stream, "block_mapping");
    if (s != PA_OK) return s;
    std::vector<int64_t> dst, src;
    for (int32_t i = 0; i < num_pairs; ++i) {
        if (m[2 * i] < 0 || m[2 * i] >= src_num_blocks || m[2 * i + 1] < 0 ||
            m[2 * i + 1] >= dst_num_blocks)
            return fail(PA_ERR_INVALID_ARG, "PA_DEBUG: pair %d (%lld -> %lld) outside the pools", i,
                        (long long)m[2 * i], (long long)m[2 * i + 1]);
        src.push_back(m[2 * i]);
        dst.push_back(m[2 * i + 1]);
    }
    std::sort(dst.begin(), dst.end());
    for (size_t i = 1; i < dst.size(); ++i)
        if (dst[i] == dst[i - 1])
            return fail(PA_ERR_INVALID_ARG, "PA_DEBUG: destination block %lld written twice",
                        (long long)dst[i]);
    if (same_pool)
        for (int64_t b : src)
            if (std::binary_search(dst.begin(), dst.end(), b))
                return fail(PA_ERR_INVALID_ARG,
                            "PA_DEBUG: block %lld is both a source and a destination", (long long)b);
    return PA_OK;
}

// ---- the decode workspace of pa_decode_no_alloc: a static device array ----
//
// For callers that cannot allocate (code under graph capture, serving loops
// that forbid hipMalloc): the partial records and the unit scan of pa_decode
// live in this file-scope device array, one copy per GPU, held until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it only names a stand-in): its device address is looked up once per
// device with hipGetSymbolAddress and that address is what the kernels get.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The device address of the current device's copy of `scratch`.
pa_status scratch_for_current_device(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(PA_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table tracks", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return PA_OK;
}

// Shared-prefix decode: the prefix pass runs on a second stream of the
// library (default priority, one per device, created on first use) beside
// the suffix pass on the caller's stream.  A prefix workgroup fits on a CU
// next to a suffix one, so the matrix-core work of the prefix pass hides under
// the memory-bound suffix pass.  The enqueue sequence (fork event, prefix
// launch, join event, suffix launch, join wait, reduce) is done under the
// device's lock, so calls from several host threads interleave safely.
struct SideStream {
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    std::mutex mu;
};
SideStream g_side[kMaxDevices];
std::mutex g_side_init_mu;

pa_status side_for_current_device(SideStream **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(PA_ERR_UNSUPPORTED, "device %d beyond the %d the library tracks", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_side_init_mu);
    SideStream &sd = g_side[dev];
    if (!sd.stream) {
        hipStream_t st = nullptr;
        hipEvent_t f = nullptr, j = nullptr;
        e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&f, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&j, hipEventDisableTiming);
        if (e != hipSuccess) {
            if (j) (void)hipEventDestroy(j);
            if (f) (void)hipEventDestroy(f);
            if (st) (void)hipStreamDestroy(st);
            return fail(PA_ERR_HIP, "side stream for the prefix pass: %s", hipGetErrorString(e));
        }
        sd.fork = f;
        sd.join = j;
        sd.stream = st;
    }
    *out = &sd;
    return PA_OK;
}

}  // namespace

extern "C" {

int32_t pa_abi_version(void) { return 1; }

const char *pa_status_string(int32_t status) {
    switch (status) {
        case PA_OK: return "PA_OK";
        case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
        case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
        case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
        case PA_ERR_HIP: return "PA_ERR_HIP";
        case PA_ERR_POOL_EXHAUSTED: return "PA_ERR_POOL_EXHAUSTED";
    }
    return "PA_UNKNOWN_STATUS";
}

const char *pa_last_error(void) { return g_error; }

pa_status pa_reshape_and_cache(const void *key, const void *value, void *key_cache,
                               void *value_cache, const int64_t *slot_mapping,
                               int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int64_t num_blocks, int32_t dtype,
                               void *stream) {
    if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens < 0");
    if (num_kv_heads <= 0) return fail(PA_ERR_INVALID_ARG, "num_kv_heads <= 0");
    if (dtype != PA_F32 && dtype != PA_BF16)
        return fail(PA_ERR_UNSUPPORTED, "dtype %d not supported", dtype);
    if ((head_dim != 64 && head_dim != 128) || (block_size != 16 && block_size != 32))
        return fail(PA_ERR_UNSUPPORTED, "head_dim %d / block_size %d not supported", head_dim,
                    block_size);
    if (num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "num_blocks <= 0");
    if (num_tokens == 0) return PA_OK;
    CHECK_PTR(key, 16);
    CHECK_PTR(value, 16);
    CHECK_PTR(key_cache, 16);
    CHECK_PTR(value_cache, 16);
    CHECK_PTR(slot_mapping, 8);
    if (debug_checks()) {
        const pa_status d = debug_slots(slot_mapping, num_tokens, num_blocks * block_size,
                                        (hipStream_t)stream);
        if (d != PA_OK) return d;
    }
    return hip_status(pa::launch_reshape_and_cache(key, value, key_cache, value_cache,
                                                   slot_mapping, num_tokens, num_kv_heads,
                                                   head_dim, block_size, num_blocks,
                                                   dtype == PA_BF16 ? 2 : 4,
                                                   (hipStream_t)stream),
                      "reshape_and_cache");
}

int32_t pa_decode_auto_partition_size(int32_t num_seqs, int32_t num_kv_heads,
                                      int32_t max_context_len, int32_t block_size) {
    // Enough (sequence, kv head, partition) workgroups to fill 256 CUs several
    // times over, without cutting partitions below one 16-token unit per wave.
    (void)block_size;
    const int64_t pairs = (int64_t)(num_seqs > 0 ? num_seqs : 1) * (num_kv_heads > 0 ? num_kv_heads : 1);
    int32_t P = 1024;
    while (P > kMinPartition && pairs * cdiv64(max_context_len > 0 ? max_context_len : 1, P) < 4096)
        P /= 2;
    return P;
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                 int32_t partition_size) {
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        num_q_heads % num_kv_heads || partition_size < 0)
        return kMinWorkspace;
    const DecodePlan p = plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                     max_context_len, partition_size);
    return p.total() > kMinWorkspace ? p.total() : kMinWorkspace;
}

int32_t pa_decode_needs_reduce(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t max_context_len,
                               int32_t partition_size) {
    if (num_seqs <= 0) return num_seqs == 0 ? 0 : 1;
    if (num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_q_heads % num_kv_heads || partition_size < 0 || max_context_len < 0)
        return 1;
    const DecodePlan p = plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                     max_context_len, partition_size);
    if (p.stream) return p.pairs ? 0 : 1;
    return 1;
}

pa_status pa_decode_partitions(void *out, const void *query, const void *key_cache,
                               const void *value_cache, const int32_t *block_tables,
                               const int32_t *context_lens, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t max_blocks_per_seq,
                               int64_t num_blocks, int32_t max_context_len,
                               int32_t partition_size, float scale, int32_t dtype,
                               void *workspace, size_t workspace_bytes, void *stream) {
    DecodeSetup st;
    pa_status s = setup_decode(st, out, query, key_cache, value_cache, block_tables,
                               context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                               block_size, max_blocks_per_seq, num_blocks, max_context_len,
                               partition_size, scale, dtype, workspace, workspace_bytes, true);
    if (s != PA_OK) return s;
    if (debug_checks() && (s = debug_decode(st.a, (hipStream_t)stream)) != PA_OK) return s;
    return hip_status(pa::launch_decode_partitions(st.a, (hipStream_t)stream),
                      "decode_partitions");
}

pa_status pa_decode_reduce(void *out, const int32_t *context_lens, int32_t num_seqs,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t max_blocks_per_seq,
                           int32_t max_context_len, int32_t partition_size, int32_t dtype,
                           const void *workspace, size_t workspace_bytes, void *stream) {
    DecodeSetup st;
    pa_status s = setup_decode(st, out, nullptr, nullptr, nullptr, nullptr, context_lens,
                               num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                               max_blocks_per_seq, 1, max_context_len, partition_size, 1.0f,
                               dtype, (void *)workspace, workspace_bytes, false);
    if (s != PA_OK) return s;
    return hip_status(pa::launch_decode_reduce(st.a, (hipStream_t)stream), "decode_reduce");
}

pa_status pa_decode(void *out, const void *query, const void *key_cache,
                    const void *value_cache, const int32_t *block_tables,
                    const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
                    int32_t partition_size, float scale, int32_t dtype, void *workspace,
                    size_t workspace_bytes, void *stream) {
    DecodeSetup st;
    pa_status s = setup_decode(st, out, query, key_cache, value_cache, block_tables,
                               context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                               block_size, max_blocks_per_seq, num_blocks, max_context_len,
                               partition_size, scale, dtype, workspace, workspace_bytes, true);
    if (s != PA_OK) return s;
    if (debug_checks() && (s = debug_decode(st.a, (hipStream_t)stream)) != PA_OK) return s;
    s = hip_status(pa::launch_decode_partitions(st.a, (hipStream_t)stream), "decode_partitions");
    if (s != PA_OK) return s;
    return hip_status(pa::launch_decode_reduce(st.a, (hipStream_t)stream), "decode_reduce");
}

size_t pa_decode_no_alloc_max_workspace(void) { return kNoAllocScratchBytes; }

pa_status pa_decode_no_alloc(void *out, const void *query, const void *key_cache,
                             const void *value_cache, const int32_t *block_tables,
                             const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t max_blocks_per_seq, int64_t num_blocks,
                             int32_t max_context_len, int32_t partition_size, float scale,
                             int32_t dtype, void *stream) {
    // Every argument check of pa_decode first (no device call), with a
    // stand-in workspace address, then the size of the plan's workspace.
    DecodeSetup st;
    pa_status s = setup_decode(st, out, query, key_cache, value_cache, block_tables,
                               context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                               block_size, max_blocks_per_seq, num_blocks, max_context_len,
                               partition_size, scale, dtype, (void *)(uintptr_t)256,
                               kNoAllocScratchBytes, true);
    if (s != PA_OK) {
        if (s == PA_ERR_WORKSPACE)
            return fail(PA_ERR_WORKSPACE,
                        "this decode needs %zu bytes of workspace; the static scratch holds %zu",
                        pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                  block_size, max_context_len, partition_size),
                        kNoAllocScratchBytes);
        return s;
    }
    if (num_seqs == 0) return PA_OK;
    void *ws = nullptr;
    s = scratch_for_current_device(&ws);
    if (s != PA_OK) return s;
    return pa_decode(out, query, key_cache, value_cache, block_tables, context_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                     num_blocks, max_context_len, partition_size, scale, dtype, ws,
                     kNoAllocScratchBytes, stream);
}

}  // extern "C"

namespace {

// Shared-prefix decode: the balanced split's workspace for the tokens past
// the prefix, then the prefix records.
struct PrefixPlan {
    DecodePlan suffix;
    int32_t prefix_tokens, suffix_max_len;
    int ksplit;
    size_t xo_bytes, xml_bytes;
    size_t total() const { return suffix.total() + xo_bytes + xml_bytes; }
};

PrefixPlan plan_prefix(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t max_context_len,
                       int32_t prefix_blocks) {
    PrefixPlan p{};
    p.prefix_tokens = prefix_blocks * block_size;
    p.suffix_max_len = max_context_len > p.prefix_tokens ? max_context_len - p.prefix_tokens : 0;
    // The suffix pass writes every pair as records for the merge with the
    // prefix records: the equal split, never one wave per pair.
    p.suffix = plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                           p.suffix_max_len, 0, false);
    p.ksplit = (num_seqs > 0 && p.prefix_tokens > 0)
                   ? pa::prefix_splits(num_seqs, num_q_heads, num_kv_heads, p.prefix_tokens)
                   : 0;
    const size_t recs = (size_t)(num_seqs > 0 ? num_seqs : 0) * num_q_heads * p.ksplit;
    p.xo_bytes = align256(recs * head_dim * 4);
    p.xml_bytes = align256(recs * 2 * 4);
    return p;
}

}  // namespace

extern "C" {

size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                               int32_t num_kv_heads, int32_t head_dim,
                                               int32_t block_size, int32_t max_context_len,
                                               int32_t prefix_blocks) {
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || num_q_heads % num_kv_heads || prefix_blocks < 0 ||
        num_seqs > pa::kStreamMaxSeqs)
        return kMinWorkspace;
    const PrefixPlan p = plan_prefix(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                     max_context_len, prefix_blocks);
    return p.total() > kMinWorkspace ? p.total() : kMinWorkspace;
}

}  // extern "C"

namespace {

// pa_decode_shared_prefix and pa_decode_fp8_shared_prefix: the same passes
// over bf16 pools or over e4m3 pools (fp8, with their two scales).
pa_status shared_prefix_decode(void *out, const void *query, const void *key_cache,
                               const void *value_cache, const int32_t *block_tables,
                               const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t max_blocks_per_seq, int64_t num_blocks,
                               int32_t max_context_len, int32_t prefix_blocks, float scale,
                               bool fp8, float k_scale, float v_scale, void *workspace,
                               size_t workspace_bytes, void *stream) {
    pa_status s = check_common(num_q_heads, num_kv_heads, head_dim, block_size, PA_BF16);
    if (s != PA_OK) return s;
    if (num_seqs < 0 || num_seqs > pa::kStreamMaxSeqs)
        return fail(num_seqs < 0 ? PA_ERR_INVALID_ARG : PA_ERR_UNSUPPORTED,
                    "num_seqs %d outside [0, %d] for the shared-prefix decode", num_seqs,
                    pa::kStreamMaxSeqs);
    if (max_blocks_per_seq <= 0) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq <= 0");
    if (prefix_blocks < 0 || prefix_blocks > max_blocks_per_seq)
        return fail(PA_ERR_INVALID_ARG, "prefix_blocks %d outside [0, %d]", prefix_blocks,
                    max_blocks_per_seq);
    if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
        return fail(PA_ERR_INVALID_ARG, "max_context_len %d outside [0, %lld]", max_context_len,
                    (long long)max_blocks_per_seq * block_size);
    const PrefixPlan plan = plan_prefix(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                        max_context_len, prefix_blocks);
    if (num_seqs > 0) {
        if (!workspace)
            return fail(PA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", plan.total());
        if (!aligned(workspace, 256))
            return fail(PA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
        if (workspace_bytes < plan.total())
            return fail(PA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes,
                        plan.total());
        CHECK_PTR(block_tables, 4);
    }
    // The pass over the tokens past the prefix: the tables advanced past the
    // prefix pages, lengths and their bound reduced by the prefix.
    DecodeSetup st;
    s = setup_decode(st, out, query, key_cache, value_cache,
                     block_tables ? block_tables + prefix_blocks : nullptr, context_lens,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     max_blocks_per_seq, num_blocks, plan.suffix_max_len, 0, scale, PA_BF16,
                     workspace, workspace_bytes, true, false);
    if (s != PA_OK) return s;
    if (fp8) {
        st.a.kv_fp8 = 1;
        st.a.k_scale = k_scale;
        st.a.v_scale = v_scale;
    }
    if (num_seqs == 0) return PA_OK;
    if (debug_checks() &&
        (s = debug_shared_prefix(block_tables, context_lens, num_seqs, max_blocks_per_seq,
                                 block_size, num_blocks, max_context_len, prefix_blocks,
                                 (hipStream_t)stream)) != PA_OK)
        return s;
    pa::PrefixArgs px;
    px.prefix_table = block_tables;
    px.prefix_tokens = plan.prefix_tokens;
    px.ksplit = plan.ksplit;
    px.x_o = (float *)((char *)workspace + plan.suffix.total());
    px.x_ml = (float *)((char *)workspace + plan.suffix.total() + plan.xo_bytes);
    if (plan.ksplit == 0) {  // no prefix: the plain balanced decode
        s = hip_status(pa::launch_decode_partitions(st.a, (hipStream_t)stream),
                       "decode_partitions");
        if (s != PA_OK) return s;
        return hip_status(pa::launch_decode_reduce(st.a, (hipStream_t)stream), "decode_reduce");
    }
    SideStream *sd = nullptr;
    s = side_for_current_device(&sd);
    if (s != PA_OK) return s;
    std::lock_guard<std::mutex> lock(sd->mu);
    const hipStream_t caller = (hipStream_t)stream;
    s = hip_status(hipEventRecord(sd->fork, caller), "hipEventRecord");
    if (s == PA_OK) s = hip_status(hipStreamWaitEvent(sd->stream, sd->fork, 0), "hipStreamWaitEvent");
    if (s == PA_OK)
        s = hip_status(pa::launch_decode_prefix(st.a, px, sd->stream), "decode_prefix");
    if (s == PA_OK) s = hip_status(hipEventRecord(sd->join, sd->stream), "hipEventRecord");
    if (s != PA_OK) return s;
    s = hip_status(pa::launch_decode_suffix(st.a, plan.prefix_tokens, caller), "decode_suffix");
    // The caller's stream waits for the prefix pass whatever happened above,
    // so that nothing later on it can overtake work already enqueued.
    const pa_status w = hip_status(hipStreamWaitEvent(caller, sd->join, 0), "hipStreamWaitEvent");
    if (s != PA_OK) return s;
    if (w != PA_OK) return w;
    return hip_status(pa::launch_decode_reduce_prefix(st.a, px, caller), "decode_reduce");
}

}  // namespace

extern "C" {

pa_status pa_decode_shared_prefix(void *out, const void *query, const void *key_cache,
                                  const void *value_cache, const int32_t *block_tables,
                                  const int32_t *context_lens, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t max_blocks_per_seq,
                                  int64_t num_blocks, int32_t max_context_len,
                                  int32_t prefix_blocks, float scale, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    return shared_prefix_decode(out, query, key_cache, value_cache, block_tables, context_lens,
                                num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                max_blocks_per_seq, num_blocks, max_context_len, prefix_blocks,
                                scale, false, 1.0f, 1.0f, workspace, workspace_bytes, stream);
}

pa_status pa_decode_fp8_shared_prefix(void *out, const void *query, const void *key_cache,
                                      const void *value_cache, const int32_t *block_tables,
                                      const int32_t *context_lens, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size,
                                      int32_t max_blocks_per_seq, int64_t num_blocks,
                                      int32_t max_context_len, int32_t prefix_blocks, float scale,
                                      float k_scale, float v_scale, void *workspace,
                                      size_t workspace_bytes, void *stream) {
    if (!(k_scale > 0.0f) || !(v_scale > 0.0f) || !isfinite(k_scale) || !isfinite(v_scale))
        return fail(PA_ERR_INVALID_ARG, "k_scale and v_scale must be positive and finite");
    return shared_prefix_decode(out, query, key_cache, value_cache, block_tables, context_lens,
                                num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                max_blocks_per_seq, num_blocks, max_context_len, prefix_blocks,
                                scale, true, k_scale, v_scale, workspace, workspace_bytes, stream);
}

pa_status pa_decode_append_partitions(void *out, const void *query, const void *new_key,
                                      const void *new_value, void *key_cache, void *value_cache,
                                      const int32_t *block_tables, const int32_t *context_lens,
                                      int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_blocks_per_seq,
                                      int64_t num_blocks, int32_t max_context_len,
                                      int32_t partition_size, float scale, int32_t dtype,
                                      void *workspace, size_t workspace_bytes, void *stream) {
    DecodeSetup st;
    pa_status s = setup_decode(st, out, query, key_cache, value_cache, block_tables,
                               context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                               block_size, max_blocks_per_seq, num_blocks, max_context_len,
                               partition_size, scale, dtype, workspace, workspace_bytes, true);
    if (s != PA_OK) return s;
    if (num_seqs > 0) {
        CHECK_PTR(new_key, 16);
        CHECK_PTR(new_value, 16);
    }
    st.a.new_key = new_key;
    st.a.new_value = new_value;
    if (debug_checks() && (s = debug_decode(st.a, (hipStream_t)stream)) != PA_OK) return s;
    return hip_status(pa::launch_decode_partitions(st.a, (hipStream_t)stream),
                      "decode_append_partitions");
}

pa_status pa_decode_append(void *out, const void *query, const void *new_key,
                           const void *new_value, void *key_cache, void *value_cache,
                           const int32_t *block_tables, const int32_t *context_lens,
                           int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                           int64_t num_blocks, int32_t max_context_len, int32_t partition_size,
                           float scale, int32_t dtype, void *workspace, size_t workspace_bytes,
                           void *stream) {
    pa_status s = pa_decode_append_partitions(
        out, query, new_key, new_value, key_cache, value_cache, block_tables, context_lens,
        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
        num_blocks, max_context_len, partition_size, scale, dtype, workspace, workspace_bytes,
        stream);
    if (s != PA_OK) return s;
    return pa_decode_reduce(out, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                            block_size, max_blocks_per_seq, max_context_len, partition_size,
                            dtype, workspace, workspace_bytes, stream);
}

pa_status pa_reshape_and_cache_fp8(const void *key, const void *value, void *key_cache,
                                   void *value_cache, const int64_t *slot_mapping,
                                   int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int64_t num_blocks, int32_t dtype,
                                   float k_scale, float v_scale, void *stream) {
    if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens < 0");
    if (num_kv_heads <= 0 || num_kv_heads > 65535)
        return fail(PA_ERR_INVALID_ARG, "num_kv_heads %d outside [1, 65535]", num_kv_heads);
    if (dtype != PA_F32 && dtype != PA_BF16)
        return fail(PA_ERR_UNSUPPORTED, "dtype %d of the new rows not supported", dtype);
    if ((head_dim != 64 && head_dim != 128) || (block_size != 16 && block_size != 32))
        return fail(PA_ERR_UNSUPPORTED, "head_dim %d / block_size %d not supported", head_dim,
                    block_size);
    if (!(k_scale > 0.0f) || !(v_scale > 0.0f) || !isfinite(k_scale) || !isfinite(v_scale))
        return fail(PA_ERR_INVALID_ARG, "k_scale and v_scale must be positive and finite");
    if (num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "num_blocks <= 0");
    if (num_tokens == 0) return PA_OK;
    CHECK_PTR(key, 16);
    CHECK_PTR(value, 16);
    CHECK_PTR(key_cache, 16);
    CHECK_PTR(value_cache, 16);
    CHECK_PTR(slot_mapping, 8);
    if (debug_checks()) {
        const pa_status d = debug_slots(slot_mapping, num_tokens, num_blocks * block_size,
                                        (hipStream_t)stream);
        if (d != PA_OK) return d;
    }
    return hip_status(pa::launch_reshape_and_cache_fp8(
                          key, value, key_cache, value_cache, slot_mapping, num_tokens,
                          num_kv_heads, head_dim, block_size, num_blocks,
                          dtype == PA_BF16 ? 2 : 4, 1.0f / k_scale, 1.0f / v_scale,
                          (hipStream_t)stream),
                      "reshape_and_cache_fp8");
}

pa_status pa_decode_fp8_partitions(void *out, const void *query, const void *key_cache,
                                   const void *value_cache, const int32_t *block_tables,
                                   const int32_t *context_lens, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t max_blocks_per_seq,
                                   int64_t num_blocks, int32_t max_context_len, float scale,
                                   float k_scale, float v_scale, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    if (num_seqs > pa::kStreamMaxSeqs)
        return fail(PA_ERR_UNSUPPORTED, "FP8 decode handles up to %d sequences per call",
                    pa::kStreamMaxSeqs);
    if (!(k_scale > 0.0f) || !(v_scale > 0.0f) || !isfinite(k_scale) || !isfinite(v_scale))
        return fail(PA_ERR_INVALID_ARG, "k_scale and v_scale must be positive and finite");
    DecodeSetup st;
    pa_status s = setup_decode(st, out, query, key_cache, value_cache, block_tables,
                               context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                               block_size, max_blocks_per_seq, num_blocks, max_context_len, 0,
                               scale, PA_BF16, workspace, workspace_bytes, true);
    if (s != PA_OK) return s;
    st.a.kv_fp8 = 1;
    st.a.k_scale = k_scale;
    st.a.v_scale = v_scale;
    if (debug_checks() && (s = debug_decode(st.a, (hipStream_t)stream)) != PA_OK) return s;
    return hip_status(pa::launch_decode_partitions(st.a, (hipStream_t)stream),
                      "decode_fp8_partitions");
}

pa_status pa_decode_fp8_append_partitions(
    void *out, const void *query, const void *new_key, const void *new_value, void *key_cache,
    void *value_cache, const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len, float scale,
    float k_scale, float v_scale, void *workspace, size_t workspace_bytes, void *stream) {
    if (num_seqs > pa::kStreamMaxSeqs)
        return fail(PA_ERR_UNSUPPORTED, "FP8 decode handles up to %d sequences per call",
                    pa::kStreamMaxSeqs);
    if (!(k_scale > 0.0f) || !(v_scale > 0.0f) || !isfinite(k_scale) || !isfinite(v_scale))
        return fail(PA_ERR_INVALID_ARG, "k_scale and v_scale must be positive and finite");
    DecodeSetup st;
    pa_status s = setup_decode(st, out, query, key_cache, value_cache, block_tables,
                               context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                               block_size, max_blocks_per_seq, num_blocks, max_context_len, 0,
                               scale, PA_BF16, workspace, workspace_bytes, true);
    if (s != PA_OK) return s;
    if (num_seqs > 0) {
        CHECK_PTR(new_key, 16);
        CHECK_PTR(new_value, 16);
    }
    st.a.kv_fp8 = 1;
    st.a.k_scale = k_scale;
    st.a.v_scale = v_scale;
    st.a.new_key = new_key;
    st.a.new_value = new_value;
    if (debug_checks() && (s = debug_decode(st.a, (hipStream_t)stream)) != PA_OK) return s;
    return hip_status(pa::launch_decode_partitions(st.a, (hipStream_t)stream),
                      "decode_fp8_append_partitions");
}

pa_status pa_decode_fp8_append(void *out, const void *query, const void *new_key,
                               const void *new_value, void *key_cache, void *value_cache,
                               const int32_t *block_tables, const int32_t *context_lens,
                               int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                               int64_t num_blocks, int32_t max_context_len, float scale,
                               float k_scale, float v_scale, void *workspace,
                               size_t workspace_bytes, void *stream) {
    pa_status s = pa_decode_fp8_append_partitions(
        out, query, new_key, new_value, key_cache, value_cache, block_tables, context_lens,
        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
        max_context_len, scale, k_scale, v_scale, workspace, workspace_bytes, stream);
    if (s != PA_OK) return s;
    return pa_decode_reduce(out, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                            block_size, max_blocks_per_seq, max_context_len, 0, PA_BF16,
                            workspace, workspace_bytes, stream);
}

pa_status pa_decode_fp8(void *out, const void *query, const void *key_cache,
                        const void *value_cache, const int32_t *block_tables,
                        const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
                        float scale, float k_scale, float v_scale, void *workspace,
                        size_t workspace_bytes, void *stream) {
    pa_status s = pa_decode_fp8_partitions(out, query, key_cache, value_cache, block_tables,
                                           context_lens, num_seqs, num_q_heads, num_kv_heads,
                                           head_dim, block_size, max_blocks_per_seq, num_blocks,
                                           max_context_len, scale, k_scale, v_scale, workspace,
                                           workspace_bytes, stream);
    if (s != PA_OK) return s;
    return pa_decode_reduce(out, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                            block_size, max_blocks_per_seq, max_context_len, 0, PA_BF16,
                            workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Checks and arguments shared by pa_prefill_chunk and pa_prefill_chunk_append.
// *done is set when there is nothing to launch.
pa_status setup_prefill(pa::PrefillArgs &a, bool *done, void *out, const void *query,
                        const void *key_cache, const void *value_cache,
                        const int32_t *block_tables, const int32_t *cu_query_lens,
                        const int32_t *context_lens, int32_t num_chunks, int32_t max_query_len,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                        float scale, int32_t dtype, void *stream) {
    *done = true;
    if (dtype != PA_BF16)
        return fail(PA_ERR_UNSUPPORTED, "prefill runs on bf16 matrix cores: dtype must be bf16");
    pa_status s = check_common(num_q_heads, num_kv_heads, head_dim, block_size, dtype);
    if (s != PA_OK) return s;
    if (num_chunks < 0 || num_chunks > 65535)
        return fail(PA_ERR_INVALID_ARG, "num_chunks %d out of range", num_chunks);
    if (max_query_len < 0) return fail(PA_ERR_INVALID_ARG, "max_query_len < 0");
    if (max_blocks_per_seq <= 0) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq <= 0");
    if (num_chunks == 0 || max_query_len == 0) return PA_OK;
    if (num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "num_blocks <= 0");
    if (!(scale > 0.0f) || !isfinite(scale))
        return fail(PA_ERR_INVALID_ARG, "prefill scale must be positive and finite");
    CHECK_PTR(out, 16);
    CHECK_PTR(query, 16);
    CHECK_PTR(key_cache, 16);
    CHECK_PTR(value_cache, 16);
    CHECK_PTR(block_tables, 4);
    CHECK_PTR(cu_query_lens, 4);
    CHECK_PTR(context_lens, 4);
    if (!pa::prefill_shape_supported(head_dim, block_size, num_q_heads / num_kv_heads))
        return fail(PA_ERR_UNSUPPORTED, "prefill shape not supported");
    if (debug_checks()) {
        const pa_status d = debug_prefill(cu_query_lens, context_lens, block_tables, num_chunks,
                                          max_query_len, max_blocks_per_seq, block_size,
                                          num_blocks, (hipStream_t)stream);
        if (d != PA_OK) return d;
    }
    a.out = out;
    a.query = query;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.block_tables = block_tables;
    a.cu_query_lens = cu_query_lens;
    a.context_lens = context_lens;
    a.num_chunks = num_chunks;
    a.max_query_len = max_query_len;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.block_size = block_size;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_blocks = num_blocks;
    a.scale = scale;
    a.kv_fp8 = 0;
    a.k_scale = 1.0f;
    a.v_scale = 1.0f;
    *done = false;
    return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_prefill_chunk(void *out, const void *query, const void *key_cache,
                           const void *value_cache, const int32_t *block_tables,
                           const int32_t *cu_query_lens, const int32_t *context_lens,
                           int32_t num_chunks, int32_t max_query_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                           int32_t dtype, void *stream) {
    pa::PrefillArgs a;
    bool done;
    const pa_status s = setup_prefill(a, &done, out, query, key_cache, value_cache, block_tables,
                                      cu_query_lens, context_lens, num_chunks, max_query_len,
                                      num_q_heads, num_kv_heads, head_dim, block_size,
                                      max_blocks_per_seq, num_blocks, scale, dtype, stream);
    if (s != PA_OK || done) return s;
    return hip_status(pa::launch_prefill_chunk(a, (hipStream_t)stream), "prefill_chunk");
}

pa_status pa_prefill_chunk_append(void *out, const void *query, const void *new_key,
                                  const void *new_value, void *key_cache, void *value_cache,
                                  const int32_t *block_tables, const int32_t *cu_query_lens,
                                  const int32_t *context_lens, int32_t num_chunks,
                                  int32_t max_query_len, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                                  int32_t dtype, void *stream) {
    pa::PrefillArgs a;
    bool done;
    const pa_status s = setup_prefill(a, &done, out, query, key_cache, value_cache, block_tables,
                                      cu_query_lens, context_lens, num_chunks, max_query_len,
                                      num_q_heads, num_kv_heads, head_dim, block_size,
                                      max_blocks_per_seq, num_blocks, scale, dtype, stream);
    if (s != PA_OK || done) return s;
    CHECK_PTR(new_key, 16);
    CHECK_PTR(new_value, 16);
    return hip_status(pa::launch_prefill_chunk_append(a, new_key, new_value, (hipStream_t)stream),
                      "prefill_chunk_append");
}

pa_status pa_prefill_chunk_fp8(void *out, const void *query, const void *key_cache,
                               const void *value_cache, const int32_t *block_tables,
                               const int32_t *cu_query_lens, const int32_t *context_lens,
                               int32_t num_chunks, int32_t max_query_len, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                               float k_scale, float v_scale, void *stream) {
    pa_status s = check_common(num_q_heads, num_kv_heads, head_dim, block_size, PA_BF16);
    if (s != PA_OK) return s;
    if (!(k_scale > 0.0f) || !(v_scale > 0.0f) || !isfinite(k_scale) || !isfinite(v_scale))
        return fail(PA_ERR_INVALID_ARG, "k_scale and v_scale must be positive and finite");
    if (num_chunks < 0 || num_chunks > 65535)
        return fail(PA_ERR_INVALID_ARG, "num_chunks %d out of range", num_chunks);
    if (max_query_len < 0) return fail(PA_ERR_INVALID_ARG, "max_query_len < 0");
    if (max_blocks_per_seq <= 0) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq <= 0");
    if (num_chunks == 0 || max_query_len == 0) return PA_OK;
    if (num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "num_blocks <= 0");
    if (!(scale > 0.0f) || !isfinite(scale))
        return fail(PA_ERR_INVALID_ARG, "prefill scale must be positive and finite");
    CHECK_PTR(out, 16);
    CHECK_PTR(query, 16);
    CHECK_PTR(key_cache, 16);
    CHECK_PTR(value_cache, 16);
    CHECK_PTR(block_tables, 4);
    CHECK_PTR(cu_query_lens, 4);
    CHECK_PTR(context_lens, 4);
    if (!pa::prefill_shape_supported(head_dim, block_size, num_q_heads / num_kv_heads))
        return fail(PA_ERR_UNSUPPORTED, "prefill shape not supported");
    if (debug_checks()) {
        const pa_status d = debug_prefill(cu_query_lens, context_lens, block_tables, num_chunks,
                                          max_query_len, max_blocks_per_seq, block_size,
                                          num_blocks, (hipStream_t)stream);
        if (d != PA_OK) return d;
    }
    pa::PrefillArgs a;
    a.out = out;
    a.query = query;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.block_tables = block_tables;
    a.cu_query_lens = cu_query_lens;
    a.context_lens = context_lens;
    a.num_chunks = num_chunks;
    a.max_query_len = max_query_len;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.block_size = block_size;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_blocks = num_blocks;
    a.scale = scale;
    a.kv_fp8 = 1;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    return hip_status(pa::launch_prefill_chunk(a, (hipStream_t)stream), "prefill_chunk_fp8");
}

pa_status pa_copy_blocks(const void *src_key_cache, const void *src_value_cache,
                         void *dst_key_cache, void *dst_value_cache,
                         const int64_t *block_mapping, int32_t num_pairs, int64_t src_num_blocks,
                         int64_t dst_num_blocks, int64_t block_bytes, void *stream) {
    if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "num_pairs < 0");
    if (src_num_blocks < 0 || dst_num_blocks < 0)
        return fail(PA_ERR_INVALID_ARG, "negative pool size");
    if (block_bytes <= 0 || block_bytes % 16)
        return fail(PA_ERR_INVALID_ARG, "block_bytes %lld is not a positive multiple of 16",
                    (long long)block_bytes);
    if (num_pairs == 0) return PA_OK;
    CHECK_PTR(src_key_cache, 16);
    CHECK_PTR(src_value_cache, 16);
    CHECK_PTR(dst_key_cache, 16);
    CHECK_PTR(dst_value_cache, 16);
    CHECK_PTR(block_mapping, 8);
    const void *ptrs[5] = {src_key_cache, src_value_cache, dst_key_cache, dst_value_cache,
                           block_mapping};
    const char *names[5] = {"src_key_cache", "src_value_cache", "dst_key_cache",
                            "dst_value_cache", "block_mapping"};
    const void *dev[5];
    for (int i = 0; i < 5; ++i)
        if (!device_view(ptrs[i], &dev[i]))
            return fail(PA_ERR_INVALID_ARG,
                        "%s is neither device memory nor pinned host memory the device can map",
                        names[i]);
    if (debug_checks()) {
        const pa_status d = debug_copy(dev[4], num_pairs, src_num_blocks, dst_num_blocks,
                                       src_key_cache == dst_key_cache, (hipStream_t)stream);
        if (d != PA_OK) return d;
    }
    return hip_status(pa::launch_copy_blocks(dev[0], dev[1], (void *)dev[2], (void *)dev[3],
                                             (const int64_t *)dev[4], num_pairs, src_num_blocks,
                                             dst_num_blocks, block_bytes, (hipStream_t)stream),
                      "copy_blocks");
}

int64_t pa_probe_sink_words(void) {
    const int g = pa::probe_read_grid() > pa::probe_mfma_grid() ? pa::probe_read_grid()
                                                                 : pa::probe_mfma_grid();
    return (int64_t)g * 256;
}

pa_status pa_probe_stream_read(const void *buf, int64_t bytes, void *sink, void *stream) {
    if (bytes <= 0 || bytes % 16)
        return fail(PA_ERR_INVALID_ARG, "bytes %lld is not a positive multiple of 16",
                    (long long)bytes);
    CHECK_PTR(buf, 16);
    CHECK_PTR(sink, 4);
    const void *dbuf, *dsink;
    if (!device_view(buf, &dbuf) || !device_view(sink, &dsink))
        return fail(PA_ERR_INVALID_ARG, "probe buffers must be memory the device can address");
    return hip_status(pa::launch_probe_stream_read(dbuf, (size_t)bytes, (void *)dsink,
                                                   (hipStream_t)stream),
                      "probe_stream_read");
}

pa_status pa_probe_mfma_bf16(void *sink, int32_t iters, double *flops, void *stream) {
    if (iters < 1) return fail(PA_ERR_INVALID_ARG, "iters must be >= 1");
    CHECK_PTR(sink, 4);
    const void *dsink;
    if (!device_view(sink, &dsink))
        return fail(PA_ERR_INVALID_ARG, "sink must be memory the device can address");
    if (flops) *flops = pa::probe_mfma_flops(iters);
    return hip_status(pa::launch_probe_mfma_bf16((void *)dsink, iters, (hipStream_t)stream),
                      "probe_mfma_bf16");
}

}  // extern "C"
