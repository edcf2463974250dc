/*
 * pa.h -- C ABI of libpa.so: paged KV-cache attention (PagedAttention) on
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed.  A sequence's keys and values live in fixed-size physical
 * blocks of B tokens drawn from one pool, and a per-sequence block table maps
 * logical block j / B to its physical block ("Configuring vLLM and
 * PagedAttention for High Throughput Enterprise LLM Serving", section
 * "Architectural Foundations: PagedAttention & Virtual Memory", attention
 * equation and the block-table lookup after it).  Attention is the plain
 * softmax(q.k^T * scale) V over the sequence's keys in logical order; the
 * paging only changes where keys and values are read from.  Blocks hold 16 or
 * 32 tokens ("vLLM Guide: High-Throughput Multi-GPU LLM Serving with
 * PagedAttention", section "What Is PagedAttention?").
 *
 * Layouts (row-major, contiguous, element type given by `dtype`):
 *   key_cache, value_cache : [num_blocks][num_kv_heads][block_size][head_dim]
 *   block_tables           : int32 [rows][max_blocks_per_seq]
 *   decode query / out     : [num_seqs][num_q_heads][head_dim]
 *   prefill query / out    : [total_query_tokens][num_q_heads][head_dim]
 *   new key / value        : [num_tokens][num_kv_heads][head_dim]
 *   slot_mapping           : int64 [num_tokens], slot = block * block_size + offset
 * Grouped-query attention: q head h reads kv head h / (num_q_heads / num_kv_heads).
 *
 * Conventions shared by every entry point.
 *   - Every pointer argument is a DEVICE pointer owned by the caller; the
 *     library allocates no memory and keeps no pointer after it returns.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and the call never synchronises.  Results are visible once the stream
 *     reaches that point.
 *   - Argument checks run on the host before anything is launched.  Any
 *     status other than PA_OK means nothing was enqueued; pa_last_error()
 *     then returns a thread-local description.
 *   - Device-side data are not validated on the host (that would need a
 *     synchronising copy).  Kernels stay inside the buffers whatever the
 *     data: a block-table entry outside [0, num_blocks) makes those tokens
 *     count as absent in decode (prefill reads block 0 in its place), a slot
 *     outside [0, num_blocks * block_size) is skipped, and context lengths are
 *     clamped to max_context_len (and to max_blocks_per_seq * block_size).
 *     Such inputs are caller errors and their results are unspecified.
 *     With the environment variable PA_DEBUG set (to anything but "0"), every
 *     entry point first copies the tables it will read to the host (after
 *     the work already queued on its stream, so the call synchronises) and
 *     checks them: table entries a context reaches inside [0, num_blocks),
 *     0 <= context_lens <= max_context_len (prefill: queries per chunk <=
 *     its context, cu_query_lens[0] == 0), slots inside the pool and distinct,
 *     copy pairs inside their pools with distinct destinations.  A violation
 *     returns PA_ERR_INVALID_ARG and launches nothing.
 *   - Supported: dtype PA_F32 or PA_BF16 (prefill: PA_BF16 only), head_dim
 *     64 or 128, block_size 16 or 32, num_q_heads / num_kv_heads in
 *     {1, 2, 4, 8}.  Other shapes return PA_ERR_UNSUPPORTED.
 *   - All pointers must be 16-byte aligned (PA_ERR_INVALID_ARG otherwise);
 *     the decode workspace 256-byte aligned (PA_ERR_WORKSPACE otherwise).
 *   - Entry points are reentrant; concurrent calls on different streams must
 *     not share output or workspace buffers.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, bad size, inconsistent shape */
    PA_ERR_UNSUPPORTED = 2,  /* dtype, head_dim, block_size or group size not built */
    PA_ERR_WORKSPACE = 3,    /* decode workspace missing or too small */
    PA_ERR_HIP = 4,          /* the HIP runtime refused the launch */
    PA_ERR_POOL_EXHAUSTED = 5  /* block manager: too few free blocks (nothing changed) */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/* Version of this ABI (bumped on any incompatible change). */
int32_t pa_abi_version(void);

/* Short name of a status code. */
const char *pa_status_string(int32_t status);

/* Thread-local detail of the last non-OK status returned on this thread. */
const char *pa_last_error(void);

/*
 * pa_reshape_and_cache -- write the keys and values of new tokens into their
 * slots of the block pools.
 *
 * For every t < num_tokens with slot_mapping[t] >= 0: block = slot / block_size,
 * offset = slot % block_size, and for each kv head h the head_dim elements
 * key[t][h][:] are copied bit for bit to key_cache[block][h][offset][:] (and
 * value likewise).  Negative slots are padding and are skipped.  Slots must be
 * distinct (two tokens writing one slot race).  Blocks are taken on demand as
 * sequences grow, which is why a new token can land anywhere in the pool
 * ("Configuring vLLM and PagedAttention ...", section "Architectural
 * Foundations: PagedAttention & Virtual Memory").
 *
 * key, value      : [num_tokens][num_kv_heads][head_dim], read
 * key_cache, value_cache : pools, written only at the given slots
 * num_tokens == 0 is valid and enqueues nothing.
 */
pa_status pa_reshape_and_cache(const void *key, const void *value, void *key_cache,
                               void *value_cache, const int64_t *slot_mapping,
                               int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int64_t num_blocks, int32_t dtype,
                               void *stream);

/*
 * Partition size that the fixed-partition decode path would pick for this
 * batch (tokens of one sequence per workgroup, a multiple of 16); a
 * convenience for callers that pass an explicit partition_size.  pa_decode
 * itself treats partition_size == 0 as the balanced split described below.
 */
int32_t pa_decode_auto_partition_size(int32_t num_seqs, int32_t num_kv_heads,
                                      int32_t max_context_len, int32_t block_size);

/*
 * Bytes of device workspace pa_decode (and pa_decode_append) needs for these
 * arguments, planned exactly as pa_decode plans them (0 is never returned; a
 * small minimum is always asked).  The workspace must be 256-byte aligned;
 * its contents need no initialisation and are scratch between calls.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size,
                                 int32_t max_context_len, int32_t partition_size);

/*
 * pa_decode -- one query token per sequence against its paged context.
 *
 * out[s][h][:] = sum_j A_j V_s[j],  A_j = exp(x_j) / sum_m exp(x_m),
 * x_j = scale * (query[s][h] . K_s[j]), j < context_lens[s],
 * with K_s[j] = key_cache[block_tables[s][j / block_size]][h / G][j % block_size]
 * (the attention equation and block-table lookup of "Configuring vLLM and
 * PagedAttention ...", section "Architectural Foundations"); decode reads every
 * cached key and value once, which is what bounds it by memory bandwidth
 * (same page, section "Memory Bottlenecks in Autoregressive LLM Inference").
 * context_lens[s] == 0 gives zeros.  The new token of a step is expected to
 * be in the cache already (pa_reshape_and_cache first), so it is at position
 * context_lens[s] - 1.
 *
 * Split of the work (split-K over the context): the keys of every (sequence,
 * kv head) are cut into units of 16 tokens.
 *   partition_size == 0 and num_seqs <= 8192: balanced split.  All units of
 *     the batch are dealt to a fixed number of waves in equal contiguous
 *     ranges, whatever the mix of context lengths; a (sequence, kv head)
 *     that spans several waves leaves one partial result per wave.
 *   partition_size > 0 (a multiple of block_size and of 16, at most 4096),
 *     or more than 8192 sequences: fixed partitions of partition_size tokens
 *     (automatic size for partition_size == 0), one workgroup each.
 * Partial results (fp32 running max, sum and unnormalised output) go through
 * the workspace and a second kernel merges them with log-sum-exp rescaling.
 * max_context_len must be >= every context_lens[s]; it sizes the launch.
 * Inputs are bf16 or fp32; arithmetic is fp32; out is written in dtype
 * (bf16 by round-to-nearest-even).  The result does not depend on the split
 * beyond fp32 rounding.
 */
pa_status pa_decode(void *out, const void *query, const void *key_cache,
                    const void *value_cache, const int32_t *block_tables,
                    const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
                    int32_t partition_size, float scale, int32_t dtype, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * pa_decode_no_alloc -- pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops that forbid hipMalloc,
 * harnesses that forbid it): the same arguments, split, kernels and results
 * as pa_decode, bit for bit, without the workspace arguments.
 *
 * The workspace lives in a static device array inside the library, one copy
 * per GPU, of pa_decode_no_alloc_max_workspace() bytes (32 MiB), held from
 * the first call on a device until the process ends.  The call allocates
 * nothing.  A batch whose pa_decode_workspace_bytes() exceeds that size is
 * rejected with PA_ERR_WORKSPACE before anything is enqueued.  The array is
 * found for the current device (hipGetDevice), which must be the device of
 * `stream`.  Every call on one GPU shares that GPU's array and leaves its
 * contents behind (no call needs them cleared): calls that overlap on one
 * GPU (on different streams, or from different threads without ordering)
 * race and their outputs are undefined; order them on one stream.
 */
pa_status pa_decode_no_alloc(void *out, const void *query, const void *key_cache,
                             const void *value_cache, const int32_t *block_tables,
                             const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t max_blocks_per_seq, int64_t num_blocks,
                             int32_t max_context_len, int32_t partition_size, float scale,
                             int32_t dtype, void *stream);

/* Bytes of the static workspace pa_decode_no_alloc uses on each GPU. */
size_t pa_decode_no_alloc_max_workspace(void);

/*
 * pa_decode_shared_prefix -- decode (bf16) for a batch whose sequences all
 * start with the same prompt blocks: entries 0 .. prefix_blocks - 1 of every
 * row of block_tables name the same physical blocks (a common prompt reused
 * through prefix caching: "Configuring vLLM and PagedAttention for High
 * Throughput Enterprise LLM Serving", section "Zero-Copy Prefix Caching &
 * Shared Sampling"; "vLLM High-Performance Inference Engine: PagedAttention
 * Principles and Deployment Guide", section "PagedAttention Architecture Deep
 * Dive").  The result is that of pa_decode on the same arguments (dtype
 * bf16), up to fp32 rounding order; pa_decode itself stays unchanged.
 *
 * Instead of streaming the prefix blocks once per sequence, one pass attends
 * the queries of all sequences to them (16 / G sequences per matrix-core
 * tile, so each K/V byte of the prefix is read once per tile), a second pass
 * streams each sequence's tokens past the prefix (the balanced split of
 * pa_decode), and the reduce merges both sets of partial results with
 * log-sum-exp rescaling.  A sequence with context_lens[s] <= prefix_blocks *
 * block_size attends to its own first context_lens[s] tokens only.
 *
 * The prefix pass runs on a stream the library creates for the current
 * device (default priority, on the first call on that device, kept until the
 * process ends), forked from `stream` and joined back into it with events
 * before the reduce, so it runs beside the suffix pass; the current device
 * must be the device of `stream`.  Everything the call enqueues is ordered
 * after earlier work on `stream`, and later work on `stream` waits for all of
 * it.  Calls from several host threads may overlap (their enqueue sequences
 * are serialised).
 *
 * Arguments as pa_decode, plus prefix_blocks in [0, max_blocks_per_seq]
 * (0: the plain balanced decode); num_seqs at most 8192 (else
 * PA_ERR_UNSUPPORTED); workspace (256-byte aligned) of at least
 * pa_decode_shared_prefix_workspace_bytes() bytes, else PA_ERR_WORKSPACE.
 * Equal prefix rows are the caller's contract; with PA_DEBUG=1 they are
 * checked on the host (PA_ERR_INVALID_ARG).
 */
pa_status pa_decode_shared_prefix(void *out, const void *query, const void *key_cache,
                                  const void *value_cache, const int32_t *block_tables,
                                  const int32_t *context_lens, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t max_blocks_per_seq,
                                  int64_t num_blocks, int32_t max_context_len,
                                  int32_t prefix_blocks, float scale, void *workspace,
                                  size_t workspace_bytes, void *stream);

size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                               int32_t num_kv_heads, int32_t head_dim,
                                               int32_t block_size, int32_t max_context_len,
                                               int32_t prefix_blocks);

/*
 * The two phases of pa_decode, callable on their own (same arguments; the
 * pair enqueued back to back on one stream is exactly pa_decode).
 * pa_decode_partitions writes the final output of every sequence that fits in
 * one partition and the per-partition partial results of the others into the
 * workspace; pa_decode_reduce merges those partials (log-sum-exp rescaling)
 * into out and writes zeros for empty contexts.  For a small batch of short
 * contexts (partition_size 0, at most 1,024 (sequence, kv head) pairs and
 * max_context_len <= 128) the first phase gives each pair one wave, writes
 * every output row itself (zeros for empty contexts), and pa_decode_reduce
 * returns PA_OK without launching anything; pa_decode_needs_reduce tells the
 * two cases apart.
 */
pa_status pa_decode_partitions(void *out, const void *query, const void *key_cache,
                               const void *value_cache, const int32_t *block_tables,
                               const int32_t *context_lens, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t max_blocks_per_seq,
                               int64_t num_blocks, int32_t max_context_len,
                               int32_t partition_size, float scale, int32_t dtype,
                               void *workspace, size_t workspace_bytes, void *stream);

pa_status pa_decode_reduce(void *out, const int32_t *context_lens, int32_t num_seqs,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t max_blocks_per_seq,
                           int32_t max_context_len, int32_t partition_size, int32_t dtype,
                           const void *workspace, size_t workspace_bytes, void *stream);

/*
 * 1 if pa_decode_reduce launches work for these sizes (the same arguments as
 * pa_decode_partitions), 0 if pa_decode_partitions finishes every row by
 * itself (the one-wave-per-pair case above, or an empty batch).  Invalid
 * sizes give 1.  A host-side query: no device access.
 */
int32_t pa_decode_needs_reduce(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t max_context_len,
                               int32_t partition_size);

/*
 * pa_decode_append -- one decode step with its new tokens: the cache write of
 * pa_reshape_and_cache and pa_decode in one pass.
 *
 * For every sequence s with 0 < context_lens[s] <= max_context_len, the new
 * token's rows new_key[s][:][:] and new_value[s][:][:] ([num_seqs]
 * [num_kv_heads][head_dim]) are written bit for bit into the slot of position
 * context_lens[s] - 1, i.e. block block_tables[s][(L - 1) / block_size] at
 * offset (L - 1) % block_size, and then the same attention as pa_decode is
 * computed over positions 0 .. L - 1, the new token included.  The result and
 * the pools afterwards equal pa_reshape_and_cache with those slots followed by
 * pa_decode.  With the balanced split the wave that reads the new token's
 * unit writes it and uses it from registers, so no extra launch is needed.
 *
 * The block holding the new token must not be shared with another sequence
 * of the batch (copy it first, as for any write into a shared block).
 * Arguments as pa_decode, plus new_key and new_value (read).
 */
pa_status pa_decode_append(void *out, const void *query, const void *new_key,
                           const void *new_value, void *key_cache, void *value_cache,
                           const int32_t *block_tables, const int32_t *context_lens,
                           int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                           int64_t num_blocks, int32_t max_context_len, int32_t partition_size,
                           float scale, int32_t dtype, void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * The first phase of pa_decode_append (the cache write and the partial
 * results); pa_decode_reduce with the same arguments completes it.
 */
pa_status pa_decode_append_partitions(void *out, const void *query, const void *new_key,
                                      const void *new_value, void *key_cache, void *value_cache,
                                      const int32_t *block_tables, const int32_t *context_lens,
                                      int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_blocks_per_seq,
                                      int64_t num_blocks, int32_t max_context_len,
                                      int32_t partition_size, float scale, int32_t dtype,
                                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_prefill_chunk -- a chunk of consecutive prompt tokens attends causally to
 * the paged cache ("Configuring vLLM and PagedAttention ...", section
 * "High-Throughput Batching: Continuous Batching & Chunked Prefill": long
 * prompts are split into chunks of e.g. 512 tokens; the prefill phase is
 * compute-bound, section "Memory Bottlenecks in Autoregressive LLM
 * Inference").
 *
 * Chunk c owns query rows cu_query_lens[c] .. cu_query_lens[c+1]-1 (n_c rows)
 * and context_lens[c] keys in the cache, which include the chunk's own
 * tokens (written by pa_reshape_and_cache first).  Query i of the chunk is at
 * position context_lens[c] - n_c + i and attends to keys 0 .. that position.
 * block_tables has one row per chunk.  max_query_len >= every n_c sizes the
 * launch.  bf16 only: QK^T and PV run on the matrix cores (bf16 inputs, fp32
 * accumulation), softmax in fp32, out in bf16.  scale must be positive and
 * finite (the attention scale 1 / sqrt(head_dim) of the pages is); other
 * values return PA_ERR_INVALID_ARG.
 */
pa_status pa_prefill_chunk(void *out, const void *query, const void *key_cache,
                           const void *value_cache, const int32_t *block_tables,
                           const int32_t *cu_query_lens, const int32_t *context_lens,
                           int32_t num_chunks, int32_t max_query_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                           int32_t dtype, void *stream);

/*
 * pa_prefill_chunk_append -- pa_prefill_chunk that also writes the chunks'
 * own K/V rows into the pools inside the same pass, as pa_decode_append does
 * for decode (the chunk's tokens are the ones a chunked-prefill step adds:
 * "Configuring vLLM and PagedAttention ...", section "High-Throughput
 * Batching: Continuous Batching & Chunked Prefill").
 *
 * new_key / new_value [Tq, Hkv, d] (bf16, device) hold the K and V rows of
 * the query tokens: row cu_query_lens[c] + i is the token at position
 * context_lens[c] - n_c + i of chunk c, written into slot
 * (block_tables[c][pos / B], pos % B) -- exactly what pa_reshape_and_cache
 * with those slots followed by pa_prefill_chunk computes and leaves in the
 * pools.  Keys at those positions are read from new_key / new_value, so no
 * ordering with the writes is needed; positions outside the table, or table
 * entries outside the pool, are not written (caller errors).  Other
 * arguments, checks and errors as pa_prefill_chunk (bf16 pools).
 */
pa_status pa_prefill_chunk_append(void *out, const void *query, const void *new_key,
                                  const void *new_value, void *key_cache, void *value_cache,
                                  const int32_t *block_tables, const int32_t *cu_query_lens,
                                  const int32_t *context_lens, int32_t num_chunks,
                                  int32_t max_query_len, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                                  int32_t dtype, void *stream);

/*
 * pa_copy_blocks -- copy whole KV blocks between pools: copy-on-write inside
 * the device pool, and swap of a paused request's pages to host memory and
 * back.
 *
 * Shared physical blocks are copied before one sequence writes into its own
 * copy ("vLLM Guide: High-Throughput Multi-GPU LLM Serving with
 * PagedAttention", section "What Is PagedAttention?": copy-on-write), and when
 * the pool is full the pages of a paused request move to host RAM over PCIe
 * and later back ("Configuring vLLM and PagedAttention for High Throughput
 * Enterprise LLM Serving", section "Quick Answers", the question on KV-cache
 * offloading).
 *
 * For every pair i < num_pairs, block block_mapping[2i] of the source pools
 * is copied bit for bit into block block_mapping[2i + 1] of the destination
 * pools, in the K pool and in the V pool.  A block is block_bytes bytes
 * (num_kv_heads * block_size * head_dim * element bytes for the pool layout
 * above; a multiple of 16).  Source and destination pools are
 * [src_num_blocks] / [dst_num_blocks] blocks; they may be the same pools
 * (copy-on-write).
 *
 * Memory: every pointer (the four pools and the int64 [num_pairs][2] mapping)
 * must be device memory or pinned host memory that the device can map
 * (hipHostMalloc); anything else is rejected with PA_ERR_INVALID_ARG before
 * any launch.  The caller owns all of it.  Host pools are read or written by
 * the kernel across PCIe; enqueue on the caller's stream, synchronise before
 * touching host pools from the CPU.
 *
 * Preconditions (not checked: the mapping is device data): destination ids
 * are distinct, and, for copies inside one pool, no block is both a source
 * and a destination; otherwise the result depends on the order of the copies.
 * Pairs with an id outside its pool are skipped.  num_pairs == 0 is a no-op.
 */
pa_status pa_copy_blocks(const void *src_key_cache, const void *src_value_cache,
                         void *dst_key_cache, void *dst_value_cache,
                         const int64_t *block_mapping, int32_t num_pairs, int64_t src_num_blocks,
                         int64_t dst_num_blocks, int64_t block_bytes, void *stream);

/*
 * FP8 KV cache -- pools of 8-bit e4m3 codes, half the bytes of bf16.
 *
 * The pages list quantised KV caches among the engine's features and run an
 * FP8 KV cache in their engine example ("vLLM Guide: High-Throughput
 * Multi-GPU LLM Serving with PagedAttention", the quantisation support among
 * the pillars of the engine, and the FP8 engine example); they give no format
 * detail, so the following is this library's reading.
 *
 * Format: every element is one byte, the OCP e4m3 code (1 sign, 4 exponent
 * bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN; largest
 * finite 448, smallest subnormal 2^-9) of x / scale, with one fp32 scale per
 * pool (k_scale for K, v_scale for V).  Encoding: y = x * (1 / scale) in
 * fp32, then the nearest e4m3 value, ties to the even code, saturating at
 * +-448; NaN -> 0x7F.  Decoding: value = code's value * scale.
 *
 * Layouts (uint8):
 *   key_cache   : [num_blocks][num_kv_heads][block_size][head_dim] (as bf16)
 *   value_cache : [num_blocks][num_kv_heads][head_dim][block_size] -- each
 *                 page transposed, so a dim's tokens are contiguous.
 * The page size is block_size * head_dim bytes.
 */

/*
 * pa_reshape_and_cache_fp8 -- pa_reshape_and_cache into FP8 pools: for every
 * t with slot_mapping[t] >= 0, the e4m3 codes of key[t][h][:] / k_scale go to
 * key_cache[block][h][offset][:] and those of value[t][h][:] / v_scale to
 * value_cache[block][h][:][offset].  key, value: [num_tokens][num_kv_heads]
 * [head_dim] in dtype (PA_F32 or PA_BF16).  Scales must be positive and
 * finite (PA_ERR_INVALID_ARG).  Other conventions as pa_reshape_and_cache.
 */
pa_status pa_reshape_and_cache_fp8(const void *key, const void *value, void *key_cache,
                                   void *value_cache, const int64_t *slot_mapping,
                                   int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int64_t num_blocks, int32_t dtype,
                                   float k_scale, float v_scale, void *stream);

/*
 * pa_decode_fp8 -- pa_decode over FP8 pools: the same attention, with
 * K_s[j] and V_s[j] the decoded codes times k_scale and v_scale.  query and
 * out are bf16 [num_seqs][num_q_heads][head_dim]; arithmetic is fp32 with
 * both products on the bf16 matrix cores (the codes widen to bf16 exactly).
 * Always the balanced split (no partition_size); num_seqs <= 8192
 * (PA_ERR_UNSUPPORTED otherwise).  The workspace is
 * pa_decode_workspace_bytes(..., partition_size = 0).  Other conventions,
 * errors and the context-length rules as pa_decode.
 * pa_decode_fp8_partitions is its first phase; pa_decode_reduce with
 * partition_size 0 and dtype PA_BF16 completes it.
 */
pa_status pa_decode_fp8(void *out, const void *query, const void *key_cache,
                        const void *value_cache, const int32_t *block_tables,
                        const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
                        float scale, float k_scale, float v_scale, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * pa_decode_fp8_append -- one FP8 decode step with its new tokens: the bf16
 * rows new_key[s], new_value[s] ([num_seqs][num_kv_heads][head_dim]) are
 * quantised into the slot of position context_lens[s] - 1 of sequence s
 * (block block_tables[s][(L - 1) / block_size], offset (L - 1) % block_size),
 * exactly as pa_reshape_and_cache_fp8 would, and the step attends over them:
 * the pools and out equal pa_reshape_and_cache_fp8 followed by pa_decode_fp8,
 * bit for bit.  The write happens inside the decode pass (no extra launch).
 * Sequences with context_lens[s] == 0 or above max_context_len get no write.
 * pa_decode_fp8_append_partitions is its first phase; pa_decode_reduce (as
 * for pa_decode_fp8) completes it.  Other conventions as pa_decode_fp8.
 */
pa_status pa_decode_fp8_append(void *out, const void *query, const void *new_key,
                               const void *new_value, void *key_cache, void *value_cache,
                               const int32_t *block_tables, const int32_t *context_lens,
                               int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                               int64_t num_blocks, int32_t max_context_len, float scale,
                               float k_scale, float v_scale, void *workspace,
                               size_t workspace_bytes, void *stream);

pa_status pa_decode_fp8_append_partitions(
    void *out, const void *query, const void *new_key, const void *new_value, void *key_cache,
    void *value_cache, const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len, float scale,
    float k_scale, float v_scale, void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_prefill_chunk_fp8 -- pa_prefill_chunk over FP8 pools: the same causal
 * chunks, with keys and values the decoded codes times k_scale and v_scale.
 * query and out are bf16 [total_query_tokens][num_q_heads][head_dim]; both
 * products run on the bf16 matrix cores (the codes widen to bf16 exactly).
 * The chunk's own new keys and values must already be in the pools
 * (pa_reshape_and_cache_fp8).  Other arguments, conventions and errors as
 * pa_prefill_chunk; scale, k_scale and v_scale must be positive and finite.
 */
pa_status pa_prefill_chunk_fp8(void *out, const void *query, const void *key_cache,
                               const void *value_cache, const int32_t *block_tables,
                               const int32_t *cu_query_lens, const int32_t *context_lens,
                               int32_t num_chunks, int32_t max_query_len, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                               float k_scale, float v_scale, void *stream);

pa_status pa_decode_fp8_partitions(void *out, const void *query, const void *key_cache,
                                   const void *value_cache, const int32_t *block_tables,
                                   const int32_t *context_lens, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t max_blocks_per_seq,
                                   int64_t num_blocks, int32_t max_context_len, float scale,
                                   float k_scale, float v_scale, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * pa_decode_fp8_shared_prefix -- pa_decode_shared_prefix over e4m3 pools:
 * the prefix blocks shared by every sequence (entries 0 .. prefix_blocks - 1
 * of every table row) are read once per matrix-core tile of 16 / G
 * sequences, the tokens past them by the balanced split of pa_decode_fp8,
 * and the reduce merges both ("Configuring vLLM and PagedAttention for High
 * Throughput Enterprise LLM Serving", section "Zero-Copy Prefix Caching &
 * Shared Sampling", with the quantised cache of "vLLM Guide: High-Throughput
 * Multi-GPU LLM Serving with PagedAttention", the quantisation support among
 * the engine's pillars).  The result is that of pa_decode_fp8 on the same
 * arguments up to fp32 rounding order.  Arguments, layouts and errors as
 * pa_decode_fp8 plus prefix_blocks, workspace and side stream as
 * pa_decode_shared_prefix; the workspace size is
 * pa_decode_shared_prefix_workspace_bytes() (the same records).
 */
pa_status pa_decode_fp8_shared_prefix(void *out, const void *query, const void *key_cache,
                                      const void *value_cache, const int32_t *block_tables,
                                      const int32_t *context_lens, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size,
                                      int32_t max_blocks_per_seq, int64_t num_blocks,
                                      int32_t max_context_len, int32_t prefix_blocks, float scale,
                                      float k_scale, float v_scale, void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * Block manager (host side) -- the allocator that produces the block tables
 * and slot mappings the kernels above read.
 *
 * The pool holds num_blocks physical blocks of block_size tokens.  Each
 * sequence's block table maps its logical blocks to physical ones; a block
 * carries a reference count; blocks come from a free pool on demand as a
 * sequence grows and go back when it is freed ("vLLM High-Performance
 * Inference Engine: PagedAttention Principles and Deployment Guide", section
 * "PagedAttention Architecture Deep Dive"; "Configuring vLLM and
 * PagedAttention for High Throughput Enterprise LLM Serving", section
 * "Architectural Foundations: PagedAttention & Virtual Memory").  Sequences
 * share blocks after a fork or through the prefix cache, and a write into a
 * shared, partly filled block first copies it ("vLLM Guide: High-Throughput
 * Multi-GPU LLM Serving with PagedAttention", section "What Is
 * PagedAttention?": copy-on-write).  With enable_prefix_cache, every full
 * block is indexed by a chained hash of the token ids of the sequence up to
 * its end, and a new sequence whose prompt starts with the same full blocks
 * reuses them (automatic prefix caching); reuse requires equal stored tokens
 * and the same preceding physical block, never a hash match alone.
 *
 * Policy: the free pool is first-in first-out (blocks 0, 1, ... at first); a
 * freed block that is in the prefix index stays reusable until the pool hands
 * it out again.  All calls are host-only, synchronous and not thread-safe
 * (one manager per scheduler thread).  Errors: PA_ERR_INVALID_ARG (bad
 * argument or unknown / duplicate sequence id), PA_ERR_POOL_EXHAUSTED (the
 * pool has too few free blocks; nothing was changed).
 */
typedef struct pa_block_manager pa_block_manager;

typedef struct pa_bm_stats {
    int64_t num_blocks;     /* pool size */
    int64_t free_blocks;    /* blocks in the free pool (cached ones included) */
    int64_t used_blocks;    /* num_blocks - free_blocks */
    int64_t shared_blocks;  /* blocks referenced more than once */
    int64_t cached_blocks;  /* blocks in the prefix index */
    int64_t num_seqs;
    int64_t seq_tokens;     /* sum of sequence lengths */
    int64_t seq_slots;      /* sum over sequences of table length x block_size */
    int64_t prefix_hits;    /* blocks reused from the prefix index so far */
} pa_bm_stats;

/* Creates a manager over a pool of num_blocks blocks; *out owns it. */
pa_status pa_bm_create(int64_t num_blocks, int32_t block_size, int32_t enable_prefix_cache,
                       pa_block_manager **out);
void pa_bm_destroy(pa_block_manager *bm);

/*
 * Registers sequence seq_id with its prompt (num_tokens token ids, host
 * memory) and allocates its blocks.  slot_mapping[t] (host, num_tokens
 * entries) receives the slot (block * block_size + offset) of prompt token t
 * for pa_reshape_and_cache, or -1 when the token's block came from the prefix
 * cache (its keys and values are already in the pool).  *num_cached_tokens
 * (optional) receives that count.  At most (num_tokens - 1) / block_size
 * leading blocks are reused, so the prompt's last token always gets a slot
 * and a query row to compute (its output gives the next token).  Reused
 * blocks that are cached but free count against the free pool: when the
 * pool cannot hold the rest, PA_ERR_POOL_EXHAUSTED is returned before any
 * change.
 */
pa_status pa_bm_add_sequence(pa_block_manager *bm, int64_t seq_id, const int32_t *tokens,
                             int32_t num_tokens, int64_t *slot_mapping,
                             int32_t *num_cached_tokens);

/*
 * Appends one token to seq_id and returns its slot in *slot.  A new block is
 * taken when the last one is full; when the last block is shared and partly
 * filled, a new block replaces it in this sequence's table and the pair
 * (old, new) is queued for pa_copy_blocks (see pa_bm_take_copies).
 */
pa_status pa_bm_append(pa_block_manager *bm, int64_t seq_id, int32_t token, int64_t *slot);

/* child shares every block of parent (reference counts + 1). */
pa_status pa_bm_fork(pa_block_manager *bm, int64_t parent, int64_t child);

/* Drops seq_id; blocks whose count reaches 0 return to the free pool. */
pa_status pa_bm_free(pa_block_manager *bm, int64_t seq_id);

/*
 * Moves the queued copy-on-write pairs (source block, destination block),
 * int64 [n][2], into pairs and returns n.  If max_pairs < n (or pairs is
 * NULL) nothing is moved and n is returned.  Run pa_copy_blocks on them
 * before the step's cache write.  Returns -1 if bm is NULL.
 */
int32_t pa_bm_take_copies(pa_block_manager *bm, int64_t *pairs, int32_t max_pairs);

/*
 * The block table row of seq_id (row: max_blocks entries, host; may be NULL
 * to query the sizes), its number of blocks and its context length.
 */
pa_status pa_bm_block_table(const pa_block_manager *bm, int64_t seq_id, int32_t *row,
                            int32_t max_blocks, int32_t *num_blocks, int32_t *context_len);

/*
 * One decode step for a batch: appends tokens[i] to seq_ids[i] (distinct
 * ids) in order, as pa_bm_append, and writes the slots (the step's
 * slot_mapping).  The blocks the step needs are checked first: on
 * PA_ERR_POOL_EXHAUSTED or PA_ERR_INVALID_ARG nothing has changed.
 */
pa_status pa_bm_append_batch(pa_block_manager *bm, const int64_t *seq_ids,
                             const int32_t *tokens, int32_t n, int64_t *slots);

/*
 * The block tables of seq_ids as the kernels take them: tables is int32
 * [n][max_blocks] (host), row i holds seq_ids[i]'s table padded with fill;
 * context_lens (optional, int32 [n]) receives the lengths.  A table longer
 * than max_blocks, or an unknown id, is PA_ERR_INVALID_ARG (nothing written).
 */
pa_status pa_bm_block_tables(const pa_block_manager *bm, const int64_t *seq_ids, int32_t n,
                             int32_t *tables, int32_t max_blocks, int32_t fill,
                             int32_t *context_lens);

/* Pool statistics; internal fragmentation = 1 - seq_tokens / seq_slots. */
pa_status pa_bm_get_stats(const pa_block_manager *bm, pa_bm_stats *stats);

/*
 * Ceiling probes -- the attainable rates the attention kernels are measured
 * against (the pages report the decode kernel as bound by memory bandwidth:
 * "vLLM High-Performance Inference Engine: PagedAttention Principles and
 * Deployment Guide", section "PagedAttention Architecture Deep Dive").  They
 * compute nothing of the method.
 *
 * pa_probe_stream_read: reads bytes (a positive multiple of 16) of device
 * memory buf once with 16-byte loads spread over the whole chip, and writes
 * pa_probe_sink_words() 32-bit words to sink (device memory, caller-owned),
 * so that the read cannot be dropped.  Bytes / time is the streaming read
 * rate.  buf must be 16-byte aligned, sink 4-byte aligned.
 *
 * pa_probe_mfma_bf16: every SIMD issues iters (>= 1) rounds of 4 independent
 * 32x32x16 bf16 matrix products on register operands and writes
 * pa_probe_sink_words() floats to sink; *flops (host, optional) receives the
 * flops the launch performs.  Flops / time is the sustained dense bf16 rate.
 *
 * Both are asynchronous on stream; errors: PA_ERR_INVALID_ARG (bad size,
 * null or misaligned pointer, pointer the device cannot address), PA_ERR_HIP.
 */
int64_t pa_probe_sink_words(void);
pa_status pa_probe_stream_read(const void *buf, int64_t bytes, void *sink, void *stream);
pa_status pa_probe_mfma_bf16(void *sink, int32_t iters, double *flops, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
