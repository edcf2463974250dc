/*
 * CPU oracle for paged KV-cache attention -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * may call this code.  It shares nothing with the GPU library: no headers,
 * no helpers, no tables.  It is plain, slow and written to be checked by eye
 * against the definition on the pages:
 *
 *   "Configuring vLLM and PagedAttention for High Throughput Enterprise LLM
 *   Serving", section "Architectural Foundations: PagedAttention & Virtual
 *   Memory", attention-matrix equation and the block-table lookup that
 *   follows it: the weight of query i on key j is exp(q_i.k_j/sqrt d) over
 *   the sum of the same term across all keys, and key j is reached through
 *   block-table entry j / B, B tokens per block.
 *
 * Everything is computed in double precision.  bf16 inputs are widened
 * exactly (their 16 bits become the top half of an fp32 word).
 *
 * Readings of points the pages leave open (each is also listed in the
 * design notes):
 *   - j / B is floor division and the offset inside the block is j mod B
 *     (the only reading that fits the diagram of "vLLM Guide:
 *     High-Throughput Multi-GPU LLM Serving with PagedAttention", section
 *     "What Is PagedAttention?", where logical tokens 0-15, 16-31 and 32-47
 *     sit in physical blocks 9, 2 and 14).
 *   - the output of attention is the weights times V: out_i = sum_j A_ij v_j.
 *   - d in sqrt(d) is the head dimension; the scale is passed in (fp32) and
 *     widened, so both sides use the same value.
 *   - grouped-query attention: q head h reads kv head h / (Hq / Hkv).
 *   - pool layout: [num_blocks][num_kv_heads][block_size][head_dim], K and V
 *     in separate pools.
 *   - a prefill chunk of n queries over L keys puts query i at absolute
 *     position L - n + i, and it sees keys 0..L-n+i (causal).
 *   - a context of length 0 gives an output of zeros.
 *   - the max-shifted softmax is used; it equals the printed form exactly in
 *     real arithmetic.
 *
 * Status codes: 0 ok, 1 invalid argument, 2 block id out of range,
 * 3 slot out of range, 4 duplicate slot, 5 out of memory.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1

/* ---- element access ---------------------------------------------------- */

static double widen(const void *base, size_t idx, int dtype)
{
    if (dtype == OR_F32)
        return (double)((const float *)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* ---- block-table resolution -------------------------------------------- */

/*
 * Gather the keys (or values) of one sequence and one kv head into a
 * contiguous [L][D] array in logical order.  Token j lives in physical block
 * block_table[j / B] at offset j mod B (the block-table address map of the
 * "Architectural Foundations" section).
 */
int oracle_gather(double *dst, const void *cache, const int32_t *block_table_row,
                  int L, int num_kv_heads, int kv_head, int block_size,
                  int head_dim, int64_t num_blocks, int dtype)
{
    for (int j = 0; j < L; ++j) {
        int64_t phys = block_table_row[j / block_size];
        int off = j % block_size;
        if (phys < 0 || phys >= num_blocks)
            return 2;
        size_t base = (((size_t)phys * num_kv_heads + kv_head) * block_size + off) * head_dim;
        for (int i = 0; i < head_dim; ++i)
            dst[(size_t)j * head_dim + i] = widen(cache, base + i, dtype);
    }
    return 0;
}

/* ---- softmax attention of one query row over contiguous K, V ------------ */

/*
 * out[i] = sum_j A_j V[j][i] with A_j = exp(x_j - max x) / sum_m exp(x_m - max x)
 * and x_j = scale * (q . K[j]).  If weights != NULL the A_j are stored there.
 */
static void attend_row(double *out, const double *q, const double *K, const double *V,
                       int L, int D, double scale, double *x, double *weights)
{
    if (L == 0) {
        for (int i = 0; i < D; ++i)
            out[i] = 0.0;
        return;
    }
    double m = -INFINITY;
    for (int j = 0; j < L; ++j) {
        double dot = 0.0;
        for (int i = 0; i < D; ++i)
            dot += q[i] * K[(size_t)j * D + i];
        x[j] = scale * dot;
        if (x[j] > m)
            m = x[j];
    }
    double Z = 0.0;
    for (int j = 0; j < L; ++j) {
        x[j] = exp(x[j] - m);
        Z += x[j];
    }
    for (int j = 0; j < L; ++j)
        x[j] /= Z;                       /* x now holds A_j */
    for (int i = 0; i < D; ++i)
        out[i] = 0.0;
    for (int j = 0; j < L; ++j)
        for (int i = 0; i < D; ++i)
            out[i] += x[j] * V[(size_t)j * D + i];
    if (weights)
        for (int j = 0; j < L; ++j)
            weights[j] = x[j];
}

/* One query row: gather the first L keys of a table row, then attend. */
static int attend_paged(double *out, const void *q_base, size_t q_off,
                        const void *key_cache, const void *value_cache,
                        const int32_t *bt_row, int L, int num_kv_heads, int kv_head,
                        int block_size, int head_dim, int64_t num_blocks,
                        double scale, int dtype, double *weights)
{
    int D = head_dim;
    size_t n = (size_t)(L > 0 ? L : 1) * D;
    double *K = malloc(n * sizeof(double));
    double *V = malloc(n * sizeof(double));
    double *x = malloc((size_t)(L > 0 ? L : 1) * sizeof(double));
    double *q = malloc((size_t)D * sizeof(double));
    int st = 0;
    if (!K || !V || !x || !q) {
        st = 5;
        goto done;
    }
    st = oracle_gather(K, key_cache, bt_row, L, num_kv_heads, kv_head, block_size, D,
                       num_blocks, dtype);
    if (!st)
        st = oracle_gather(V, value_cache, bt_row, L, num_kv_heads, kv_head, block_size, D,
                           num_blocks, dtype);
    if (st)
        goto done;
    for (int i = 0; i < D; ++i)
        q[i] = widen(q_base, q_off + i, dtype);
    attend_row(out, q, K, V, L, D, scale, x, weights);
done:
    free(K);
    free(V);
    free(x);
    free(q);
    return st;
}

/* ---- decode: one query token per sequence ------------------------------- */

/*
 * out     : double [S][Hq][D]
 * query   : [S][Hq][D] in dtype
 * caches  : [NB][Hkv][B][D] in dtype
 * tables  : int32 [S][max_blocks]; context_lens int32 [S]
 * weights : optional double [S][Hq][max_blocks * B] (attention weights A)
 */
int oracle_decode(double *out, const void *query, const void *key_cache,
                  const void *value_cache, const int32_t *block_tables,
                  const int32_t *context_lens, int num_seqs, int num_q_heads,
                  int num_kv_heads, int head_dim, int block_size, int max_blocks,
                  int64_t num_blocks, float scale, int dtype, double *weights)
{
    if (num_seqs < 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads || head_dim <= 0 ||
        block_size <= 0 || max_blocks < 0)
        return 1;
    for (int s = 0; s < num_seqs; ++s)
        if (context_lens[s] < 0 || context_lens[s] > max_blocks * block_size)
            return 1;
    int group = num_q_heads / num_kv_heads;
    int status = 0;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int s = 0; s < num_seqs; ++s) {
        for (int h = 0; h < num_q_heads; ++h) {
            size_t row = (size_t)s * num_q_heads + h;
            double *w = weights ? weights + row * (size_t)max_blocks * block_size : NULL;
            int st = attend_paged(out + row * head_dim, query, row * head_dim, key_cache,
                                  value_cache, block_tables + (size_t)s * max_blocks,
                                  context_lens[s], num_kv_heads, h / group, block_size,
                                  head_dim, num_blocks, (double)scale, dtype, w);
            if (st) {
#pragma omp atomic write
                status = st;
            }
        }
    }
    return status;
}

/* ---- prefill chunk: causal queries against the paged cache -------------- */

/*
 * Chunk c holds queries cu_query_lens[c] .. cu_query_lens[c+1]-1 of the packed
 * query array; context_lens[c] counts the keys in the cache including the
 * chunk's own.  Query i of the chunk sits at absolute position
 * context_lens[c] - n_c + i and attends to keys 0 .. that position.
 *
 * out   : double [Tq][Hq][D];  query : [Tq][Hq][D]
 */
int oracle_prefill(double *out, const void *query, const void *key_cache,
                   const void *value_cache, const int32_t *block_tables,
                   const int32_t *cu_query_lens, const int32_t *context_lens,
                   int num_chunks, int num_q_heads, int num_kv_heads, int head_dim,
                   int block_size, int max_blocks, int64_t num_blocks, float scale,
                   int dtype)
{
    if (num_chunks < 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
        return 1;
    for (int c = 0; c < num_chunks; ++c) {
        int n = cu_query_lens[c + 1] - cu_query_lens[c];
        if (n < 0 || n > context_lens[c] || context_lens[c] > max_blocks * block_size)
            return 1;
    }
    int group = num_q_heads / num_kv_heads;
    int total = cu_query_lens[num_chunks];
    int status = 0;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int t = 0; t < total; ++t) {
        for (int h = 0; h < num_q_heads; ++h) {
            int c = 0;
            while (cu_query_lens[c + 1] <= t)
                ++c;
            int n = cu_query_lens[c + 1] - cu_query_lens[c];
            int i = t - cu_query_lens[c];
            int pos = context_lens[c] - n + i;
            size_t row = (size_t)t * num_q_heads + h;
            int st = attend_paged(out + row * head_dim, query, row * head_dim, key_cache,
                                  value_cache, block_tables + (size_t)c * max_blocks,
                                  pos + 1, num_kv_heads, h / group, block_size, head_dim,
                                  num_blocks, (double)scale, dtype, NULL);
            if (st) {
#pragma omp atomic write
                status = st;
            }
        }
    }
    return status;
}

/* ---- cache write: scatter new K/V into their slots ---------------------- */

/*
 * For every new token t with slot_mapping[t] >= 0: block = slot / B,
 * offset = slot mod B, and for every kv head the head_dim elements are copied
 * bit for bit into [block][head][offset][:] of each pool.  Negative slots
 * are padding and are skipped.  A slot at or beyond num_blocks * B, or one
 * that appears twice, is an error and nothing is written.
 */
int oracle_reshape_and_cache(const void *key, const void *value, void *key_cache,
                             void *value_cache, const int64_t *slot_mapping,
                             int num_tokens, int num_kv_heads, int head_dim,
                             int block_size, int64_t num_blocks, int elem_bytes)
{
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        (elem_bytes != 2 && elem_bytes != 4))
        return 1;
    int64_t nslots = num_blocks * block_size;
    unsigned char *seen = calloc((size_t)(nslots > 0 ? nslots : 1), 1);
    if (!seen)
        return 5;
    for (int t = 0; t < num_tokens; ++t) {
        int64_t s = slot_mapping[t];
        if (s < 0)
            continue;
        if (s >= nslots) {
            free(seen);
            return 3;
        }
        if (seen[s]) {
            free(seen);
            return 4;
        }
        seen[s] = 1;
    }
    free(seen);
    size_t row_bytes = (size_t)head_dim * elem_bytes;
    for (int t = 0; t < num_tokens; ++t) {
        int64_t s = slot_mapping[t];
        if (s < 0)
            continue;
        int64_t blk = s / block_size;
        int off = (int)(s % block_size);
        for (int h = 0; h < num_kv_heads; ++h) {
            size_t src = ((size_t)t * num_kv_heads + h) * row_bytes;
            size_t dst = (((size_t)blk * num_kv_heads + h) * block_size + off) * row_bytes;
            memcpy((char *)key_cache + dst, (const char *)key + src, row_bytes);
            memcpy((char *)value_cache + dst, (const char *)value + src, row_bytes);
        }
    }
    return 0;
}

/* ---- block copy: copy-on-write and swap --------------------------------- */

/*
 * Blocks that several sequences share are copied before one of them writes
 * into its own copy ("vLLM Guide: High-Throughput Multi-GPU LLM Serving with
 * PagedAttention", section "What Is PagedAttention?": shared physical blocks
 * with copy-on-write), and under memory pressure the pages of a paused
 * request move to host memory and later back ("Configuring vLLM and
 * PagedAttention for High Throughput Enterprise LLM Serving", section "Quick
 * Answers", the question on KV-cache offloading when VRAM is full).
 *
 * For every pair i, block mapping[2i] of the source pools is copied bit for
 * bit (block_bytes per pool: all kv heads, block_size rows, head_dim) into
 * block mapping[2i + 1] of the destination pools, K and V alike.  Every read
 * happens before any write (the sources are snapshotted).  Errors, with
 * nothing written: a block id outside its pool (2), a destination named twice
 * (4), and, when source and destination are the same pools (in_place), a
 * block that is both a source and a destination (6).
 */
int oracle_copy_blocks(const void *src_key, const void *src_value, void *dst_key,
                       void *dst_value, const int64_t *mapping, int num_pairs,
                       int64_t src_num_blocks, int64_t dst_num_blocks, int64_t block_bytes,
                       int in_place)
{
    if (num_pairs < 0 || block_bytes <= 0 || src_num_blocks < 0 || dst_num_blocks < 0)
        return 1;
    if (num_pairs == 0)
        return 0;
    unsigned char *is_dst = calloc((size_t)(dst_num_blocks > 0 ? dst_num_blocks : 1), 1);
    if (!is_dst)
        return 5;
    for (int i = 0; i < num_pairs; ++i) {
        int64_t s = mapping[2 * i], d = mapping[2 * i + 1];
        if (s < 0 || s >= src_num_blocks || d < 0 || d >= dst_num_blocks) {
            free(is_dst);
            return 2;
        }
        if (is_dst[d]) {
            free(is_dst);
            return 4;
        }
        is_dst[d] = 1;
    }
    if (in_place) {
        for (int i = 0; i < num_pairs; ++i) {
            if (is_dst[mapping[2 * i]]) {
                free(is_dst);
                return 6;
            }
        }
    }
    free(is_dst);
    size_t snap_bytes = (size_t)num_pairs * (size_t)block_bytes;
    char *snap_k = malloc(snap_bytes), *snap_v = malloc(snap_bytes);
    if (!snap_k || !snap_v) {
        free(snap_k);
        free(snap_v);
        return 5;
    }
    for (int i = 0; i < num_pairs; ++i) {
        size_t src = (size_t)mapping[2 * i] * (size_t)block_bytes;
        memcpy(snap_k + (size_t)i * block_bytes, (const char *)src_key + src, (size_t)block_bytes);
        memcpy(snap_v + (size_t)i * block_bytes, (const char *)src_value + src, (size_t)block_bytes);
    }
    for (int i = 0; i < num_pairs; ++i) {
        size_t dst = (size_t)mapping[2 * i + 1] * (size_t)block_bytes;
        memcpy((char *)dst_key + dst, snap_k + (size_t)i * block_bytes, (size_t)block_bytes);
        memcpy((char *)dst_value + dst, snap_v + (size_t)i * block_bytes, (size_t)block_bytes);
    }
    free(snap_k);
    free(snap_v);
    return 0;
}

/* ---- FP8 KV cache: e4m3 codes with a per-tensor scale -------------------- */

/*
 * Quantised KV cache ("vLLM Guide: High-Throughput Multi-GPU LLM Serving with
 * PagedAttention", the pillars section's quantisation support, and the FP8
 * engine example on the same page): every element is stored as an 8-bit
 * floating-point code (OCP e4m3: 1 sign bit, 4 exponent bits with bias 7, 3
 * mantissa bits, no infinities, code S.1111.111 is NaN; largest finite value
 * 448, smallest subnormal 2^-9) of x / scale, with one fp32 scale per pool.
 * Readings (the pages give no rounding rule):
 *   - x / scale is taken in fp32 as x * (1 / scale), both roundings fp32 RNE;
 *   - the code is the nearest e4m3 value, ties to the even code, saturating
 *     at +-448 (infinities included); NaN gives code 0x7F;
 *   - the V pool of the FP8 cache is stored transposed per page,
 *     [block][kv head][head_dim][block_size], the K pool as the bf16 one.
 */
static double e4m3_value(unsigned c)
{
    unsigned s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -v : v;
}

static unsigned e4m3_encode(float y)
{
    if (y != y)
        return 0x7F;
    unsigned sign = signbit(y) ? 0x80u : 0u;
    double a = fabs((double)y);
    if (a > 448.0)
        a = 448.0;
    unsigned best = 0;
    double best_d = INFINITY;
    for (unsigned c = 0; c < 0x7F; ++c) {  /* every finite non-negative code */
        double d = fabs(e4m3_value(c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return sign | best;
}

int oracle_fp8_encode(const float *x, int n, float scale, unsigned char *codes)
{
    if (n < 0 || !(scale > 0.0f))
        return 1;
    float inv = 1.0f / scale;
    for (int i = 0; i < n; ++i)
        codes[i] = (unsigned char)e4m3_encode(x[i] * inv);
    return 0;
}

int oracle_fp8_decode(const unsigned char *codes, int n, double *out)
{
    for (int i = 0; i < n; ++i)
        out[i] = e4m3_value(codes[i]);
    return 0;
}

/*
 * Cache write into FP8 pools: as oracle_reshape_and_cache, with each element
 * encoded as above; K goes to [block][head][offset][d], V to
 * [block][head][d][offset].
 */
int oracle_reshape_and_cache_fp8(const void *key, const void *value, unsigned char *key_cache,
                                 unsigned char *value_cache, const int64_t *slot_mapping,
                                 int num_tokens, int num_kv_heads, int head_dim, int block_size,
                                 int64_t num_blocks, int dtype, float k_scale, float v_scale)
{
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        !(k_scale > 0.0f) || !(v_scale > 0.0f))
        return 1;
    int64_t nslots = num_blocks * block_size;
    unsigned char *seen = calloc((size_t)(nslots > 0 ? nslots : 1), 1);
    if (!seen)
        return 5;
    for (int t = 0; t < num_tokens; ++t) {
        int64_t s = slot_mapping[t];
        if (s < 0)
            continue;
        if (s >= nslots || seen[s]) {
            free(seen);
            return s >= nslots ? 3 : 4;
        }
        seen[s] = 1;
    }
    free(seen);
    float kinv = 1.0f / k_scale, vinv = 1.0f / v_scale;
    for (int t = 0; t < num_tokens; ++t) {
        int64_t s = slot_mapping[t];
        if (s < 0)
            continue;
        int64_t blk = s / block_size;
        int off = (int)(s % block_size);
        for (int h = 0; h < num_kv_heads; ++h) {
            size_t src = ((size_t)t * num_kv_heads + h) * head_dim;
            size_t page = ((size_t)blk * num_kv_heads + h) * (size_t)block_size * head_dim;
            for (int d = 0; d < head_dim; ++d) {
                float k = (float)widen(key, src + d, dtype);
                float v = (float)widen(value, src + d, dtype);
                key_cache[page + (size_t)off * head_dim + d] = (unsigned char)e4m3_encode(k * kinv);
                value_cache[page + (size_t)d * block_size + off] =
                    (unsigned char)e4m3_encode(v * vinv);
            }
        }
    }
    return 0;
}

/*
 * Decode over FP8 pools: every element read is its code's value times the
 * pool's scale (in fp64), then the same attention as oracle_decode.
 */
int oracle_decode_fp8(double *out, const void *query, const unsigned char *key_cache,
                      const unsigned char *value_cache, const int32_t *block_tables,
                      const int32_t *context_lens, int num_seqs, int num_q_heads,
                      int num_kv_heads, int head_dim, int block_size, int max_blocks,
                      int64_t num_blocks, float scale, int q_dtype, float k_scale, float v_scale)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
        head_dim <= 0 || block_size <= 0)
        return 1;
    const int group = num_q_heads / num_kv_heads;
    const int D = head_dim;
    int status = 0;
#pragma omp parallel for schedule(dynamic) reduction(max : status)
    for (int sh = 0; sh < num_seqs * num_q_heads; ++sh) {
        int s = sh / num_q_heads, h = sh % num_q_heads, g = h / group;
        int L = context_lens[s];
        int err = 0;  /* this row's error; folded into status at the end */
        double *o = out + (size_t)sh * D;
        for (int d = 0; d < D; ++d)
            o[d] = 0.0;
        if (L <= 0)
            continue;
        double *K = malloc(sizeof(double) * (size_t)L * D), *V = malloc(sizeof(double) * (size_t)L * D);
        double *q = malloc(sizeof(double) * D), *x = malloc(sizeof(double) * L);
        if (!K || !V || !q || !x) {
            err = 5;
        } else {
            const int32_t *row = block_tables + (size_t)s * max_blocks;
            for (int j = 0; j < L && !err; ++j) {
                int32_t phys = row[j / block_size];
                int off = j % block_size;
                if (phys < 0 || phys >= num_blocks) {
                    err = 2;
                    break;
                }
                size_t page = ((size_t)phys * num_kv_heads + g) * (size_t)block_size * D;
                for (int d = 0; d < D; ++d) {
                    K[(size_t)j * D + d] = e4m3_value(key_cache[page + (size_t)off * D + d]) * (double)k_scale;
                    V[(size_t)j * D + d] = e4m3_value(value_cache[page + (size_t)d * block_size + off]) * (double)v_scale;
                }
            }
            if (!err) {
                for (int d = 0; d < D; ++d)
                    q[d] = widen(query, ((size_t)s * num_q_heads + h) * D + d, q_dtype);
                double m = -INFINITY;
                for (int j = 0; j < L; ++j) {
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d)
                        dot += q[d] * K[(size_t)j * D + d];
                    x[j] = (double)scale * dot;
                    if (x[j] > m)
                        m = x[j];
                }
                double Z = 0.0;
                for (int j = 0; j < L; ++j) {
                    x[j] = exp(x[j] - m);
                    Z += x[j];
                }
                for (int j = 0; j < L; ++j) {
                    double w = x[j] / Z;
                    for (int d = 0; d < D; ++d)
                        o[d] += w * V[(size_t)j * D + d];
                }
            }
        }
        free(K);
        free(V);
        free(q);
        free(x);
        if (err > status)
            status = err;
    }
    return status;
}

/*
 * One query row over FP8 pools: gather the first L keys of a table row, each
 * element its code's value times the pool's scale (K [block][head][offset][d],
 * V [block][head][d][offset]), then the same attention as attend_row.
 */
static int attend_paged_fp8(double *out, const void *q_base, size_t q_off, int q_dtype,
                            const unsigned char *key_cache, const unsigned char *value_cache,
                            const int32_t *bt_row, int L, int num_kv_heads, int kv_head,
                            int block_size, int D, int64_t num_blocks, double scale,
                            double k_scale, double v_scale)
{
    size_t n = (size_t)(L > 0 ? L : 1) * D;
    double *K = malloc(n * sizeof(double));
    double *V = malloc(n * sizeof(double));
    double *x = malloc((size_t)(L > 0 ? L : 1) * sizeof(double));
    double *q = malloc((size_t)D * sizeof(double));
    int st = 0;
    if (!K || !V || !x || !q) {
        st = 5;
        goto done;
    }
    for (int j = 0; j < L; ++j) {
        int32_t phys = bt_row[j / block_size];
        int off = j % block_size;
        if (phys < 0 || phys >= num_blocks) {
            st = 2;
            goto done;
        }
        size_t page = ((size_t)phys * num_kv_heads + kv_head) * (size_t)block_size * D;
        for (int d = 0; d < D; ++d) {
            K[(size_t)j * D + d] = e4m3_value(key_cache[page + (size_t)off * D + d]) * k_scale;
            V[(size_t)j * D + d] = e4m3_value(value_cache[page + (size_t)d * block_size + off]) * v_scale;
        }
    }
    for (int i = 0; i < D; ++i)
        q[i] = widen(q_base, q_off + i, q_dtype);
    attend_row(out, q, K, V, L, D, scale, x, NULL);
done:
    free(K);
    free(V);
    free(x);
    free(q);
    return st;
}

/*
 * Prefill chunks over FP8 pools: as oracle_prefill (query i of chunk c at
 * position context_lens[c] - n_c + i sees keys 0 .. that position), with the
 * keys and values decoded as in oracle_decode_fp8.
 */
int oracle_prefill_fp8(double *out, const void *query, const unsigned char *key_cache,
                       const unsigned char *value_cache, const int32_t *block_tables,
                       const int32_t *cu_query_lens, const int32_t *context_lens, int num_chunks,
                       int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                       int max_blocks, int64_t num_blocks, float scale, int q_dtype,
                       float k_scale, float v_scale)
{
    if (num_chunks < 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
        return 1;
    for (int c = 0; c < num_chunks; ++c) {
        int n = cu_query_lens[c + 1] - cu_query_lens[c];
        if (n < 0 || n > context_lens[c] || context_lens[c] > max_blocks * block_size)
            return 1;
    }
    int group = num_q_heads / num_kv_heads;
    int total = cu_query_lens[num_chunks];
    int status = 0;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int t = 0; t < total; ++t) {
        for (int h = 0; h < num_q_heads; ++h) {
            int c = 0;
            while (cu_query_lens[c + 1] <= t)
                ++c;
            int n = cu_query_lens[c + 1] - cu_query_lens[c];
            int i = t - cu_query_lens[c];
            int pos = context_lens[c] - n + i;
            size_t row = (size_t)t * num_q_heads + h;
            int st = attend_paged_fp8(out + row * head_dim, query, row * head_dim, q_dtype,
                                      key_cache, value_cache, block_tables + (size_t)c * max_blocks,
                                      pos + 1, num_kv_heads, h / group, block_size, head_dim,
                                      num_blocks, (double)scale, (double)k_scale,
                                      (double)v_scale);
            if (st) {
#pragma omp atomic write
                status = st;
            }
        }
    }
    return status;
}
