// Decode attention over a paged KV cache on gfx950.
//
// One new query token per sequence attends to all of its cached keys and
// values.  Key j of a sequence lives in physical block BlockTable[j / B] at
// offset j mod B, and the weights are exp(q.k_j * scale) normalised over all
// keys ("Configuring vLLM and PagedAttention for High Throughput Enterprise
// LLM Serving", section "Architectural Foundations: PagedAttention & Virtual
// Memory").  Decode must stream every cached K and V row from HBM once per
// step and does little arithmetic per byte, so it is bound by memory
// bandwidth (same page, section "Memory Bottlenecks in Autoregressive LLM
// Inference"); the design below is therefore about feeding HBM, not about the
// matrix cores.
//
// Work split (split-K).  A workgroup of NW waves owns one (sequence, kv head,
// partition of P tokens).  All G = Hq / Hkv query heads of the kv head are
// served by the same pass over K and V (grouped-query attention), so each K/V
// byte is read once per kv head.  Inside the workgroup the partition is cut
// into units of 16 tokens (a whole block for B = 16, half a block for B = 32)
// handed round-robin to the waves.
//
// Lane mapping inside a unit.  A token row is D * sizeof(T) bytes = NCH
// chunks of 16 bytes.  LPT lanes share a row, each holding CPL chunks
// (chunk r + LPT * k for lane r of the group), so one 16-byte load per lane
// covers TPP = 64 / LPT whole rows and every row segment an instruction
// touches is LPT * 16 contiguous bytes (a full 128-byte line for LPT = 8).
// The q.k partial sums are combined across the LPT lanes with DPP row
// operations, never through LDS.
//
// Softmax.  Online softmax (Milakov & Gimelshein, "Online normalizer
// calculation for softmax", 2018) in base 2 (scale * log2 e is folded into
// one multiply).  Each wave keeps one reference maximum per head, identical
// in all its lanes; it is raised only when a new logit exceeds it by more
// than kRescaleThreshold (log2 units), so the rescale of the accumulators is
// rare.  Any reference value gives the same result in exact arithmetic; the
// bound keeps every weight <= 2^8.
//
// Partials.  The waves' (max, sum, unnormalised output) are merged in LDS.  A
// sequence with one partition is finished there; otherwise each partition's
// partials go to the workspace and decode_reduce_kernel merges them with the
// usual log-sum-exp rescaling.
#include <type_traits>

#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

constexpr float kRescaleThreshold = 8.0f;
constexpr int kUnitTokens = 16;
constexpr int kDecodeWaves = 4;

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a),
                                           __builtin_bit_cast(bf16x2_v, b), c, false);
}

// q . k over one 16-byte chunk, accumulated into acc.
template <typename T>
__device__ __forceinline__ float chunk_dot(const uint4 &q, const uint4 &k, float acc) {
    if constexpr (std::is_same<T, bf16_t>::value) {
        acc = dot2_bf16(q.x, k.x, acc);
        acc = dot2_bf16(q.y, k.y, acc);
        acc = dot2_bf16(q.z, k.z, acc);
        acc = dot2_bf16(q.w, k.w, acc);
    } else {
        acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
        acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
        acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
        acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
    }
    return acc;
}

// Widen the elements of a 16-byte chunk to fp32.
template <typename T>
__device__ __forceinline__ void chunk_widen(const uint4 &c, float *v) {
    if constexpr (std::is_same<T, bf16_t>::value) {
        v[0] = bf16_lo(c.x); v[1] = bf16_hi(c.x);
        v[2] = bf16_lo(c.y); v[3] = bf16_hi(c.y);
        v[4] = bf16_lo(c.z); v[5] = bf16_hi(c.z);
        v[6] = bf16_lo(c.w); v[7] = bf16_hi(c.w);
    } else {
        v[0] = __uint_as_float(c.x); v[1] = __uint_as_float(c.y);
        v[2] = __uint_as_float(c.z); v[3] = __uint_as_float(c.w);
    }
}

template <typename T, int D, int G>
struct DecodeShape {
    static constexpr int EB = sizeof(T);
    static constexpr int ROWB = D * EB;                 // bytes of a token row
    static constexpr int NCH = ROWB / 16;               // 16-byte chunks per row
    static constexpr int LPT = (NCH == 8) ? 8 : (NCH == 32 ? 16 : (G <= 4 ? 8 : 16));
    static constexpr int CPL = NCH / LPT;               // chunks per lane
    static constexpr int TPP = 64 / LPT;                // rows per load instruction
    static constexpr int NPASS = kUnitTokens / TPP;     // loads per unit, per tensor
    static constexpr int EPC = 16 / EB;                 // elements per chunk
    static constexpr int OPL = CPL * EPC;               // output elements per lane per head
    static_assert(NCH % LPT == 0 && kUnitTokens % TPP == 0, "shape");
};

template <typename T, int D, int G>
struct UnitRegs {
    using S = DecodeShape<T, D, G>;
    uint4 k[S::NPASS][S::CPL];
    uint4 v[S::NPASS][S::CPL];
};

template <typename T, int D, int B, int G, int NW>
__global__ __launch_bounds__(NW * 64) void decode_partition_kernel(
    T *__restrict__ out, const T *__restrict__ query, const T *__restrict__ key_cache,
    const T *__restrict__ value_cache, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, int num_q_heads, int num_kv_heads,
    int max_blocks, int max_tokens, int64_t num_blocks, int P, int np_max, float scale_log2,
    float *__restrict__ ws_o, float *__restrict__ ws_ml) {
    using S = DecodeShape<T, D, G>;
    constexpr int LPT = S::LPT, CPL = S::CPL, TPP = S::TPP, NPASS = S::NPASS, EPC = S::EPC,
                  OPL = S::OPL, ROWB = S::ROWB;
    constexpr float NEG_INF = -__builtin_inff();

    const int p = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
    // max_tokens = min(max_blocks * B, np_max * P): lengths beyond what the
    // table or the launch covers are clamped, so no access leaves the buffers.
    int L = context_lens[s];
    L = L < 0 ? 0 : (L > max_tokens ? max_tokens : L);
    const int np = cdiv(L, P);
    if (p >= np) return;  // whole workgroup: this partition is empty
    const int tok0 = p * P;
    const int tok1 = min(L, tok0 + P);
    const int nunits = cdiv(tok1 - tok0, kUnitTokens);
    const int u_first = tok0 / kUnitTokens;

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int tg = lane / LPT, r = lane % LPT;

    // Query chunks of the G heads of this kv head (raw, reused for every key).
    uint4 qr[G][CPL];
    const char *qbase = (const char *)query + ((int64_t)s * num_q_heads + (int64_t)g * G) * ROWB;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int k = 0; k < CPL; ++k)
            qr[h][k] = *(const uint4 *)(qbase + h * ROWB + (r + LPT * k) * 16);

    float o[G][OPL];
    float l[G], m[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        l[h] = 0.f;
        m[h] = NEG_INF;
#pragma unroll
        for (int i = 0; i < OPL; ++i) o[h][i] = 0.f;
    }

    const int32_t *bt = block_tables + (int64_t)s * max_blocks;
    const char *kbase = (const char *)key_cache;
    const char *vbase = (const char *)value_cache;
    const int64_t head_bytes = (int64_t)B * ROWB;
    const int64_t block_bytes = head_bytes * num_kv_heads;
    const int lane_off = tg * ROWB + r * 16;

    // Byte offset of unit u (relative to the pool) and its count of valid rows.
    auto locate = [&](int u, int &nvalid) -> int64_t {
        const int tok = (u_first + u) * kUnitTokens;
        int phys = uniform(bt[tok / B]);
        nvalid = min(kUnitTokens, tok1 - tok);
        if (phys < 0 || (int64_t)phys >= num_blocks) {
            phys = 0;  // caller error: read a valid block, count no token
            nvalid = 0;
        }
        return (int64_t)phys * block_bytes + (int64_t)g * head_bytes + (tok % B) * ROWB + lane_off;
    };
    auto load = [&](UnitRegs<T, D, G> &R, int64_t off) {
#pragma unroll
        for (int pp = 0; pp < NPASS; ++pp)
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const int64_t a = off + pp * TPP * ROWB + LPT * k * 16;
                R.k[pp][k] = *(const uint4 *)(kbase + a);
                R.v[pp][k] = *(const uint4 *)(vbase + a);
            }
    };
    auto process = [&](UnitRegs<T, D, G> &R, int nvalid) {
        float sc[NPASS][G];
#pragma unroll
        for (int pp = 0; pp < NPASS; ++pp)
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float a = 0.f;
#pragma unroll
                for (int k = 0; k < CPL; ++k) a = chunk_dot<T>(qr[h][k], R.k[pp][k], a);
                sc[pp][h] = group_sum<LPT>(a) * scale_log2;
            }
        if (nvalid < kUnitTokens) {
            // Rows past the end of the context: weight exactly 0 and value
            // zeroed (their slots may hold anything, NaN included).
#pragma unroll
            for (int pp = 0; pp < NPASS; ++pp) {
                const bool ok = pp * TPP + tg < nvalid;
#pragma unroll
                for (int h = 0; h < G; ++h) sc[pp][h] = ok ? sc[pp][h] : NEG_INF;
#pragma unroll
                for (int k = 0; k < CPL; ++k)
                    if (!ok) R.v[pp][k] = make_uint4(0, 0, 0, 0);
            }
        }
        float lmax[G];
        bool need = false;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float x = sc[0][h];
#pragma unroll
            for (int pp = 1; pp < NPASS; ++pp) x = fmaxf(x, sc[pp][h]);
            lmax[h] = x;
            need |= x > m[h] + kRescaleThreshold;
        }
        if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float mn = fmaxf(m[h], wave_max(lmax[h]));
                const float alpha = (m[h] == NEG_INF) ? 0.f : fast_exp2(m[h] - mn);
                m[h] = mn;
                l[h] *= alpha;
#pragma unroll
                for (int i = 0; i < OPL; ++i) o[h][i] *= alpha;
            }
        }
#pragma unroll
        for (int pp = 0; pp < NPASS; ++pp) {
            float pr[G];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                pr[h] = fast_exp2(sc[pp][h] - m[h]);
                l[h] += pr[h];
            }
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                float v[EPC];
                chunk_widen<T>(R.v[pp][k], v);
#pragma unroll
                for (int h = 0; h < G; ++h)
#pragma unroll
                    for (int e = 0; e < EPC; ++e) o[h][k * EPC + e] = fmaf(pr[h], v[e], o[h][k * EPC + e]);
            }
        }
    };

    // Two register buffers: the loads of the next unit are in flight while
    // the current one is processed.
    UnitRegs<T, D, G> ra, rb;
    int na = 0, nb = 0;
    int u = w;
    if (u < nunits) load(ra, locate(u, na));
    for (; u < nunits; u += 2 * NW) {
        if (u + NW < nunits) load(rb, locate(u + NW, nb));
        if (na > 0) process(ra, na);
        if (u + NW >= nunits) break;
        if (u + 2 * NW < nunits) load(ra, locate(u + 2 * NW, na));
        if (nb > 0) process(rb, nb);
    }

    // ---- merge the waves (and the token groups inside each wave) ----------
    // Rows of 16 lanes that still hold separate token groups; with a large
    // G * D two of them are folded first so the LDS buffer stays <= 32 KB.
    constexpr int RS = (G * D > 512) ? 2 : 4;
    __shared__ float red_o[NW][RS][G * D];
    __shared__ float red_l[NW][RS][G];
    __shared__ float red_m[NW][G];
    if (LPT == 8) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            l[h] += dpp<DPP_ROR8>(l[h]);
#pragma unroll
            for (int i = 0; i < OPL; ++i) o[h][i] += dpp<DPP_ROR8>(o[h][i]);
        }
    }
    if (RS == 2) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            l[h] += __shfl_xor(l[h], 16);
#pragma unroll
            for (int i = 0; i < OPL; ++i) o[h][i] += __shfl_xor(o[h][i], 16);
        }
    }
    const int slot = (RS == 2) ? (lane >> 5) : (lane >> 4);
    const bool row_writer = (RS == 4) || ((lane & 16) == 0);
    if (row_writer && (LPT == 16 || (lane & 8) == 0)) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int k = 0; k < CPL; ++k)
#pragma unroll
                for (int e = 0; e < EPC; ++e)
                    red_o[w][slot][h * D + (r + LPT * k) * EPC + e] = o[h][k * EPC + e];
    }
    if (row_writer && (lane & 15) == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) red_l[w][slot][h] = l[h];
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) red_m[w][h] = m[h];
    }
    __syncthreads();

    for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
        const int h = idx / D, d = idx - h * D;
        float M = NEG_INF;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, red_m[ww][h]);
        float acc = 0.f, lsum = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const float mw = red_m[ww][h];
            const float f = (mw == NEG_INF) ? 0.f : fast_exp2(mw - M);
            float so = 0.f, sl = 0.f;
#pragma unroll
            for (int rr = 0; rr < RS; ++rr) {
                so += red_o[ww][rr][idx];
                sl += red_l[ww][rr][h];
            }
            acc = fmaf(f, so, acc);
            lsum = fmaf(f, sl, lsum);
        }
        const int64_t qrow = (int64_t)s * num_q_heads + (int64_t)g * G + h;
        if (np == 1) {
            Elem<T>::store(out + qrow * D + d, lsum > 0.f ? acc / lsum : 0.f);
        } else {
            ws_o[(qrow * np_max + p) * D + d] = acc;
            if (d == 0) {
                ws_ml[(qrow * np_max + p) * 2 + 0] = M;
                ws_ml[(qrow * np_max + p) * 2 + 1] = lsum;
            }
        }
    }
}

// Merge the partitions of each (sequence, q head): with M = max_p m_p,
// out = sum_p o_p 2^(m_p - M) / sum_p l_p 2^(m_p - M).  One thread per output
// element; sequences with a single partition were finished by the partition
// kernel, empty ones get zeros.
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(
    T *__restrict__ out, const int32_t *__restrict__ context_lens, int num_q_heads,
    int max_tokens, int P, int np_max, const float *__restrict__ ws_o,
    const float *__restrict__ ws_ml) {
    constexpr float NEG_INF = -__builtin_inff();
    const int64_t qrow = blockIdx.x;
    const int s = (int)(qrow / num_q_heads);
    const int d = threadIdx.x;
    int L = context_lens[s];
    L = L < 0 ? 0 : (L > max_tokens ? max_tokens : L);
    const int np = cdiv(L, P);
    if (np == 1) return;
    if (np == 0) {
        Elem<T>::store(out + qrow * D + d, 0.f);
        return;
    }
    const float *ml = ws_ml + qrow * np_max * 2;
    float M = NEG_INF;
    for (int p = 0; p < np; ++p) M = fmaxf(M, ml[2 * p]);
    float acc = 0.f, lsum = 0.f;
    for (int p = 0; p < np; ++p) {
        const float mp = ml[2 * p];
        const float f = (mp == NEG_INF) ? 0.f : fast_exp2(mp - M);
        lsum = fmaf(f, ml[2 * p + 1], lsum);
        acc = fmaf(f, ws_o[(qrow * np_max + p) * D + d], acc);
    }
    Elem<T>::store(out + qrow * D + d, lsum > 0.f ? acc / lsum : 0.f);
}

// ---- dispatch ---------------------------------------------------------------

// Tokens of a sequence that the launch covers: the table's capacity and the
// partitions in the grid.  Both kernels clamp context lengths to it.
static int max_tokens(const DecodeArgs &a) {
    const int64_t by_table = (int64_t)a.max_blocks_per_seq * a.block_size;
    const int64_t by_grid = (int64_t)a.num_partitions * a.partition_size;
    return (int)(by_table < by_grid ? by_table : by_grid);
}

template <typename T, int D, int B, int G>
static hipError_t launch_part(const DecodeArgs &a, hipStream_t stream) {
    dim3 grid(a.num_partitions, a.num_kv_heads, a.num_seqs);
    hipLaunchKernelGGL((decode_partition_kernel<T, D, B, G, kDecodeWaves>), grid,
                       dim3(kDecodeWaves * 64), 0, stream, (T *)a.out, (const T *)a.query,
                       (const T *)a.key_cache, (const T *)a.value_cache, a.block_tables,
                       a.context_lens, a.num_q_heads, a.num_kv_heads, a.max_blocks_per_seq,
                       max_tokens(a), a.num_blocks, a.partition_size, a.num_partitions,
                       a.scale * kLog2e, a.ws_o, a.ws_ml);
    return hipGetLastError();
}

template <typename T, int D, int B>
static hipError_t by_group(const DecodeArgs &a, hipStream_t stream) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_part<T, D, B, 1>(a, stream);
        case 2: return launch_part<T, D, B, 2>(a, stream);
        case 4: return launch_part<T, D, B, 4>(a, stream);
        case 8: return launch_part<T, D, B, 8>(a, stream);
    }
    return hipErrorNotSupported;
}

template <typename T, int D>
static hipError_t by_block(const DecodeArgs &a, hipStream_t stream) {
    switch (a.block_size) {
        case 16: return by_group<T, D, 16>(a, stream);
        case 32: return by_group<T, D, 32>(a, stream);
    }
    return hipErrorNotSupported;
}

template <typename T>
static hipError_t by_dim(const DecodeArgs &a, hipStream_t stream) {
    switch (a.head_dim) {
        case 64: return by_block<T, 64>(a, stream);
        case 128: return by_block<T, 128>(a, stream);
    }
    return hipErrorNotSupported;
}

bool decode_shape_supported(int dtype, int head_dim, int block_size, int group) {
    return (dtype == 0 || dtype == 1) && (head_dim == 64 || head_dim == 128) &&
           (block_size == 16 || block_size == 32) &&
           (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_decode_partitions(const DecodeArgs &a, hipStream_t stream) {
    if (a.num_seqs == 0 || a.num_partitions == 0) return hipSuccess;
    return a.dtype == 1 ? by_dim<bf16_t>(a, stream) : by_dim<float>(a, stream);
}

template <typename T, int D>
static hipError_t launch_red(const DecodeArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((decode_reduce_kernel<T, D>),
                       dim3((unsigned)((int64_t)a.num_seqs * a.num_q_heads)), dim3(D), 0, stream,
                       (T *)a.out, a.context_lens, a.num_q_heads, max_tokens(a), a.partition_size,
                       a.num_partitions, a.ws_o, a.ws_ml);
    return hipGetLastError();
}

hipError_t launch_decode_reduce(const DecodeArgs &a, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    if (a.dtype == 1)
        return a.head_dim == 64 ? launch_red<bf16_t, 64>(a, stream)
                                : launch_red<bf16_t, 128>(a, stream);
    return a.head_dim == 64 ? launch_red<float, 64>(a, stream) : launch_red<float, 128>(a, stream);
}

}  // namespace pa
