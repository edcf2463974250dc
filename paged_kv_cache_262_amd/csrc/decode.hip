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
// Inference"); the design below is about feeding HBM, not about the matrix
// cores.
//
// Unit of work.  The keys of one (sequence, kv head) are cut into units of 16
// tokens (a whole block for B = 16, half a block for B = 32).  A wave streams
// units and serves all G = Hq / Hkv query heads of the kv head from the same
// pass (grouped-query attention), so each K/V byte is read once.
//
// Lane mapping inside a unit.  A token row is D * sizeof(T) bytes = NCH
// chunks of 16 bytes.  LPT lanes share a row, each holding CPL chunks (chunk
// r + LPT * k for lane r of the group), so one 16-byte load per lane covers
// TPP = 64 / LPT whole rows and every row segment a load touches is LPT * 16
// contiguous bytes (a full 128-byte line for LPT = 8).  q.k partial sums are
// combined across the LPT lanes with DPP row operations.
//
// Softmax.  Online softmax (Milakov & Gimelshein, "Online normalizer
// calculation for softmax", 2018) in base 2, with scale * log2 e folded into
// one multiply.  A wave keeps one reference maximum per head, the same in all
// its lanes, and raises it only when a logit exceeds it by more than
// kRescaleThreshold (log2 units), so rescaling the accumulators is rare.  Any
// reference gives the same result in exact arithmetic; the bound keeps every
// weight <= 2^8.
//
// Split of the work (split-K over the context).  Two kernels produce partial
// results (running max, sum, unnormalised output) that a reduce kernel merges
// with log-sum-exp rescaling:
//   - decode_stream_kernel (the default): all units of all (sequence, kv head)
//     pairs form one sequence; every wave takes an equal contiguous range of
//     it, crossing pair boundaries as needed, and emits one partial record per
//     pair it touches.  The load is balanced whatever the mix of context
//     lengths, waves never synchronise, and a pair that falls inside one wave
//     is finished by that wave.
//   - decode_stream_mma_kernel: the same split for bf16 with both products
//     on the matrix cores (see its comment); the default for bf16.
//   - decode_partition_kernel (an explicit partition size): one workgroup per
//     (sequence, kv head, partition of P tokens), waves merged in LDS.
#include <type_traits>

#include "pa_common.h"
#include "pa_internal.h"
#include "pa_prefix.h"

namespace pa {

constexpr float kRescaleThreshold = 8.0f;
constexpr int kUnitTokens = 16;
constexpr int kDecodeWaves = 4;
#ifndef PA_WIDE_GROUP
#define PA_WIDE_GROUP 8
#endif
#ifndef PA_BUFFER_BUDGET
#define PA_BUFFER_BUDGET 256
#endif
constexpr int kWideGroup = PA_WIDE_GROUP;       // groups >= this use 16 lanes per row
constexpr int kBufferBudget = PA_BUFFER_BUDGET;  // VGPRs for q, accumulators and buffers
constexpr float NEG_INF = -__builtin_inff();

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // native vector: no memcpy

// fp32 pair -> bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef float floatx2_t __attribute__((ext_vector_type(2)));
    const floatx2_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_v));
}

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
    // 16 lanes per row halve the per-lane q and output registers for the
    // larger groups, which buys one more unit in flight.
    static constexpr int LPT = (NCH == 8) ? 8 : (NCH == 32 ? 16 : (G < kWideGroup ? 8 : 16));
    static constexpr int CPL = NCH / LPT;               // chunks per lane
    static constexpr int TPP = 64 / LPT;                // rows per load instruction
    static constexpr int NPASS = kUnitTokens / TPP;     // loads per unit, per tensor
    static constexpr int EPC = 16 / EB;                 // elements per chunk
    static constexpr int OPL = CPL * EPC;               // output elements per lane per head
    static constexpr int UNIT_BYTES = kUnitTokens * ROWB;
    // Units in flight + 1: as many register buffers as fit next to q, the
    // accumulators and temporaries in the 256 VGPRs of 2 waves per SIMD.
    static constexpr int BUF_REGS = NPASS * CPL * 8;
    static constexpr int FIXED_REGS = G * CPL * 4 + G * OPL + NPASS * G + 40;
    static constexpr int NBUF_FIT = (kBufferBudget - FIXED_REGS) / BUF_REGS;
    static constexpr int NBUF = NBUF_FIT < 2 ? 2 : (NBUF_FIT > 4 ? 4 : NBUF_FIT);
    static_assert(NCH % LPT == 0 && kUnitTokens % TPP == 0, "shape");
};

template <typename T, int D, int G>
struct UnitRegs {
    using S = DecodeShape<T, D, G>;
    uint4 k[S::NPASS][S::CPL];
    uint4 v[S::NPASS][S::CPL];
};

// Cache policy of the buffer loads that stream K and V from the pools (the
// cache-policy operand of the load builtins; bit 1 is gfx950's nt bit).  A
// decode launch reads most of the cache once, so those loads are
// non-temporal: their lines are not kept for reuse in L2 and the last-level
// cache.  Against the default policy this shortened the 8B decode step from
// 113.4 to 98.6 us and the 32K one from 187.6 to 170.0 us; K alone or V alone
// non-temporal gave about a third of that each.  Bytes that other waves read
// again keep the default policy: blocks shared with a neighbouring sequence
// (below; the plain decode of 128 sequences over one 1,024-token prefix took
// 175 us with every load non-temporal, 140 us with this rule), the
// shared-prefix pass, whose blocks every tile of the batch reads, and the
// FP8 pages of 32-token blocks, whose 32-byte V rows the two units of a
// block read half each.  The policy is an immediate of the load, so the
// kernels split their unit runs where it changes and run one copy of the
// load pipeline per policy (a branch per load made the compiler wait for
// each load at the join).
constexpr int kOnce = 2;   // read once: non-temporal
constexpr int kReuse = 0;  // read again soon: default policy

// Whether physical block phys, at column col of sequence s's table, is also
// at that column of the previous or the next sequence's table.  Sequences
// that share blocks (a common prompt, forked samples) hold them at the same
// positions of their tables and usually sit next to each other in a batch,
// so their waves read those blocks again and the loads keep the default
// policy.  Table entries past a neighbour's length are compared as they are:
// a false match only changes the cache policy.
__device__ __forceinline__ bool shared_with_neighbour(const int32_t *__restrict__ block_tables,
                                                      int S, int max_blocks, int s, int col,
                                                      int phys) {
    const int32_t *row = block_tables + (int64_t)s * max_blocks + col;
    const int prev = s > 0 ? row[-max_blocks] : -1;
    const int next = s + 1 < S ? row[max_blocks] : -1;
    return prev == phys || next == phys;
}

// Buffer resources of one unit in the K and V pools: base = the unit's first
// byte, range = the unit, or an empty range when there is nothing to read
// (then every load returns zeros without touching memory).  Loads are thus
// issued unconditionally, which keeps the count of loads in flight identical
// on every path and lets the compiler wait for exactly the unit it processes.
struct UnitRes {
    __amdgpu_buffer_rsrc_t k, v;
};

__device__ __forceinline__ UnitRes unit_res(const char *kbase, const char *vbase, int64_t off,
                                            int range) {
    return UnitRes{__builtin_amdgcn_make_buffer_rsrc((void *)(kbase + off), (short)0, range,
                                                     0x00020000),
                   __builtin_amdgcn_make_buffer_rsrc((void *)(vbase + off), (short)0, range,
                                                     0x00020000)};
}

template <int POL, typename T, int D, int G>
__device__ __forceinline__ void load_unit(UnitRegs<T, D, G> &R, const UnitRes &res, int lane_off) {
    using S = DecodeShape<T, D, G>;
#pragma unroll
    for (int pp = 0; pp < S::NPASS; ++pp)
#pragma unroll
        for (int k = 0; k < S::CPL; ++k) {
            const int a = lane_off + pp * S::TPP * S::ROWB + S::LPT * k * 16;
            R.k[pp][k] =
                __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(res.k, a, 0, POL));
            R.v[pp][k] =
                __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(res.v, a, 0, POL));
        }
}

// Online-softmax state of one wave for one (sequence, kv head): the G query
// heads, their running maxima (wave-uniform), and per-lane partial sums and
// outputs over the rows this lane's token group has seen.
template <typename T, int D, int G>
struct WaveAcc {
    using S = DecodeShape<T, D, G>;
    uint4 q[G][S::CPL];
    float o[G][S::OPL];
    float l[G], m[G];

    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            l[h] = 0.f;
            m[h] = NEG_INF;
#pragma unroll
            for (int i = 0; i < S::OPL; ++i) o[h][i] = 0.f;
        }
    }

    // q rows of the G heads: qrow points at head 0 of the group.
    __device__ __forceinline__ void load_q(const char *qrow, int r) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int k = 0; k < S::CPL; ++k)
                q[h][k] = *(const uint4 *)(qrow + h * S::ROWB + (r + S::LPT * k) * 16);
    }

    __device__ __forceinline__ void process(UnitRegs<T, D, G> &R, int nvalid, float scale_log2,
                                            int tg) {
        constexpr int NPASS = S::NPASS, CPL = S::CPL, EPC = S::EPC, TPP = S::TPP;
        float sc[NPASS][G];
#pragma unroll
        for (int pp = 0; pp < NPASS; ++pp)
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float a = 0.f;
#pragma unroll
                for (int k = 0; k < CPL; ++k) a = chunk_dot<T>(q[h][k], R.k[pp][k], a);
                sc[pp][h] = group_sum<S::LPT>(a) * scale_log2;
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
                for (int i = 0; i < S::OPL; ++i) o[h][i] *= alpha;
            }
        }
        if constexpr (std::is_same<T, bf16_t>::value) {
            // bf16: the two passes pp, pp + 1 a lane holds are two tokens.
            // Their weights are rounded to a bf16 pair (as the matrix-core
            // prefill does) and the matching V elements of both tokens are
            // packed into pairs, so one dot2 per head and element pair does
            // the work of two FMAs.  The row sums use the same rounded
            // weights, so numerator and denominator agree.
            static_assert(NPASS % 2 == 0, "token pairs");
#pragma unroll
            for (int pp = 0; pp < NPASS; pp += 2) {
                uint32_t pk[G];
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    pk[h] = pack_bf16x2(fast_exp2(sc[pp][h] - m[h]),
                                        fast_exp2(sc[pp + 1][h] - m[h]));
                    l[h] = dot2_bf16(pk[h], 0x3F803F80u, l[h]);  // + both rounded weights
                }
#pragma unroll
                for (int k = 0; k < CPL; ++k) {
                    const uint32_t a[4] = {R.v[pp][k].x, R.v[pp][k].y, R.v[pp][k].z,
                                           R.v[pp][k].w};
                    const uint32_t b[4] = {R.v[pp + 1][k].x, R.v[pp + 1][k].y, R.v[pp + 1][k].z,
                                           R.v[pp + 1][k].w};
#pragma unroll
                    for (int w2 = 0; w2 < 4; ++w2) {
                        const uint32_t lo = __builtin_amdgcn_perm(b[w2], a[w2], 0x05040100u);
                        const uint32_t hi = __builtin_amdgcn_perm(b[w2], a[w2], 0x07060302u);
#pragma unroll
                        for (int h = 0; h < G; ++h) {
                            float &o0 = o[h][k * EPC + 2 * w2];
                            float &o1 = o[h][k * EPC + 2 * w2 + 1];
                            o0 = dot2_bf16(pk[h], lo, o0);
                            o1 = dot2_bf16(pk[h], hi, o1);
                        }
                    }
                }
            }
        } else {
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
                        for (int e = 0; e < EPC; ++e)
                            o[h][k * EPC + e] = fmaf(pr[h], v[e], o[h][k * EPC + e]);
                }
            }
        }
    }

    // Sum l and o over the wave's token groups; afterwards every lane holds
    // the totals for the dims of its chunks.
    __device__ __forceinline__ void reduce_groups() {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            if (S::LPT == 8) {
                l[h] += dpp<DPP_ROR8>(l[h]);
#pragma unroll
                for (int i = 0; i < S::OPL; ++i) o[h][i] += dpp<DPP_ROR8>(o[h][i]);
            }
            l[h] += __shfl_xor(l[h], 16);
            l[h] += __shfl_xor(l[h], 32);
#pragma unroll
            for (int i = 0; i < S::OPL; ++i) {
                o[h][i] += __shfl_xor(o[h][i], 16);
                o[h][i] += __shfl_xor(o[h][i], 32);
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Balanced split: every wave streams an equal share of all units.
// ---------------------------------------------------------------------------

// Context length as the kernels use it: clamped to what the table holds.
__device__ __forceinline__ int clamp_len(int L, int max_tokens) {
    return L < 0 ? 0 : (L > max_tokens ? max_tokens : L);
}

// Tokens of a length-L sequence past its first skip (none when L <= skip).
__device__ __forceinline__ int past_skip(int L, int skip) { return L > skip ? L - skip : 0; }

// Wave (of nw <= U) whose range [U*w/nw, U*(w+1)/nw) contains unit u < U.
__device__ __forceinline__ int wave_of_unit(int64_t u, int64_t U, int nw) {
    return (int)(((u + 1) * nw - 1) / U);
}

// Exclusive scan of the per-sequence unit counts into scan[0..S], by a
// workgroup of NW waves.  scan[S] is the total per kv head.  Sequence s counts
// context_lens[s] - len_skip tokens (its tokens past the first len_skip).
// The unit range [ua, ub) of wave gw: an equal share of the batch's U units
// over nw waves (the balanced split), or with nw == 0 the units of pair gw
// (one wave per sequence and kv head; the range is empty for an empty pair).
// False: the wave has nothing to do.
__device__ __forceinline__ bool wave_range(const int *scan, int S, int Hkv, int64_t U, int nw,
                                           int gw, int64_t &ua, int64_t &ub) {
    if (nw == 0) {
        if (gw >= S * Hkv) return false;
        const int s = gw / Hkv, g = gw - s * Hkv;
        const int us = scan[s + 1] - scan[s];
        ua = (int64_t)scan[s] * Hkv + (int64_t)g * us;
        ub = ua + us;
        return true;
    }
    // With fewer units than waves only the first U waves work, so that every
    // working wave owns at least one unit (the reduce relies on it).
    const int nwe = (int)min((int64_t)nw, U);
    if (gw >= nwe) return false;
    ua = U * gw / nwe;
    ub = U * (gw + 1) / nwe;
    return true;
}

// One wave per pair: the G output rows of an empty pair (a sequence of
// length 0) are zero, as the reduce writes them in the balanced split.
template <typename T, int D>
__device__ __forceinline__ void zero_pair_rows(T *out, int gw, int Hkv, int num_q_heads, int G,
                                               int lane) {
    const int s = gw / Hkv, g = gw - s * Hkv;
    T *dst = out + ((int64_t)s * num_q_heads + (int64_t)g * G) * D;
    for (int i = lane; i < G * D; i += 64) Elem<T>::store(dst + i, 0.f);
}

template <int NW>
__device__ void scan_units(int *scan, const int32_t *__restrict__ context_lens, int S,
                           int max_tokens, int len_skip = 0) {
    __shared__ int wave_sums[NW];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int per = cdiv(S, NW * 64);
    const int lo = min(S, t * per), hi = min(S, lo + per);
    int sum = 0;
    for (int s = lo; s < hi; ++s)
        sum += cdiv(clamp_len(past_skip(context_lens[s], len_skip), max_tokens), kUnitTokens);
    int incl = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d);
        if (lane >= d) incl += y;
    }
    if (lane == 63) wave_sums[w] = incl;
    __syncthreads();
    int run = incl - sum, total = 0;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
        run += (ww < w) ? wave_sums[ww] : 0;
        total += wave_sums[ww];
    }
    for (int s = lo; s < hi; ++s) {
        scan[s] = run;
        run += cdiv(clamp_len(past_skip(context_lens[s], len_skip), max_tokens), kUnitTokens);
    }
    if (t == 0) scan[S] = total;
    __syncthreads();
}

// Largest s with scan[s] * Hkv <= u (u inside the flattened range).
__device__ __forceinline__ int seq_of_unit(const int *scan, int S, int64_t u, int Hkv) {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)scan[mid] * Hkv <= u) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// AP (append): the step's new token of sequence s (rows new_key[s],
// new_value[s], [S][Hkv][D]) sits at position L_s - 1.  The wave that streams
// the unit holding that position writes the rows into their slot before it
// loads the unit, so the write needs no ordering with any other wave: no other
// wave reads that unit.
template <typename T, int D, int B, int G, int NW, bool AP>
__global__ __launch_bounds__(NW * 64) void decode_stream_kernel(
    T *__restrict__ out, const T *__restrict__ query, T *__restrict__ key_cache,
    T *__restrict__ value_cache, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, int S, int num_q_heads, int num_kv_heads,
    int max_blocks, int max_tokens, int64_t num_blocks, int nw, float scale_log2,
    float *__restrict__ rec_o, float *__restrict__ rec_ml, int *__restrict__ ws_scan,
    const T *__restrict__ new_key, const T *__restrict__ new_value) {
    using SH = DecodeShape<T, D, G>;
    constexpr int LPT = SH::LPT, CPL = SH::CPL, EPC = SH::EPC, ROWB = SH::ROWB;
    __shared__ int scan[kStreamMaxSeqs + 1];
    scan_units<NW>(scan, context_lens, S, max_tokens);
    const int Hkv = num_kv_heads;
    const int64_t U = (int64_t)scan[S] * Hkv;
    if (blockIdx.x == 0)
        for (int s = threadIdx.x; s <= S; s += NW * 64) ws_scan[s] = scan[s];

    const int lane = threadIdx.x & 63, w = uniform(threadIdx.x >> 6);
    const int tg = lane / LPT, r = lane % LPT;
    const int gw = blockIdx.x * NW + w;
    int64_t ua, ub;
    if (!wave_range(scan, S, Hkv, U, nw, gw, ua, ub)) return;
    if (ua == ub) {  // one wave per pair, and this pair is empty
        zero_pair_rows<T, D>(out, gw, Hkv, num_q_heads, G, lane);
        return;
    }

    const int64_t head_bytes = (int64_t)B * ROWB;
    const int64_t block_bytes = head_bytes * Hkv;
    const char *kbase = (const char *)key_cache;
    const char *vbase = (const char *)value_cache;
    const int lane_off = tg * ROWB + r * 16;

    WaveAcc<T, D, G> acc;
    int cur_item = -1, cur_s = 0, cur_g = 0;

    // Write the finished (sequence, kv head) pair: directly to out when this
    // wave saw all of it, else as a partial record for the reduce kernel.
    auto finish = [&]() __attribute__((always_inline)) {
        acc.reduce_groups();
        const int us = scan[cur_s + 1] - scan[cur_s];
        const int64_t u0 = (int64_t)scan[cur_s] * Hkv + (int64_t)cur_g * us;
        const bool whole = u0 >= ua && u0 + us <= ub;
        if (tg != 0) return;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const int64_t qrow = (int64_t)cur_s * num_q_heads + (int64_t)cur_g * G + h;
            if (whole) {
                const float inv = acc.l[h] > 0.f ? 1.f / acc.l[h] : 0.f;
#pragma unroll
                for (int k = 0; k < CPL; ++k)
#pragma unroll
                    for (int e = 0; e < EPC; ++e)
                        Elem<T>::store(out + qrow * D + (r + LPT * k) * EPC + e,
                                       acc.o[h][k * EPC + e] * inv);
            } else {
                const int64_t rid = (int64_t)(cur_item + gw) * G + h;
#pragma unroll
                for (int k = 0; k < CPL; ++k)
#pragma unroll
                    for (int e = 0; e < EPC; e += 4)
                        *(float4 *)(rec_o + rid * D + (r + LPT * k) * EPC + e) =
                            make_float4(acc.o[h][k * EPC + e], acc.o[h][k * EPC + e + 1],
                                        acc.o[h][k * EPC + e + 2], acc.o[h][k * EPC + e + 3]);
                if (r == 0) *(float2 *)(rec_ml + rid * 2) = make_float2(acc.m[h], acc.l[h]);
            }
        }
    };

    for (int64_t base = ua; base < ub; base += 64) {
        const int n = (int)min((int64_t)64, ub - base);
        // Lane k describes unit base + k: its pair, row count and block.
        // With AP, l_new is the row of the unit that holds the new token
        // (its last unit, when the length was not clamped), else -1.
        int l_item = 0, l_nvalid = 0, l_phys = 0, l_tokoff = 0, l_new = -1, l_keep = 0;
        int l_s = 0, l_j = 0, l_us = 1;
        if (lane < n) {  // from the LDS scan alone
            const int64_t u = base + lane;
            l_s = seq_of_unit(scan, S, u, Hkv);
            l_us = scan[l_s + 1] - scan[l_s];
            const int rem = (int)(u - (int64_t)scan[l_s] * Hkv);
            const int g = rem / l_us;
            l_j = rem - g * l_us;
            l_item = l_s * Hkv + g;
        }
        // Append: the new tokens of the pairs that end in this chunk go to
        // their slots before this wave loads those units (its own stores
        // precede its loads of the same bytes).  The lanes form groups of
        // 2 * NCH, one 16-byte chunk of the K or V row each, one pair per
        // group.  The rows of the first PE pairs are fetched together with the
        // descriptors below, so they cost no extra round trip.
        constexpr int NCH = ROWB / 16, PE = 64 / (2 * NCH);
        const int grp = lane / (2 * NCH), c2 = lane % (2 * NCH);
        const bool c2v = c2 >= NCH;
        const int c2ch = c2v ? c2 - NCH : c2;
        uint64_t ends = 0;
        int first = -1;
        u32x4 first_row = {0, 0, 0, 0};
        if (AP) {
            ends = __builtin_amdgcn_ballot_w64(lane < n && l_j == l_us - 1);
#pragma unroll
            for (int e = 0; e < PE; ++e) {
                if (ends) {
                    const int bit = (int)__builtin_ctzll(ends);
                    ends &= ends - 1;
                    if (grp == e) first = bit;
                }
            }
            const int it = __shfl(l_item, first < 0 ? 0 : first);
            if (first >= 0)
                first_row = *(const u32x4 *)((const char *)(c2v ? new_value : new_key) +
                                             (int64_t)it * ROWB + c2ch * 16);
        }
        if (lane < n) {
            const int Lraw = context_lens[l_s];
            const int L = clamp_len(Lraw, max_tokens);
            const int tok = l_j * kUnitTokens;
            l_nvalid = min(kUnitTokens, L - tok);
            l_tokoff = tok % B;
            const int phys = block_tables[(int64_t)l_s * max_blocks + tok / B];
            if (phys < 0 || (int64_t)phys >= num_blocks) l_nvalid = 0;  // caller error
            l_phys = phys;
            l_keep = shared_with_neighbour(block_tables, S, max_blocks, l_s, tok / B, phys);
            if (AP && Lraw == L && l_j == l_us - 1 && l_nvalid > 0) l_new = l_nvalid - 1;
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // the descriptors above: vmcnt(0)

        if (AP) {
            // Store the row of pair unit `mine` (a lane index of this chunk).
            auto put = [&](int mine, const u32x4 &row) __attribute__((always_inline)) {
                const int src_lane = mine < 0 ? 0 : mine;
                const int it = __shfl(l_item, src_lane), ph = __shfl(l_phys, src_lane);
                const int to = __shfl(l_tokoff, src_lane), nr = __shfl(l_new, src_lane);
                if (mine >= 0 && nr >= 0) {
                    char *dst = (char *)(c2v ? value_cache : key_cache) + (int64_t)ph * block_bytes +
                                (int64_t)(it % Hkv) * head_bytes + (int64_t)(to + nr) * ROWB +
                                c2ch * 16;
                    *(u32x4 *)dst = row;
                }
            };
            put(first, first_row);
            while (ends) {  // more pairs end in this chunk than one batch holds
                int mine = -1;
#pragma unroll
                for (int e = 0; e < PE; ++e) {
                    if (ends) {
                        const int bit = (int)__builtin_ctzll(ends);
                        ends &= ends - 1;
                        if (grp == e) mine = bit;
                    }
                }
                const int it = __shfl(l_item, mine < 0 ? 0 : mine);
                u32x4 row = {0, 0, 0, 0};
                if (mine >= 0)
                    row = *(const u32x4 *)((const char *)(c2v ? new_value : new_key) +
                                           (int64_t)it * ROWB + c2ch * 16);
                put(mine, row);
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        }

        // Unit i of the chunk, or an empty range past the current segment.
        auto locate = [&](int i, int seg_end, int &nvalid) __attribute__((always_inline)) -> UnitRes {
            const int ii = i & 63;
            nvalid = (i < seg_end) ? __builtin_amdgcn_readlane(l_nvalid, ii) : 0;
            const int item = __builtin_amdgcn_readlane(l_item, ii);
            const int phys = __builtin_amdgcn_readlane(l_phys, ii);
            const int tokoff = __builtin_amdgcn_readlane(l_tokoff, ii);
            const int g = item % Hkv;
            const int64_t off = nvalid > 0 ? (int64_t)phys * block_bytes + (int64_t)g * head_bytes +
                                                 (int64_t)tokoff * ROWB
                                           : 0;
            return unit_res(kbase, vbase, off, nvalid > 0 ? SH::UNIT_BYTES : 0);
        };

        // Segments: runs of units of one (sequence, kv head) pair with one
        // cache policy.  At a pair boundary the previous pair is finished and
        // the next q is loaded together with the segment's first NBUF units;
        // inside a segment NBUF - 1 units stay in flight.
        constexpr int NB = SH::NBUF;
        UnitRegs<T, D, G> buf[NB];
        int nv[NB];
        for (int i0 = 0; i0 < n;) {
            const int item = __builtin_amdgcn_readlane(l_item, i0);
            const int keep = __builtin_amdgcn_readlane(l_keep, i0);
            const uint64_t other = __builtin_amdgcn_ballot_w64(
                lane < n && lane > i0 && (l_item != item || l_keep != keep));
            const int i1 = other ? (int)__builtin_ctzll(other) : n;  // segment end
            if (item != cur_item) {
                if (cur_item >= 0) finish();
                cur_item = item;
                cur_s = item / Hkv;
                cur_g = item - cur_s * Hkv;
                acc.reset();
                acc.load_q((const char *)query +
                               ((int64_t)cur_s * num_q_heads + (int64_t)cur_g * G) * ROWB, r);
            }
            // One copy of the pipeline per cache policy: the loads of a
            // segment and the uses of their results stay in one copy.
            auto run = [&](auto pol) __attribute__((always_inline)) {
                constexpr int POL = decltype(pol)::value;
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    load_unit<POL>(buf[b], locate(i0 + b, i1, nv[b]), lane_off);
                for (int i = i0; i < i1; i += NB) {
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        if (nv[b] > 0) acc.process(buf[b], nv[b], scale_log2, tg);
                        load_unit<POL>(buf[b], locate(i + NB + b, i1, nv[b]), lane_off);
                    }
                }
            };
            if (keep)
                run(std::integral_constant<int, kReuse>{});
            else
                run(std::integral_constant<int, kOnce>{});
            i0 = i1;
        }
    }
    if (cur_item >= 0) finish();
}

// ---------------------------------------------------------------------------
// Balanced split on the matrix cores (bf16).
//
// With grouped-query attention the G query heads of a kv head meet the same
// 16-token unit: per unit a G x 16 x D contraction for the logits and a
// G x D x 16 one for the output.  Done on the vector ALUs (the kernel above)
// that arithmetic is one fp32 operation per head per element, which at G = 8
// takes longer than streaming the unit from HBM.  Here both products run on
// MFMA, transposed so that the softmax weights pass from one to the other in
// registers (as in the prefill kernel):
//   S^T [16 tokens x 16 columns] = K [16 x D] . Q^T [D x 16]   (16x16x32, D/32 steps)
//   O^T [D x 16 columns]        += V^T [D x 16] . P^T [16 x 16] (16x16x16, D/16 tiles)
// Column c < G is query head c of the group (the others carry zeros).  K goes
// from HBM straight into the A-operand registers; V goes by DMA into a LDS
// slot of the wave and comes back transposed (ds_read_b64_tr_b16), 4 tokens
// of one dim per lane.  The loads of a unit use buffer resources whose range
// is the unit's valid rows, so rows past the context arrive as zeros.  The
// work split, records and reduce are those of decode_stream_kernel.
// ---------------------------------------------------------------------------

#ifndef PA_MMA_BUFFERS
#define PA_MMA_BUFFERS 3
#endif
constexpr int kMmaBuffers = PA_MMA_BUFFERS;  // units in flight + 1 per wave
constexpr int kMmaWaves = 4;    // waves per workgroup

typedef __bf16 bf16x8_mv __attribute__((ext_vector_type(8)));
typedef short s16x4_mv __attribute__((ext_vector_type(4)));
typedef float f32x4_mv __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_mv;

__device__ __forceinline__ s16x4_mv lds_tr16(uint32_t addr) {
    s16x4_mv r;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr));
    return r;
}
// Completes the transposing reads above (and orders later memory operations,
// the next DMA into the slot among them, after it).
template <int N>
__device__ __forceinline__ void lds_tr_wait(s16x4_mv (&v)[N]) {
    static_assert(N == 4 || N == 8, "batch");
    if constexpr (N == 4)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]) : : "memory");
    else
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                       "+v"(v[6]), "+v"(v[7])
                     : : "memory");
}

// Chunk permutation of a V row in its LDS slot: chunk c of row r sits at
// c ^ mma_swz(r), so the transposing reads of 16 rows hit distinct banks.
template <int D>
__device__ __forceinline__ int mma_swz(int row) {
    return D == 128 ? (row & 7) << 1 : ((row >> 1) & 3) << 1;
}

// 16 bytes per lane from a buffer (offset voff) into LDS at lds + 16 * lane,
// with cache policy POL; lanes outside the buffer's range write zeros.
template <int POL>
__device__ __forceinline__ void dma16_to_lds(__amdgpu_buffer_rsrc_t r, void *lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_mv *)lds, 16, voff, 0, 0, POL);
}

__device__ __forceinline__ uint32_t lds_offset(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

__device__ __forceinline__ float max4_lanes(float x) {  // over lanes l, l^16, l^32, l^48
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <int D, int B, int G, int NW, bool AP>
__global__ __launch_bounds__(NW * 64) void decode_stream_mma_kernel(
    bf16_t *__restrict__ out, const bf16_t *__restrict__ query, bf16_t *__restrict__ key_cache,
    bf16_t *__restrict__ value_cache, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, int S, int num_q_heads, int num_kv_heads,
    int max_blocks, int max_tokens, int64_t num_blocks, int nw, float scale_log2,
    float *__restrict__ rec_o, float *__restrict__ rec_ml, int *__restrict__ ws_scan,
    const bf16_t *__restrict__ new_key, const bf16_t *__restrict__ new_value, int len_skip,
    int force_records) {
    constexpr int ROWB = D * 2, NCH = ROWB / 16, KS = D / 32, DT = D / 16;
    constexpr int UNIT_BYTES = kUnitTokens * ROWB, NB = kMmaBuffers;
    constexpr int KPS = 1024 / ROWB;               // rows per 1 KB DMA segment
    constexpr int SEGS = UNIT_BYTES / 1024;        // DMA instructions per unit
    static_assert(G <= 16, "group fits the 16 columns");
    extern __shared__ int scan[];                  // [S + 1], sized at launch
    __shared__ __attribute__((aligned(1024))) char vslot[NW][NB][UNIT_BYTES];
    scan_units<NW>(scan, context_lens, S, max_tokens, len_skip);
    const int Hkv = num_kv_heads;
    const int64_t U = (int64_t)scan[S] * Hkv;
    if (blockIdx.x == 0)
        for (int s = threadIdx.x; s <= S; s += NW * 64) ws_scan[s] = scan[s];

    const int lane = threadIdx.x & 63, w = uniform(threadIdx.x >> 6);
    const int l16 = lane & 15, lg = lane >> 4;
    const int gw = blockIdx.x * NW + w;
    int64_t ua, ub;
    if (!wave_range(scan, S, Hkv, U, nw, gw, ua, ub)) return;
    if (ua == ub) {  // one wave per pair, and this pair is empty
        zero_pair_rows<bf16_t, D>(out, gw, Hkv, num_q_heads, G, lane);
        return;
    }

    const int64_t head_bytes = (int64_t)B * ROWB;
    const int64_t block_bytes = head_bytes * Hkv;
    const char *kbase = (const char *)key_cache;
    const char *vbase = (const char *)value_cache;

    // Lane offsets.  K operand of k-step ks: token l16, dims ks * 32 + lg * 8.
    const int k_off = l16 * ROWB + lg * 16;
    // V DMA: lane i of segment sg moves chunk i % NCH of row sg * KPS + i / NCH,
    // stored at chunk position (i % NCH) ^ swz(row) of that row.
    const int dma_row = lane / NCH, dma_ch = lane % NCH;
    // V^T operand of dim tile dt: the lanes of group lg read rows 4 * lg + (l16 >> 2),
    // dims dt * 16 + 4 * (l16 & 3), i.e. chunk 2 * dt + ((l16 & 3) >> 1), half l16 & 1.
    const int v_row = 4 * lg + (l16 >> 2);
    const uint32_t v_lane =
        v_row * ROWB + (l16 & 1) * 8 + ((mma_swz<D>(v_row) ^ ((l16 & 3) >> 1)) << 4);
    // A operand whose row 0 is all ones (for the column sums of P^T).
    const s16x4_mv ones_a = l16 == 0 ? s16x4_mv{0x3F80, 0x3F80, 0x3F80, 0x3F80} : s16x4_mv{0, 0, 0, 0};

    u32x4 qt[KS];          // Q^T operand of the current pair
    f32x4_mv acc_o[DT];    // O^T: lane holds dims dt * 16 + 4 * lg + i of column l16
    f32x4_mv acc_l;        // element 0 of lanes 0..15: sum of weights of column l16
    float m_col = NEG_INF; // reference maximum of column l16 (log2 units)
    int cur_item = -1, cur_s = 0, cur_g = 0;

    auto reset = [&](int s, int g) __attribute__((always_inline)) {
        const bool valid = l16 < G;
        const char *qrow = (const char *)query +
                           ((int64_t)s * num_q_heads + (int64_t)g * G + (valid ? l16 : 0)) * ROWB;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 v = *(const u32x4 *)(qrow + ks * 64 + lg * 16);
            qt[ks] = valid ? v : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc_o[dt] = f32x4_mv{0.f, 0.f, 0.f, 0.f};
        acc_l = f32x4_mv{0.f, 0.f, 0.f, 0.f};
        m_col = NEG_INF;
    };

    // Write the finished pair: to out when this wave saw all of it, else as a
    // partial record (the layout decode_stream_kernel writes).
    auto finish = [&]() __attribute__((always_inline)) {
        const int us = scan[cur_s + 1] - scan[cur_s];
        const int64_t u0 = (int64_t)scan[cur_s] * Hkv + (int64_t)cur_g * us;
        const bool whole = !force_records && u0 >= ua && u0 + us <= ub;
        const float lsum = __shfl(acc_l[0], l16);
        if (l16 >= G) return;
        const int64_t qrow = (int64_t)cur_s * num_q_heads + (int64_t)cur_g * G + l16;
        if (whole) {
            const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                uint2 v;
                v.x = pack_bf16x2(acc_o[dt][0] * inv, acc_o[dt][1] * inv);
                v.y = pack_bf16x2(acc_o[dt][2] * inv, acc_o[dt][3] * inv);
                *(uint2 *)(out + qrow * D + dt * 16 + lg * 4) = v;
            }
        } else {
            const int64_t rid = (int64_t)(cur_item + gw) * G + l16;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                *(float4 *)(rec_o + rid * D + dt * 16 + lg * 4) =
                    make_float4(acc_o[dt][0], acc_o[dt][1], acc_o[dt][2], acc_o[dt][3]);
            if (lg == 0) *(float2 *)(rec_ml + rid * 2) = make_float2(m_col, lsum);
        }
    };

    for (int64_t base = ua; base < ub; base += 64) {
        const int n = (int)min((int64_t)64, ub - base);
        int l_item = 0, l_nvalid = 0, l_phys = 0, l_tokoff = 0, l_new = -1, l_keep = 0;
        int l_s = 0, l_j = 0, l_us = 1;
        if (lane < n) {  // from the LDS scan alone
            const int64_t u = base + lane;
            l_s = seq_of_unit(scan, S, u, Hkv);
            l_us = scan[l_s + 1] - scan[l_s];
            const int rem = (int)(u - (int64_t)scan[l_s] * Hkv);
            const int g = rem / l_us;
            l_j = rem - g * l_us;
            l_item = l_s * Hkv + g;
        }
        // Append (see decode_stream_kernel): the rows of the first PE pairs
        // that end in this chunk are fetched with the descriptors.
        constexpr int PE = 64 / (2 * NCH);
        const int grp = lane / (2 * NCH), c2 = lane % (2 * NCH);
        const bool c2v = c2 >= NCH;
        const int c2ch = c2v ? c2 - NCH : c2;
        uint64_t ends = 0;
        int first = -1;
        u32x4 first_row = {0, 0, 0, 0};
        if (AP) {
            ends = __builtin_amdgcn_ballot_w64(lane < n && l_j == l_us - 1);
#pragma unroll
            for (int e = 0; e < PE; ++e) {
                if (ends) {
                    const int bit = (int)__builtin_ctzll(ends);
                    ends &= ends - 1;
                    if (grp == e) first = bit;
                }
            }
            const int it = __shfl(l_item, first < 0 ? 0 : first);
            if (first >= 0)
                first_row = *(const u32x4 *)((const char *)(c2v ? new_value : new_key) +
                                             (int64_t)it * ROWB + c2ch * 16);
        }
        if (lane < n) {
            const int Lraw = past_skip(context_lens[l_s], len_skip);
            const int L = clamp_len(Lraw, max_tokens);
            const int tok = l_j * kUnitTokens;
            l_nvalid = min(kUnitTokens, L - tok);
            l_tokoff = tok % B;
            const int phys = block_tables[(int64_t)l_s * max_blocks + tok / B];
            if (phys < 0 || (int64_t)phys >= num_blocks) l_nvalid = 0;  // caller error
            l_phys = phys;
            l_keep = shared_with_neighbour(block_tables, S, max_blocks, l_s, tok / B, phys);
            if (AP && Lraw == L && l_j == l_us - 1 && l_nvalid > 0) l_new = l_nvalid - 1;
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // the descriptors above: vmcnt(0)
        if (AP) {
            auto put = [&](int mine, const u32x4 &row) __attribute__((always_inline)) {
                const int src_lane = mine < 0 ? 0 : mine;
                const int it = __shfl(l_item, src_lane), ph = __shfl(l_phys, src_lane);
                const int to = __shfl(l_tokoff, src_lane), nr = __shfl(l_new, src_lane);
                if (mine >= 0 && nr >= 0) {
                    char *dst = (char *)(c2v ? value_cache : key_cache) + (int64_t)ph * block_bytes +
                                (int64_t)(it % Hkv) * head_bytes + (int64_t)(to + nr) * ROWB +
                                c2ch * 16;
                    *(u32x4 *)dst = row;
                }
            };
            put(first, first_row);
            while (ends) {
                int mine = -1;
#pragma unroll
                for (int e = 0; e < PE; ++e) {
                    if (ends) {
                        const int bit = (int)__builtin_ctzll(ends);
                        ends &= ends - 1;
                        if (grp == e) mine = bit;
                    }
                }
                const int it = __shfl(l_item, mine < 0 ? 0 : mine);
                u32x4 row = {0, 0, 0, 0};
                if (mine >= 0)
                    row = *(const u32x4 *)((const char *)(c2v ? new_value : new_key) +
                                           (int64_t)it * ROWB + c2ch * 16);
                put(mine, row);
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        }

        // Issue unit i of the chunk into buffer b: V by DMA into the wave's
        // slot b, then K into registers (waiting for K then also covers the
        // older DMA).  Units past the segment get empty ranges: no memory is
        // touched and zeros land.
        u32x4 kb[NB][KS];
        int nv[NB];
        auto issue = [&](auto pol, int b, int i, int seg_end) __attribute__((always_inline)) {
            constexpr int POL = decltype(pol)::value;
            const int ii = i & 63;
            const int nvalid = (i < seg_end) ? __builtin_amdgcn_readlane(l_nvalid, ii) : 0;
            const int item = __builtin_amdgcn_readlane(l_item, ii);
            const int phys = __builtin_amdgcn_readlane(l_phys, ii);
            const int tokoff = __builtin_amdgcn_readlane(l_tokoff, ii);
            const int64_t off = nvalid > 0 ? (int64_t)phys * block_bytes +
                                                 (int64_t)(item % Hkv) * head_bytes +
                                                 (int64_t)tokoff * ROWB
                                           : 0;
            const int range = nvalid > 0 ? nvalid * ROWB : 0;
            nv[b] = nvalid;
            const __amdgpu_buffer_rsrc_t rk =
                __builtin_amdgcn_make_buffer_rsrc((void *)(kbase + off), (short)0, range, 0x00020000);
            const __amdgpu_buffer_rsrc_t rv =
                __builtin_amdgcn_make_buffer_rsrc((void *)(vbase + off), (short)0, range, 0x00020000);
#pragma unroll
            for (int sg = 0; sg < SEGS; ++sg) {
                const int row = sg * KPS + dma_row;
                dma16_to_lds<POL>(rv, &vslot[w][b][sg * 1024],
                                  row * ROWB + ((dma_ch ^ mma_swz<D>(row)) << 4));
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kb[b][ks] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, k_off + ks * 64, 0, POL));
        };

        // One unit: logits, online softmax per column, P V.
        auto process = [&](int b) __attribute__((always_inline)) {
            f32x4_mv st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_mv, kb[b][ks]),
                                                             __builtin_bit_cast(bf16x8_mv, qt[ks]),
                                                             st, 0, 0, 0);
            // V^T reads of the slot, in flight while the softmax runs.
            const uint32_t vb = lds_offset(&vslot[w][b][0]) + v_lane;
            s16x4_mv va[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) va[dt] = lds_tr16(vb ^ ((uint32_t)dt << 5));
            float x[4];
            bool need = m_col == NEG_INF;
            float lmax = NEG_INF;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = (4 * lg + i < nv[b]) ? st[i] * scale_log2 : NEG_INF;
                lmax = fmaxf(lmax, x[i]);
            }
            need |= lmax > m_col + kRescaleThreshold;
            if (__builtin_amdgcn_ballot_w64(need)) {
                const float mn = fmaxf(m_col, max4_lanes(lmax));
                const float alpha = (m_col == NEG_INF) ? 0.f : fast_exp2(m_col - mn);
                m_col = mn;
                acc_l *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc_o[dt] *= alpha;
            }
            const float mneg = (m_col == NEG_INF) ? 0.f : -m_col;
            uint32_t p01 = pack_bf16x2(fast_exp2(x[0] + mneg), fast_exp2(x[1] + mneg));
            uint32_t p23 = pack_bf16x2(fast_exp2(x[2] + mneg), fast_exp2(x[3] + mneg));
            const s16x4_mv pt = __builtin_bit_cast(s16x4_mv, (uint64_t)p01 | ((uint64_t)p23 << 32));
            acc_l = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones_a, pt, acc_l, 0, 0, 0);
            if constexpr (DT == 8) lds_tr_wait<8>(va); else lds_tr_wait<4>(va);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[dt], pt, acc_o[dt], 0, 0, 0);
        };

        // Segments: runs of units of one pair with one cache policy.
        for (int i0 = 0; i0 < n;) {
            const int item = __builtin_amdgcn_readlane(l_item, i0);
            const int keep = __builtin_amdgcn_readlane(l_keep, i0);
            const uint64_t other = __builtin_amdgcn_ballot_w64(
                lane < n && lane > i0 && (l_item != item || l_keep != keep));
            const int i1 = other ? (int)__builtin_ctzll(other) : n;  // segment end
            if (item != cur_item) {
                if (cur_item >= 0) finish();
                cur_item = item;
                cur_s = item / Hkv;
                cur_g = item - cur_s * Hkv;
                reset(cur_s, cur_g);
            }
            // One copy of the pipeline per cache policy: the loads of a
            // segment and the uses of their results stay in one copy.
            auto run = [&](auto pol) __attribute__((always_inline)) {
#pragma unroll
                for (int b = 0; b < NB; ++b) issue(pol, b, i0 + b, i1);
                for (int i = i0; i < i1; i += NB) {
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        if (nv[b] > 0) process(b);
                        issue(pol, b, i + NB + b, i1);
                    }
                }
            };
            if (keep)
                run(std::integral_constant<int, kReuse>{});
            else
                run(std::integral_constant<int, kOnce>{});
            i0 = i1;
        }
    }
    if (cur_item >= 0) finish();
}

// ---------------------------------------------------------------------------
// Shared prefix (bf16).  When the first P tokens of every sequence lie in the
// same physical blocks (a common prompt reused through prefix caching:
// "Configuring vLLM and PagedAttention for High Throughput Enterprise LLM
// Serving", section "Zero-Copy Prefix Caching & Shared Sampling"), the decode
// kernels above stream those blocks once per sequence.  This kernel reads them
// once per group of sequences: the 16 MFMA columns of a wave carry 16 / G
// sequences x the G query heads of one kv head, so every K/V unit it loads
// serves all of them.  A wave covers a 1 / ksplit share of the prefix's units
// and writes one record (m, l, unnormalised o) per column; the reduce merges
// those with the records of the balanced split over each sequence's tokens
// past P.  Column c's keys stop at min(L_s, P), so a sequence no longer than
// the prefix attends to its own tokens only.  Products, softmax and V path are
// those of decode_stream_mma_kernel.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, one L2 each
// Unit buffers of the prefix pass: two keep it at 188 + 40 registers and
// 32 KiB of LDS per workgroup, so one of its workgroups fits on a CU beside
// one of the suffix pass (the two run on separate streams at once).
constexpr int kPrefixBuffers = 2;

template <int D, int B, int G, int NW>
__global__ __launch_bounds__(NW * 64) void decode_prefix_mma_kernel(
    const bf16_t *__restrict__ query, const bf16_t *__restrict__ key_cache,
    const bf16_t *__restrict__ value_cache, const int32_t *__restrict__ prefix_table,
    const int32_t *__restrict__ context_lens, int S, int num_q_heads, int num_kv_heads,
    int64_t num_blocks, int prefix_tokens, int ksplit, float scale_log2, float *__restrict__ x_o,
    float *__restrict__ x_ml) {
    constexpr int ROWB = D * 2, NCH = ROWB / 16, KS = D / 32, DT = D / 16;
    constexpr int UNIT_BYTES = kUnitTokens * ROWB, NB = kPrefixBuffers;
    constexpr int KPS = 1024 / ROWB;               // rows per 1 KB DMA segment
    constexpr int SEGS = UNIT_BYTES / 1024;        // DMA instructions per unit
    constexpr int CPW = 16 / G;                    // sequences per wave
    __shared__ __attribute__((aligned(1024))) char vslot[NW][NB][UNIT_BYTES];

    const int lane = threadIdx.x & 63, w = uniform(threadIdx.x >> 6);
    const int l16 = lane & 15, lg = lane >> 4;
    const int Hkv = num_kv_heads;
    const int ncg = cdiv(S, CPW);
    // Workgroups are dispatched round-robin over the 8 XCDs (each with its own
    // L2).  Renumber them so that consecutive wave numbers, which share a kv
    // head and so read the same prefix pages, run on one XCD.
    const int total = gridDim.x, bid = blockIdx.x;
    const int xcd = bid % kXcds, idx = bid / kXcds;
    const int q8 = total / kXcds, rem = total % kXcds;
    const int lin = xcd < rem ? xcd * (q8 + 1) + idx : rem * (q8 + 1) + (xcd - rem) * q8 + idx;
    const int gw = lin * NW + w;
    const int k = gw % ksplit, rest = gw / ksplit;
    const int cg = rest % ncg, g = rest / ncg;
    if (g >= Hkv) return;

    // This lane's column: sequence s, head hh of kv head g.
    const int s = cg * CPW + l16 / G, hh = l16 % G;
    const bool col_ok = s < S;
    int lim = 0;
    if (col_ok) {
        const int L = context_lens[s];
        lim = L < 0 ? 0 : min(L, prefix_tokens);
    }
    const int nu = cdiv(prefix_tokens, kUnitTokens);
    const int u0 = (int)((int64_t)nu * k / ksplit), u1 = (int)((int64_t)nu * (k + 1) / ksplit);

    const int64_t head_bytes = (int64_t)B * ROWB;
    const int64_t block_bytes = head_bytes * Hkv;
    const char *kbase = (const char *)key_cache;
    const char *vbase = (const char *)value_cache;
    const int k_off = l16 * ROWB + lg * 16;
    const int dma_row = lane / NCH, dma_ch = lane % NCH;
    const int v_row = 4 * lg + (l16 >> 2);
    const uint32_t v_lane =
        v_row * ROWB + (l16 & 1) * 8 + ((mma_swz<D>(v_row) ^ ((l16 & 3) >> 1)) << 4);
    const s16x4_mv ones_a = l16 == 0 ? s16x4_mv{0x3F80, 0x3F80, 0x3F80, 0x3F80} : s16x4_mv{0, 0, 0, 0};

    u32x4 qt[KS];
    {
        const char *qrow = (const char *)query +
                           ((int64_t)(col_ok ? s : 0) * num_q_heads + (int64_t)g * G + hh) * ROWB;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 v = *(const u32x4 *)(qrow + ks * 64 + lg * 16);
            qt[ks] = col_ok ? v : u32x4{0, 0, 0, 0};
        }
    }
    f32x4_mv acc_o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc_o[dt] = f32x4_mv{0.f, 0.f, 0.f, 0.f};
    f32x4_mv acc_l = {0.f, 0.f, 0.f, 0.f};
    float m_col = NEG_INF;

    for (int c0 = u0; c0 < u1; c0 += 64) {
        const int n = min(64, u1 - c0);
        // Lane j: unit c0 + j of the prefix (its page from row 0 of the table).
        int l_nvalid = 0, l_phys = 0, l_tokoff = 0;
        if (lane < n) {
            const int tok = (c0 + lane) * kUnitTokens;
            l_nvalid = min(kUnitTokens, prefix_tokens - tok);
            l_tokoff = tok % B;
            const int phys = prefix_table[tok / B];
            if (phys < 0 || (int64_t)phys >= num_blocks) l_nvalid = 0;  // caller error
            l_phys = phys;
        }

        u32x4 kb[NB][KS];
        int nv[NB], ut[NB];
        auto issue = [&](int b, int i) __attribute__((always_inline)) {
            const int ii = i & 63;
            const int nvalid = i < n ? __builtin_amdgcn_readlane(l_nvalid, ii) : 0;
            const int phys = __builtin_amdgcn_readlane(l_phys, ii);
            const int tokoff = __builtin_amdgcn_readlane(l_tokoff, ii);
            const int64_t off = nvalid > 0 ? (int64_t)phys * block_bytes + (int64_t)g * head_bytes +
                                                 (int64_t)tokoff * ROWB
                                           : 0;
            const int range = nvalid > 0 ? nvalid * ROWB : 0;
            nv[b] = nvalid;
            ut[b] = (c0 + i) * kUnitTokens;
            const __amdgpu_buffer_rsrc_t rk =
                __builtin_amdgcn_make_buffer_rsrc((void *)(kbase + off), (short)0, range, 0x00020000);
            const __amdgpu_buffer_rsrc_t rv =
                __builtin_amdgcn_make_buffer_rsrc((void *)(vbase + off), (short)0, range, 0x00020000);
#pragma unroll
            for (int sg = 0; sg < SEGS; ++sg) {
                const int row = sg * KPS + dma_row;
                dma16_to_lds<kReuse>(rv, &vslot[w][b][sg * 1024],
                             row * ROWB + ((dma_ch ^ mma_swz<D>(row)) << 4));
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kb[b][ks] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, k_off + ks * 64, 0, kReuse));
        };

        auto process = [&](int b) __attribute__((always_inline)) {
            f32x4_mv st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_mv, kb[b][ks]),
                                                             __builtin_bit_cast(bf16x8_mv, qt[ks]),
                                                             st, 0, 0, 0);
            const uint32_t vb = lds_offset(&vslot[w][b][0]) + v_lane;
            s16x4_mv va[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) va[dt] = lds_tr16(vb ^ ((uint32_t)dt << 5));
            float x[4];
            bool need = m_col == NEG_INF;
            float lmax = NEG_INF;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = (ut[b] + 4 * lg + i < lim) ? st[i] * scale_log2 : NEG_INF;
                lmax = fmaxf(lmax, x[i]);
            }
            need |= lmax > m_col + kRescaleThreshold;
            if (__builtin_amdgcn_ballot_w64(need)) {
                const float mn = fmaxf(m_col, max4_lanes(lmax));
                const float alpha = (m_col == NEG_INF) ? 0.f : fast_exp2(m_col - mn);
                m_col = mn;
                acc_l *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc_o[dt] *= alpha;
            }
            const float mneg = (m_col == NEG_INF) ? 0.f : -m_col;
            uint32_t p01 = pack_bf16x2(fast_exp2(x[0] + mneg), fast_exp2(x[1] + mneg));
            uint32_t p23 = pack_bf16x2(fast_exp2(x[2] + mneg), fast_exp2(x[3] + mneg));
            const s16x4_mv pt = __builtin_bit_cast(s16x4_mv, (uint64_t)p01 | ((uint64_t)p23 << 32));
            acc_l = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones_a, pt, acc_l, 0, 0, 0);
            if constexpr (DT == 8) lds_tr_wait<8>(va); else lds_tr_wait<4>(va);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[dt], pt, acc_o[dt], 0, 0, 0);
        };

#pragma unroll
        for (int b = 0; b < NB; ++b) issue(b, b);
        for (int i = 0; i < n; i += NB) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if (nv[b] > 0) process(b);
                issue(b, i + NB + b);
            }
        }
    }

    const float lsum = __shfl(acc_l[0], l16);
    if (!col_ok) return;
    const int64_t rid = ((int64_t)s * num_q_heads + (int64_t)g * G + hh) * ksplit + k;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        *(float4 *)(x_o + rid * D + dt * 16 + lg * 4) =
            make_float4(acc_o[dt][0], acc_o[dt][1], acc_o[dt][2], acc_o[dt][3]);
    if (lg == 0) *(float2 *)(x_ml + rid * 2) = make_float2(m_col, lsum);
}

// ---------------------------------------------------------------------------
// Balanced split over an FP8 (e4m3) cache: the same work split, records and
// reduce as decode_stream_mma_kernel, reading one byte per element.
//
// Every element of the pools is an e4m3 code of value / scale, with one fp32
// scale per pool (quantised KV cache: "vLLM Guide: High-Throughput Multi-GPU
// LLM Serving with PagedAttention", the quantisation support among the
// engine's pillars and its FP8 engine example).  An e4m3 value has a 3-bit
// mantissa and an exponent inside bf16's range, so every code widens to bf16
// exactly (v_cvt_scalef32_pk_bf16_fp8 with a unit scale); the pools' scales
// are applied outside the products: k_scale inside the softmax scale, v_scale
// on the output.  Both products then run on the bf16 matrix cores exactly as
// in the kernel above.
//
// Layouts.  K: [block][kv head][token][dim], a unit of 16 tokens is 16 * D
// contiguous bytes.  V: [block][kv head][dim][token] (each page transposed),
// so a unit's V is D rows of 16 bytes, one per dim, and the V^T operand of the
// P V product (one dim x 4 consecutive tokens per lane) is one 4-byte word of
// such a row.
//   K operand, k-step ks: lane (l16, lg) holds token l16, dims lg * D/4 + 8 ks
//     + [0, 8) -- one contiguous D/4-byte piece of the token's row per lane
//     (16-byte loads); the Q^T operand takes the same dims, so the
//     contraction is unchanged.
//   V^T operand, tile dt: lane (l16, lg) holds dim dt * 16 + l16, tokens
//     4 lg + [0, 4).  The unit's rows go by DMA (16 bytes a lane, 1 KB an
//     instruction) into a LDS slot of the wave, and come back as 4-byte LDS
//     reads.  Loading the words straight from HBM would take D / 16 loads of
//     256 bytes each per unit; the vector memory path keeps a bounded number
//     of load instructions in flight, so the bytes in flight, and the rate,
//     fall with the bytes per instruction.
// K rows past the unit's valid tokens come back as zeros (buffer range); in V
// they share a row with valid tokens, so a partial unit masks its bytes.
// ---------------------------------------------------------------------------

// Three unit buffers (two units in flight): 1.5-2% faster than five on the
// FP8 8B, 32K and prefix-sharing decodes once the loads became non-temporal.
#ifndef PA_FP8_BUFFERS
#define PA_FP8_BUFFERS 3
#endif
constexpr int kFp8Buffers = PA_FP8_BUFFERS;  // units in flight + 1 per wave
constexpr int kFp8Waves = 4;                 // waves per workgroup

__device__ __forceinline__ uint32_t lds_read_b32(uint32_t addr) {
    uint32_t r;
    asm volatile("ds_read_b32 %0, %1" : "=v"(r) : "v"(addr));
    return r;
}
// Completes the LDS reads above: their registers stay live until here.
template <int N>
__device__ __forceinline__ void lds_b32_wait(uint32_t (&v)[N]) {
    static_assert(N == 4 || N == 8, "batch");
    if constexpr (N == 4)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]) : : "memory");
    else
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                       "+v"(v[6]), "+v"(v[7])
                     : : "memory");
}

// Two e4m3 codes (bytes 0-1, or 2-3 when HI) -> two bf16, exactly.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// AP (append): the step's new token of sequence s (bf16 rows new_key[s],
// new_value[s], [S][Hkv][D]) sits at position L_s - 1; the wave that streams
// the unit holding it quantises the rows (codes of x * k_inv, x * v_inv, as
// the FP8 cache write) into their slot before it loads the unit.
template <int D, int B, int G, int NW, bool AP>
__global__ __launch_bounds__(NW * 64) void decode_stream_fp8_kernel(
    bf16_t *__restrict__ out, const bf16_t *__restrict__ query,
    uint8_t *__restrict__ key_cache, uint8_t *__restrict__ value_cache,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ context_lens, int S,
    int num_q_heads, int num_kv_heads, int max_blocks, int max_tokens, int64_t num_blocks, int nw,
    float scale_log2, float v_scale, float *__restrict__ rec_o, float *__restrict__ rec_ml,
    int *__restrict__ ws_scan, const bf16_t *__restrict__ new_key,
    const bf16_t *__restrict__ new_value, float k_inv, float v_inv, int len_skip,
    int force_records) {
    constexpr int KS = D / 32, DT = D / 16, KB = D / 4, KW = KB / 16;
    constexpr int NB = kFp8Buffers;
    static_assert(G <= 16, "group fits the 16 columns");
    constexpr int VSEG = D / 64;  // V DMA instructions per unit
    extern __shared__ int scan[];  // [S + 1], sized at launch
    __shared__ __attribute__((aligned(1024))) char vslot[NW][NB][D * 16];
    scan_units<NW>(scan, context_lens, S, max_tokens, len_skip);
    const int Hkv = num_kv_heads;
    const int64_t U = (int64_t)scan[S] * Hkv;
    if (blockIdx.x == 0)
        for (int s = threadIdx.x; s <= S; s += NW * 64) ws_scan[s] = scan[s];

    const int lane = threadIdx.x & 63, w = uniform(threadIdx.x >> 6);
    const int l16 = lane & 15, lg = lane >> 4;
    const int gw = blockIdx.x * NW + w;
    int64_t ua, ub;
    if (!wave_range(scan, S, Hkv, U, nw, gw, ua, ub)) return;
    if (ua == ub) {  // one wave per pair, and this pair is empty
        zero_pair_rows<bf16_t, D>(out, gw, Hkv, num_q_heads, G, lane);
        return;
    }

    const int64_t head_bytes = (int64_t)B * D;
    const int64_t block_bytes = head_bytes * Hkv;
    const char *kbase = (const char *)key_cache;
    const char *vbase = (const char *)value_cache;
    const int k_off = l16 * D + lg * KB;  // from the unit's first K row
    // V^T reads: row dt * 16 + l16 of the slot (16 bytes a row), word lg.
    const uint32_t v_lane = (uint32_t)(l16 * 16 + lg * 4);
    const s16x4_mv ones_a = l16 == 0 ? s16x4_mv{0x3F80, 0x3F80, 0x3F80, 0x3F80} : s16x4_mv{0, 0, 0, 0};

    u32x4 qt[KS];
    f32x4_mv acc_o[DT];
    f32x4_mv acc_l;
    float m_col = NEG_INF;
    int cur_item = -1, cur_s = 0, cur_g = 0;

    auto reset = [&](int s, int g) __attribute__((always_inline)) {
        const bool valid = l16 < G;
        const char *qrow = (const char *)query +
                           ((int64_t)s * num_q_heads + (int64_t)g * G + (valid ? l16 : 0)) * (D * 2);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 v = *(const u32x4 *)(qrow + (lg * KB + 8 * ks) * 2);
            qt[ks] = valid ? v : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc_o[dt] = f32x4_mv{0.f, 0.f, 0.f, 0.f};
        acc_l = f32x4_mv{0.f, 0.f, 0.f, 0.f};
        m_col = NEG_INF;
    };

    auto finish = [&]() __attribute__((always_inline)) {
        const int us = scan[cur_s + 1] - scan[cur_s];
        const int64_t u0 = (int64_t)scan[cur_s] * Hkv + (int64_t)cur_g * us;
        const bool whole = !force_records && u0 >= ua && u0 + us <= ub;
        const float lsum = __shfl(acc_l[0], l16);
        if (l16 >= G) return;
        const int64_t qrow = (int64_t)cur_s * num_q_heads + (int64_t)cur_g * G + l16;
        if (whole) {
            const float inv = lsum > 0.f ? v_scale / lsum : 0.f;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                uint2 v;
                v.x = pack_bf16x2(acc_o[dt][0] * inv, acc_o[dt][1] * inv);
                v.y = pack_bf16x2(acc_o[dt][2] * inv, acc_o[dt][3] * inv);
                *(uint2 *)(out + qrow * D + dt * 16 + lg * 4) = v;
            }
        } else {
            const int64_t rid = (int64_t)(cur_item + gw) * G + l16;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                *(float4 *)(rec_o + rid * D + dt * 16 + lg * 4) =
                    make_float4(acc_o[dt][0] * v_scale, acc_o[dt][1] * v_scale,
                                acc_o[dt][2] * v_scale, acc_o[dt][3] * v_scale);
            if (lg == 0) *(float2 *)(rec_ml + rid * 2) = make_float2(m_col, lsum);
        }
    };

    for (int64_t base = ua; base < ub; base += 64) {
        const int n = (int)min((int64_t)64, ub - base);
        int l_item = 0, l_nvalid = 0, l_phys = 0, l_tokoff = 0, l_new = -1, l_keep = 0;
        int l_s = 0, l_j = 0, l_us = 1;
        if (lane < n) {  // from the LDS scan alone
            const int64_t u = base + lane;
            l_s = seq_of_unit(scan, S, u, Hkv);
            l_us = scan[l_s + 1] - scan[l_s];
            const int rem = (int)(u - (int64_t)scan[l_s] * Hkv);
            const int g = rem / l_us;
            l_j = rem - g * l_us;
            l_item = l_s * Hkv + g;
        }
        // Append: the new rows of the pairs ending in this chunk, PE pairs per
        // pass.  A group of D / 4 lanes takes one pair, D / 8 lanes on its K
        // row and D / 8 on its V row, 8 elements a lane; the first pass's
        // rows are fetched together with the descriptors.
        constexpr int GL = D / 4, PE = 64 / GL;
        const int grp = lane / GL, c8 = lane % GL;
        const bool isv = c8 >= GL / 2;
        const int e0 = (isv ? c8 - GL / 2 : c8) * 8;  // first element of the lane
        uint64_t ends = 0;
        int first = -1;
        u32x4 first_row = {0, 0, 0, 0};
        auto take_ends = [&]() __attribute__((always_inline)) -> int {
            int mine = -1;
#pragma unroll
            for (int e = 0; e < PE; ++e) {
                if (ends) {
                    const int bit = (int)__builtin_ctzll(ends);
                    ends &= ends - 1;
                    if (grp == e) mine = bit;
                }
            }
            return mine;
        };
        auto fetch_row = [&](int mine) __attribute__((always_inline)) -> u32x4 {
            const int it = __shfl(l_item, mine < 0 ? 0 : mine);
            if (mine < 0) return u32x4{0, 0, 0, 0};
            return *(const u32x4 *)((isv ? new_value : new_key) + (int64_t)it * D + e0);
        };
        if (AP) {
            ends = __builtin_amdgcn_ballot_w64(lane < n && l_j == l_us - 1);
            first = take_ends();
            first_row = fetch_row(first);
        }
        if (lane < n) {
            const int Lraw = past_skip(context_lens[l_s], len_skip);
            const int L = clamp_len(Lraw, max_tokens);
            const int tok = l_j * kUnitTokens;
            l_nvalid = min(kUnitTokens, L - tok);
            l_tokoff = tok % B;
            const int phys = block_tables[(int64_t)l_s * max_blocks + tok / B];
            if (phys < 0 || (int64_t)phys >= num_blocks) l_nvalid = 0;  // caller error
            l_phys = phys;
            l_keep = shared_with_neighbour(block_tables, S, max_blocks, l_s, tok / B, phys);
            if (AP && Lraw == L && l_j == l_us - 1 && l_nvalid > 0) l_new = l_nvalid - 1;
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // the descriptors above: vmcnt(0)
        if (AP) {
            // Quantise and store the rows of one pass (ends whose position
            // turned out invalid store nothing).
            auto put = [&](int mine, const u32x4 &row) __attribute__((always_inline)) {
                const int src = mine < 0 ? 0 : mine;
                const int it = __shfl(l_item, src), ph = __shfl(l_phys, src);
                const int to = __shfl(l_tokoff, src), nr = __shfl(l_new, src);
                if (mine >= 0 && nr >= 0) {
                    const float inv = isv ? v_inv : k_inv;
                    uint32_t wd[2] = {0u, 0u};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t word = row[e >> 1];
                        const float x = (e & 1) ? bf16_hi(word) : bf16_lo(word);
                        wd[e >> 2] |= e4m3_code(x * inv) << (8 * (e & 3));
                    }
                    const int64_t page = (int64_t)ph * block_bytes + (int64_t)(it % Hkv) * head_bytes;
                    if (!isv) {
                        *(uint2 *)(key_cache + page + (int64_t)(to + nr) * D + e0) =
                            make_uint2(wd[0], wd[1]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            value_cache[page + (int64_t)(e0 + e) * B + to + nr] =
                                (uint8_t)(wd[e >> 2] >> (8 * (e & 3)));
                    }
                }
            };
            put(first, first_row);
            while (ends) {
                const int mine = take_ends();
                put(mine, fetch_row(mine));
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        }

        // Issue unit i of the chunk into buffer b.  Units past the segment get
        // empty ranges: no memory is touched and zeros land.
        u32x4 kb[NB][KW];
        int nv[NB];
        auto issue = [&](auto pol, int b, int i, int seg_end) __attribute__((always_inline)) {
            constexpr int POL = decltype(pol)::value;
            const int ii = i & 63;
            const int nvalid = (i < seg_end) ? __builtin_amdgcn_readlane(l_nvalid, ii) : 0;
            const int item = __builtin_amdgcn_readlane(l_item, ii);
            const int phys = __builtin_amdgcn_readlane(l_phys, ii);
            const int tokoff = __builtin_amdgcn_readlane(l_tokoff, ii);
            const int64_t page = nvalid > 0 ? (int64_t)phys * block_bytes + (int64_t)(item % Hkv) * head_bytes : 0;
            nv[b] = nvalid;
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(kbase + page + (int64_t)tokoff * D), (short)0, nvalid > 0 ? nvalid * D : 0,
                0x00020000);
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(vbase + page + tokoff), (short)0, nvalid > 0 ? (D - 1) * B + kUnitTokens : 0,
                0x00020000);
            // V first: waiting for this unit's K registers then also covers
            // its DMA (loads complete in issue order).
            // A unit of a 32-token block reads half of each 32-byte V row
            // and the block's other unit the rest, from the caches: there
            // both tensors keep the default policy (non-temporal K alone made
            // the FP8 32K decode 4% slower).
            constexpr int UPOL = B == kUnitTokens ? POL : kReuse;
#pragma unroll
            for (int sg = 0; sg < VSEG; ++sg)
                dma16_to_lds<UPOL>(rv, &vslot[w][b][sg * 1024], (sg * 64 + lane) * B);
#pragma unroll
            for (int c = 0; c < KW; ++c)
                kb[b][c] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, k_off + c * 16, 0, UPOL));
        };

        auto process = [&](int b) __attribute__((always_inline)) {
            f32x4_mv st = {0.f, 0.f, 0.f, 0.f};
            // This unit's loads are the oldest in flight: the NB - 1 younger
            // units issued VSEG + KW loads each.  Once they are done, its V
            // rows are in the slot.
            asm volatile("s_waitcnt vmcnt(%0)" : : "n"((NB - 1) * (VSEG + KW)) : "memory");
            const uint32_t vb0 = lds_offset(&vslot[w][b][0]) + v_lane;
            uint32_t vw[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) vw[dt] = lds_read_b32(vb0 + dt * 256);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const uint32_t w0 = kb[b][ks >> 1][(ks & 1) * 2];
                const uint32_t w1 = kb[b][ks >> 1][(ks & 1) * 2 + 1];
                const u32x4 kop = {e4m3x2_to_bf16x2<false>(w0), e4m3x2_to_bf16x2<true>(w0),
                                   e4m3x2_to_bf16x2<false>(w1), e4m3x2_to_bf16x2<true>(w1)};
                st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_mv, kop),
                                                             __builtin_bit_cast(bf16x8_mv, qt[ks]),
                                                             st, 0, 0, 0);
            }
            float x[4];
            bool need = m_col == NEG_INF;
            float lmax = NEG_INF;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = (4 * lg + i < nv[b]) ? st[i] * scale_log2 : NEG_INF;
                lmax = fmaxf(lmax, x[i]);
            }
            need |= lmax > m_col + kRescaleThreshold;
            if (__builtin_amdgcn_ballot_w64(need)) {
                const float mn = fmaxf(m_col, max4_lanes(lmax));
                const float alpha = (m_col == NEG_INF) ? 0.f : fast_exp2(m_col - mn);
                m_col = mn;
                acc_l *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc_o[dt] *= alpha;
            }
            const float mneg = (m_col == NEG_INF) ? 0.f : -m_col;
            const uint32_t p01 = pack_bf16x2(fast_exp2(x[0] + mneg), fast_exp2(x[1] + mneg));
            const uint32_t p23 = pack_bf16x2(fast_exp2(x[2] + mneg), fast_exp2(x[3] + mneg));
            const s16x4_mv pt = __builtin_bit_cast(s16x4_mv, (uint64_t)p01 | ((uint64_t)p23 << 32));
            acc_l = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones_a, pt, acc_l, 0, 0, 0);
            // Tokens past the valid ones share their 4-byte words with valid
            // tokens; their codes (stale or poison) must not reach the product.
            uint32_t vmask = 0xFFFFFFFFu;
            if (nv[b] < kUnitTokens) {
                const int cnt = min(max(nv[b] - 4 * lg, 0), 4);
                vmask = cnt == 4 ? 0xFFFFFFFFu : ((1u << (8 * cnt)) - 1u);
            }
            lds_b32_wait<DT>(vw);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const uint32_t wv = vw[dt] & vmask;
                const s16x4_mv va = __builtin_bit_cast(
                    s16x4_mv, (uint64_t)e4m3x2_to_bf16x2<false>(wv) |
                                  ((uint64_t)e4m3x2_to_bf16x2<true>(wv) << 32));
                acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pt, acc_o[dt], 0, 0, 0);
            }
        };

        // Segments: runs of units of one pair with one cache policy.
        for (int i0 = 0; i0 < n;) {
            const int item = __builtin_amdgcn_readlane(l_item, i0);
            const int keep = __builtin_amdgcn_readlane(l_keep, i0);
            const uint64_t other = __builtin_amdgcn_ballot_w64(
                lane < n && lane > i0 && (l_item != item || l_keep != keep));
            const int i1 = other ? (int)__builtin_ctzll(other) : n;  // segment end
            if (item != cur_item) {
                if (cur_item >= 0) finish();
                cur_item = item;
                cur_s = item / Hkv;
                cur_g = item - cur_s * Hkv;
                reset(cur_s, cur_g);
            }
            // One copy of the pipeline per cache policy: the loads of a
            // segment and the uses of their results stay in one copy.
            auto run = [&](auto pol) __attribute__((always_inline)) {
#pragma unroll
                for (int b = 0; b < NB; ++b) issue(pol, b, i0 + b, i1);
                for (int i = i0; i < i1; i += NB) {
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        if (nv[b] > 0) process(b);
                        issue(pol, b, i + NB + b, i1);
                    }
                }
            };
            if (keep)
                run(std::integral_constant<int, kReuse>{});
            else
                run(std::integral_constant<int, kOnce>{});
            i0 = i1;
        }
    }
    if (cur_item >= 0) finish();
}

// ---------------------------------------------------------------------------
// Shared prefix over an FP8 cache: the work split, columns and records of
// decode_prefix_mma_kernel (16 / G sequences x the G query heads of one kv
// head per wave, a 1 / ksplit share of the prefix's units, one record per
// column), with the loads, code widening and V path of
// decode_stream_fp8_kernel (K codes into registers and widened to bf16 for
// the S^T product; V pages by DMA into a slot and read back as 4-byte words
// of 4 tokens).  Records hold v_scale * o, as the FP8 balanced split's do,
// so the reduce merges both kinds unchanged.  Every prefix unit is whole
// (the prefix is whole blocks); column c's keys stop at min(L_s, P) through
// its logits, and the codes past that are written cache entries of the
// shared blocks.
// ---------------------------------------------------------------------------
template <int D, int B, int G, int NW>
__global__ __launch_bounds__(NW * 64) void decode_prefix_fp8_kernel(
    const bf16_t *__restrict__ query, const uint8_t *__restrict__ key_cache,
    const uint8_t *__restrict__ value_cache, const int32_t *__restrict__ prefix_table,
    const int32_t *__restrict__ context_lens, int S, int num_q_heads, int num_kv_heads,
    int64_t num_blocks, int prefix_tokens, int ksplit, float scale_log2, float v_scale,
    float *__restrict__ x_o, float *__restrict__ x_ml) {
    constexpr int KS = D / 32, DT = D / 16, KB = D / 4, KW = KB / 16;
    constexpr int NB = kPrefixBuffers;
    constexpr int VSEG = D / 64;  // V DMA instructions per unit
    constexpr int CPW = 16 / G;   // sequences per wave
    __shared__ __attribute__((aligned(1024))) char vslot[NW][NB][D * 16];

    const int lane = threadIdx.x & 63, w = uniform(threadIdx.x >> 6);
    const int l16 = lane & 15, lg = lane >> 4;
    const int Hkv = num_kv_heads;
    const int ncg = cdiv(S, CPW);
    // Consecutive wave numbers share a kv head, so its prefix pages: keep
    // them on one XCD (workgroups are dispatched round-robin over the XCDs).
    const int total = gridDim.x, bid = blockIdx.x;
    const int xcd = bid % kXcds, idx = bid / kXcds;
    const int q8 = total / kXcds, rem = total % kXcds;
    const int lin = xcd < rem ? xcd * (q8 + 1) + idx : rem * (q8 + 1) + (xcd - rem) * q8 + idx;
    const int gw = lin * NW + w;
    const int k = gw % ksplit, rest = gw / ksplit;
    const int cg = rest % ncg, g = rest / ncg;
    if (g >= Hkv) return;

    const int s = cg * CPW + l16 / G, hh = l16 % G;  // this lane's column
    const bool col_ok = s < S;
    int lim = 0;
    if (col_ok) {
        const int L = context_lens[s];
        lim = L < 0 ? 0 : min(L, prefix_tokens);
    }
    const int nu = cdiv(prefix_tokens, kUnitTokens);
    const int u0 = (int)((int64_t)nu * k / ksplit), u1 = (int)((int64_t)nu * (k + 1) / ksplit);

    const int64_t head_bytes = (int64_t)B * D;
    const int64_t block_bytes = head_bytes * Hkv;
    const char *kbase = (const char *)key_cache;
    const char *vbase = (const char *)value_cache;
    const int k_off = l16 * D + lg * KB;  // from the unit's first K row
    const uint32_t v_lane = (uint32_t)(l16 * 16 + lg * 4);
    const s16x4_mv ones_a = l16 == 0 ? s16x4_mv{0x3F80, 0x3F80, 0x3F80, 0x3F80} : s16x4_mv{0, 0, 0, 0};

    u32x4 qt[KS];
    {
        const char *qrow = (const char *)query +
                           ((int64_t)(col_ok ? s : 0) * num_q_heads + (int64_t)g * G + hh) * (D * 2);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 v = *(const u32x4 *)(qrow + (lg * KB + 8 * ks) * 2);
            qt[ks] = col_ok ? v : u32x4{0, 0, 0, 0};
        }
    }
    f32x4_mv acc_o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc_o[dt] = f32x4_mv{0.f, 0.f, 0.f, 0.f};
    f32x4_mv acc_l = {0.f, 0.f, 0.f, 0.f};
    float m_col = NEG_INF;

    for (int c0 = u0; c0 < u1; c0 += 64) {
        const int n = min(64, u1 - c0);
        // Lane j: unit c0 + j of the prefix (its page from row 0 of the table).
        int l_nvalid = 0, l_phys = 0, l_tokoff = 0;
        if (lane < n) {
            const int tok = (c0 + lane) * kUnitTokens;
            l_nvalid = min(kUnitTokens, prefix_tokens - tok);
            l_tokoff = tok % B;
            const int phys = prefix_table[tok / B];
            if (phys < 0 || (int64_t)phys >= num_blocks) l_nvalid = 0;  // caller error
            l_phys = phys;
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // the descriptors above: vmcnt(0)

        u32x4 kb[NB][KW];
        int nv[NB], ut[NB];
        auto issue = [&](int b, int i) __attribute__((always_inline)) {
            const int ii = i & 63;
            const int nvalid = i < n ? __builtin_amdgcn_readlane(l_nvalid, ii) : 0;
            const int phys = __builtin_amdgcn_readlane(l_phys, ii);
            const int tokoff = __builtin_amdgcn_readlane(l_tokoff, ii);
            const int64_t page =
                nvalid > 0 ? (int64_t)phys * block_bytes + (int64_t)g * head_bytes : 0;
            nv[b] = nvalid;
            ut[b] = (c0 + i) * kUnitTokens;
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(kbase + page + (int64_t)tokoff * D), (short)0, nvalid > 0 ? nvalid * D : 0,
                0x00020000);
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(vbase + page + tokoff), (short)0,
                nvalid > 0 ? (D - 1) * B + kUnitTokens : 0, 0x00020000);
#pragma unroll
            for (int sg = 0; sg < VSEG; ++sg)
                dma16_to_lds<kReuse>(rv, &vslot[w][b][sg * 1024], (sg * 64 + lane) * B);
#pragma unroll
            for (int c = 0; c < KW; ++c)
                kb[b][c] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, k_off + c * 16, 0, kReuse));
        };

        auto process = [&](int b) __attribute__((always_inline)) {
            // The NB - 1 younger units issued VSEG + KW loads each: once they
            // are the only ones left, this unit's K and V have arrived.
            asm volatile("s_waitcnt vmcnt(%0)" : : "n"((NB - 1) * (VSEG + KW)) : "memory");
            const uint32_t vb0 = lds_offset(&vslot[w][b][0]) + v_lane;
            uint32_t vw[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) vw[dt] = lds_read_b32(vb0 + dt * 256);
            f32x4_mv st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const uint32_t w0 = kb[b][ks >> 1][(ks & 1) * 2];
                const uint32_t w1 = kb[b][ks >> 1][(ks & 1) * 2 + 1];
                const u32x4 kop = {e4m3x2_to_bf16x2<false>(w0), e4m3x2_to_bf16x2<true>(w0),
                                   e4m3x2_to_bf16x2<false>(w1), e4m3x2_to_bf16x2<true>(w1)};
                st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_mv, kop),
                                                             __builtin_bit_cast(bf16x8_mv, qt[ks]),
                                                             st, 0, 0, 0);
            }
            float x[4];
            bool need = m_col == NEG_INF;
            float lmax = NEG_INF;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = (ut[b] + 4 * lg + i < lim) ? st[i] * scale_log2 : NEG_INF;
                lmax = fmaxf(lmax, x[i]);
            }
            need |= lmax > m_col + kRescaleThreshold;
            if (__builtin_amdgcn_ballot_w64(need)) {
                const float mn = fmaxf(m_col, max4_lanes(lmax));
                const float alpha = (m_col == NEG_INF) ? 0.f : fast_exp2(m_col - mn);
                m_col = mn;
                acc_l *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc_o[dt] *= alpha;
            }
            const float mneg = (m_col == NEG_INF) ? 0.f : -m_col;
            const uint32_t p01 = pack_bf16x2(fast_exp2(x[0] + mneg), fast_exp2(x[1] + mneg));
            const uint32_t p23 = pack_bf16x2(fast_exp2(x[2] + mneg), fast_exp2(x[3] + mneg));
            const s16x4_mv pt = __builtin_bit_cast(s16x4_mv, (uint64_t)p01 | ((uint64_t)p23 << 32));
            acc_l = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones_a, pt, acc_l, 0, 0, 0);
            lds_b32_wait<DT>(vw);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const s16x4_mv va = __builtin_bit_cast(
                    s16x4_mv, (uint64_t)e4m3x2_to_bf16x2<false>(vw[dt]) |
                                  ((uint64_t)e4m3x2_to_bf16x2<true>(vw[dt]) << 32));
                acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pt, acc_o[dt], 0, 0, 0);
            }
        };

#pragma unroll
        for (int b = 0; b < NB; ++b) issue(b, b);
        for (int i = 0; i < n; i += NB) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if (nv[b] > 0) process(b);
                issue(b, i + NB + b);
            }
        }
    }

    const float lsum = __shfl(acc_l[0], l16);
    if (!col_ok) return;
    const int64_t rid = ((int64_t)s * num_q_heads + (int64_t)g * G + hh) * ksplit + k;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        *(float4 *)(x_o + rid * D + dt * 16 + lg * 4) =
            make_float4(acc_o[dt][0] * v_scale, acc_o[dt][1] * v_scale, acc_o[dt][2] * v_scale,
                        acc_o[dt][3] * v_scale);
    if (lg == 0) *(float2 *)(x_ml + rid * 2) = make_float2(m_col, lsum);
}

// Merge the nrec partial records (m_k: max in log2 units, l_k: sum, o_k:
// unnormalised output) of one output row: with M = max_k m_k,
// dst = sum_k o_k 2^(m_k - M) / sum_k l_k 2^(m_k - M) (log-sum-exp merge of
// split softmax results).  Record k's (m, l) pair is at ml + k * ml_stride, its
// output at o + k * o_stride.  Lane k loads the weights of record k, and the
// outputs of 8 records are loaded before any is used, so a row costs a few
// memory round trips rather than one per record.  XR: x_n further records
// (x_ml + 2k, x_o + k * D; the shared-prefix records) follow the nrec ones
// as records nrec .. nrec + x_n - 1; nrec may then be 0.
template <typename T, int D, bool XR = false>
__device__ __forceinline__ void merge_records(T *__restrict__ dst, const float *__restrict__ ml,
                                              int64_t ml_stride, const float *__restrict__ o,
                                              int64_t o_stride, int nrec, int lane,
                                              const float *__restrict__ x_ml = nullptr,
                                              const float *__restrict__ x_o = nullptr,
                                              int x_n = 0) {
    constexpr int DPL = D / 64;  // dims per lane
    typedef float vecd __attribute__((ext_vector_type(DPL)));
    const int nall = XR ? nrec + x_n : nrec;
    auto ml_at = [&](int k) __attribute__((always_inline)) -> const float * {
        if (XR && k >= nrec) return x_ml + 2 * (k - nrec);
        return ml + k * ml_stride;
    };
    auto o_at = [&](int k) __attribute__((always_inline)) -> const float * {
        if (XR && k >= nrec) return x_o + (int64_t)(k - nrec) * D;
        return o + k * o_stride;
    };
    float2 w0 = make_float2(NEG_INF, 0.f);
    if (lane < nall) w0 = *(const float2 *)ml_at(lane);
    // The outputs of the first 8 records go out with the weights (they do not
    // depend on them), so a row of up to 8 records costs one round trip.
    vecd v0[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v0[j] = *(const vecd *)(o_at(min(j, nall - 1)) + lane * DPL);
    float M = w0.x;
    for (int k = lane + 64; k < nall; k += 64) M = fmaxf(M, *ml_at(k));
    M = wave_max(M);
    float lsum = 0.f;
    vecd acc = {};
    for (int c0 = 0; c0 < nall; c0 += 64) {
        float2 w = w0;
        if (c0 > 0) {
            w = make_float2(NEG_INF, 0.f);
            if (c0 + lane < nall) w = *(const float2 *)ml_at(c0 + lane);
        }
        const float f = (w.x == NEG_INF) ? 0.f : fast_exp2(w.x - M);  // 0 past nall
        lsum = fmaf(f, w.y, lsum);
        const int n = min(64, nall - c0);
        for (int j0 = 0; j0 < n; j0 += 8) {
            vecd v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int k = c0 + min(j0 + j, n - 1);  // padded slots reload a valid record
                v[j] = (c0 == 0 && j0 == 0) ? v0[j] : *(const vecd *)(o_at(k) + lane * DPL);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float fj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), j0 + j));
                acc += fj * v[j];
            }
        }
    }
    lsum = group_sum<16>(lsum);
    lsum = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lsum), 0)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lsum), 16)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lsum), 32)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lsum), 48));
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) Elem<T>::store(dst + lane * DPL + e, acc[e] * inv);
}

// Merge the partial records of each (sequence, q head): records of pair i
// come from waves wave_of_unit(first unit) .. wave_of_unit(last unit), stored
// at record i + wave.  One wave per output row.
// XR: every row also merges its x_n (1 .. 8) shared-prefix records (x_o
// [row][x_n][D], x_ml [row][x_n][2]), and the decode kernel wrote every pair
// as records.
template <typename T, int D, bool XR>
__global__ __launch_bounds__(256) void decode_stream_reduce_kernel(
    T *__restrict__ out, const int *__restrict__ ws_scan, int S, int num_q_heads,
    int num_kv_heads, int nw, const float *__restrict__ rec_o, const float *__restrict__ rec_ml,
    const float *__restrict__ x_o, const float *__restrict__ x_ml, int x_n) {
    constexpr int DPL = D / 64;  // dims per lane
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= (int64_t)S * num_q_heads) return;
    const int s = (int)(row / num_q_heads), h = (int)(row - (int64_t)s * num_q_heads);
    const int G = num_q_heads / num_kv_heads;
    const int g = h / G, hh = h - g * G;
    const int us = ws_scan[s + 1] - ws_scan[s];
    const float *xo = XR ? x_o + row * x_n * D : nullptr;
    const float *xml = XR ? x_ml + row * x_n * 2 : nullptr;
    if (us == 0) {
        if (XR) {
            merge_records<T, D, XR>(out + row * D, nullptr, 0, nullptr, 0, 0, lane, xml, xo, x_n);
            return;
        }
#pragma unroll
        for (int e = 0; e < DPL; ++e) Elem<T>::store(out + row * D + lane * DPL + e, 0.f);
        return;
    }
    const int64_t U = (int64_t)ws_scan[S] * num_kv_heads;
    const int nwe = (int)min((int64_t)nw, U);  // the waves that worked (us > 0, so U > 0)
    const int64_t u0 = (int64_t)ws_scan[s] * num_kv_heads + (int64_t)g * us;
    const int w0 = wave_of_unit(u0, U, nwe), w1 = wave_of_unit(u0 + us - 1, U, nwe);
    if (w0 == w1 && !XR) return;  // finished by its wave
    const int64_t item = (int64_t)s * num_kv_heads + g;
    const int64_t rid0 = (item + w0) * G + hh;
    merge_records<T, D, XR>(out + row * D, rec_ml + rid0 * 2, 2 * G, rec_o + rid0 * D,
                            (int64_t)G * D, w1 - w0 + 1, lane, xml, xo, x_n);
}

// ---------------------------------------------------------------------------
// Fixed partitions: one workgroup per (sequence, kv head, partition).
// ---------------------------------------------------------------------------

template <typename T, int D, int B, int G, int NW>
__global__ __launch_bounds__(NW * 64) void decode_partition_kernel(
    T *__restrict__ out, const T *__restrict__ query, const T *__restrict__ key_cache,
    const T *__restrict__ value_cache, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, int num_q_heads, int num_kv_heads,
    int max_blocks, int max_tokens, int64_t num_blocks, int P, int np_max, float scale_log2,
    float *__restrict__ ws_o, float *__restrict__ ws_ml) {
    using SH = DecodeShape<T, D, G>;
    constexpr int LPT = SH::LPT, CPL = SH::CPL, EPC = SH::EPC, ROWB = SH::ROWB;

    const int p = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
    // max_tokens = min(max_blocks * B, max_context_len, np_max * P): longer
    // lengths are clamped, so no access leaves the buffers.
    const int L = clamp_len(context_lens[s], max_tokens);
    const int np = cdiv(L, P);
    if (p >= np) return;  // whole workgroup: this partition is empty
    const int tok0 = p * P;
    const int tok1 = min(L, tok0 + P);
    const int nunits = cdiv(tok1 - tok0, kUnitTokens);
    const int u_first = tok0 / kUnitTokens;

    const int lane = threadIdx.x & 63, w = uniform(threadIdx.x >> 6);
    const int tg = lane / LPT, r = lane % LPT;

    WaveAcc<T, D, G> acc;
    acc.reset();
    acc.load_q((const char *)query + ((int64_t)s * num_q_heads + (int64_t)g * G) * ROWB, r);

    const int32_t *bt = block_tables + (int64_t)s * max_blocks;
    const char *kbase = (const char *)key_cache;
    const char *vbase = (const char *)value_cache;
    const int64_t head_bytes = (int64_t)B * ROWB;
    const int64_t block_bytes = head_bytes * num_kv_heads;
    const int lane_off = tg * ROWB + r * 16;

    // Units of this wave: w, w + NW, ... (at most 64, so P <= 64 * NW * 16);
    // lane i holds the physical block of the i-th.
    const int nmine = nunits > w ? cdiv(nunits - w, NW) : 0;
    int lane_phys = 0;
    {
        const int u = w + NW * lane;
        if (u < nunits) lane_phys = bt[((u_first + u) * kUnitTokens) / B];
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // that load: vmcnt(0), once, on every path

    auto locate = [&](int i, int &nvalid) __attribute__((always_inline)) -> UnitRes {
        const int u = w + NW * i;
        const int tok = (u_first + u) * kUnitTokens;
        const int phys = __builtin_amdgcn_readlane(lane_phys, i & 63);
        nvalid = (i < nmine) ? min(kUnitTokens, tok1 - tok) : 0;
        if (phys < 0 || (int64_t)phys >= num_blocks) nvalid = 0;  // caller error
        const int64_t off = nvalid > 0
            ? (int64_t)phys * block_bytes + (int64_t)g * head_bytes + (tok % B) * ROWB : 0;
        return unit_res(kbase, vbase, off, nvalid > 0 ? SH::UNIT_BYTES : 0);
    };

    constexpr int NB = SH::NBUF;
    UnitRegs<T, D, G> buf[NB];
    int nv[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) load_unit<kOnce>(buf[b], locate(b, nv[b]), lane_off);
    for (int i = 0; i < nmine; i += NB) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (nv[b] > 0) acc.process(buf[b], nv[b], scale_log2, tg);
            load_unit<kOnce>(buf[b], locate(i + NB + b, nv[b]), lane_off);
        }
    }

    // ---- merge the waves -------------------------------------------------------
    acc.reduce_groups();
    __shared__ float red_o[NW][G * D];
    __shared__ float red_l[NW][G];
    __shared__ float red_m[NW][G];
    if (tg == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int k = 0; k < CPL; ++k)
#pragma unroll
                for (int e = 0; e < EPC; ++e)
                    red_o[w][h * D + (r + LPT * k) * EPC + e] = acc.o[h][k * EPC + e];
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            red_l[w][h] = acc.l[h];
            red_m[w][h] = acc.m[h];
        }
    }
    __syncthreads();

    for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
        const int h = idx / D, d = idx - h * D;
        float M = NEG_INF;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, red_m[ww][h]);
        float o = 0.f, lsum = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const float mw = red_m[ww][h];
            const float f = (mw == NEG_INF) ? 0.f : fast_exp2(mw - M);
            o = fmaf(f, red_o[ww][idx], o);
            lsum = fmaf(f, red_l[ww][h], lsum);
        }
        const int64_t qrow = (int64_t)s * num_q_heads + (int64_t)g * G + h;
        if (np == 1) {
            Elem<T>::store(out + qrow * D + d, lsum > 0.f ? o / lsum : 0.f);
        } else {
            ws_o[(qrow * np_max + p) * D + d] = o;
            if (d == 0) *(float2 *)(ws_ml + (qrow * np_max + p) * 2) = make_float2(M, lsum);
        }
    }
}

// Merge the partitions of each (sequence, q head): with M = max_p m_p,
// out = sum_p o_p 2^(m_p - M) / sum_p l_p 2^(m_p - M).  One wave per output
// row; sequences with a single partition were finished by the partition
// kernel, empty ones get zeros.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(
    T *__restrict__ out, const int32_t *__restrict__ context_lens, int S, int num_q_heads,
    int max_tokens, int P, int np_max, const float *__restrict__ ws_o,
    const float *__restrict__ ws_ml) {
    constexpr int DPL = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= (int64_t)S * num_q_heads) return;
    const int s = (int)(row / num_q_heads);
    const int np = cdiv(clamp_len(context_lens[s], max_tokens), P);
    if (np == 1) return;
    if (np == 0) {
#pragma unroll
        for (int e = 0; e < DPL; ++e) Elem<T>::store(out + row * D + lane * DPL + e, 0.f);
        return;
    }
    merge_records<T, D>(out + row * D, ws_ml + row * np_max * 2, 2, ws_o + row * np_max * D, D, np,
                        lane);
}

// ---- dispatch ---------------------------------------------------------------

// Tokens of a sequence the kernels will read: the table's capacity, the
// declared maximum context and, for fixed partitions, the partitions in the
// grid.  Longer context lengths are clamped to it.
static int max_tokens(const DecodeArgs &a) {
    int64_t m = (int64_t)a.max_blocks_per_seq * a.block_size;
    if (a.max_context_len < m) m = a.max_context_len;
    if (a.stream_waves == 0) {
        const int64_t by_grid = (int64_t)a.num_partitions * a.partition_size;
        if (by_grid < m) m = by_grid;
    }
    return (int)m;
}

// The balanced-split kernels' wave count argument: the equal split over
// stream_waves waves, or 0 for one wave per (sequence, kv head) pair.
static int kernel_waves(const DecodeArgs &a) { return a.pairs ? 0 : a.stream_waves; }

#ifndef PA_DECODE_MMA
#define PA_DECODE_MMA 1
#endif

template <int D, int B, int G>
static hipError_t launch_stream_mma(const DecodeArgs &a, hipStream_t stream, int len_skip = 0,
                                    int force_records = 0) {
    const dim3 grid(cdiv(a.stream_waves, kMmaWaves));
    const size_t dyn = (size_t)(a.num_seqs + 1) * sizeof(int);
    if (a.new_key)
        hipLaunchKernelGGL((decode_stream_mma_kernel<D, B, G, kMmaWaves, true>), grid,
                           dim3(kMmaWaves * 64), dyn, stream, (bf16_t *)a.out,
                           (const bf16_t *)a.query, (bf16_t *)a.key_cache, (bf16_t *)a.value_cache,
                           a.block_tables, a.context_lens, a.num_seqs, a.num_q_heads,
                           a.num_kv_heads, a.max_blocks_per_seq, max_tokens(a), a.num_blocks,
                           kernel_waves(a), a.scale * kLog2e, a.ws_o, a.ws_ml, a.ws_scan,
                           (const bf16_t *)a.new_key, (const bf16_t *)a.new_value, len_skip,
                           force_records);
    else
        hipLaunchKernelGGL((decode_stream_mma_kernel<D, B, G, kMmaWaves, false>), grid,
                           dim3(kMmaWaves * 64), dyn, stream, (bf16_t *)a.out,
                           (const bf16_t *)a.query, (bf16_t *)a.key_cache, (bf16_t *)a.value_cache,
                           a.block_tables, a.context_lens, a.num_seqs, a.num_q_heads,
                           a.num_kv_heads, a.max_blocks_per_seq, max_tokens(a), a.num_blocks,
                           kernel_waves(a), a.scale * kLog2e, a.ws_o, a.ws_ml, a.ws_scan,
                           (const bf16_t *)nullptr, (const bf16_t *)nullptr, len_skip,
                           force_records);
    return hipGetLastError();
}

template <int D, int B, int G, bool AP>
static void launch_stream_fp8_as(const DecodeArgs &a, hipStream_t stream, int len_skip = 0,
                                 int force_records = 0) {
    hipLaunchKernelGGL((decode_stream_fp8_kernel<D, B, G, kFp8Waves, AP>),
                       dim3(cdiv(a.stream_waves, kFp8Waves)), dim3(kFp8Waves * 64),
                       (size_t)(a.num_seqs + 1) * sizeof(int), stream, (bf16_t *)a.out,
                       (const bf16_t *)a.query, (uint8_t *)a.key_cache, (uint8_t *)a.value_cache,
                       a.block_tables, a.context_lens, a.num_seqs, a.num_q_heads, a.num_kv_heads,
                       a.max_blocks_per_seq, max_tokens(a), a.num_blocks, kernel_waves(a),
                       a.scale * kLog2e * a.k_scale, a.v_scale, a.ws_o, a.ws_ml, a.ws_scan,
                       (const bf16_t *)a.new_key, (const bf16_t *)a.new_value, 1.0f / a.k_scale,
                       1.0f / a.v_scale, len_skip, force_records);
}

template <int D, int B, int G>
static hipError_t launch_stream_fp8(const DecodeArgs &a, hipStream_t stream) {
    if (a.new_key)
        launch_stream_fp8_as<D, B, G, true>(a, stream);
    else
        launch_stream_fp8_as<D, B, G, false>(a, stream);
    return hipGetLastError();
}

template <typename T, int D, int B, int G>
static hipError_t launch_part(const DecodeArgs &a, hipStream_t stream) {
    if (a.kv_fp8) {  // bf16 query and output over e4m3 pools, balanced split only
        if constexpr (std::is_same<T, bf16_t>::value)
            if (a.stream_waves > 0) return launch_stream_fp8<D, B, G>(a, stream);
        return hipErrorNotSupported;
    }
    if (PA_DECODE_MMA && std::is_same<T, bf16_t>::value && a.stream_waves > 0)
        return launch_stream_mma<D, B, G>(a, stream);
    if (a.stream_waves > 0) {
        dim3 grid(cdiv(a.stream_waves, kDecodeWaves));
        if (a.new_key)
            hipLaunchKernelGGL((decode_stream_kernel<T, D, B, G, kDecodeWaves, true>), grid,
                               dim3(kDecodeWaves * 64), 0, stream, (T *)a.out, (const T *)a.query,
                               (T *)a.key_cache, (T *)a.value_cache, a.block_tables,
                               a.context_lens, a.num_seqs, a.num_q_heads, a.num_kv_heads,
                               a.max_blocks_per_seq, max_tokens(a), a.num_blocks, kernel_waves(a),
                               a.scale * kLog2e, a.ws_o, a.ws_ml, a.ws_scan, (const T *)a.new_key,
                               (const T *)a.new_value);
        else
            hipLaunchKernelGGL((decode_stream_kernel<T, D, B, G, kDecodeWaves, false>), grid,
                               dim3(kDecodeWaves * 64), 0, stream, (T *)a.out, (const T *)a.query,
                               (T *)a.key_cache, (T *)a.value_cache, a.block_tables,
                               a.context_lens, a.num_seqs, a.num_q_heads, a.num_kv_heads,
                               a.max_blocks_per_seq, max_tokens(a), a.num_blocks, kernel_waves(a),
                               a.scale * kLog2e, a.ws_o, a.ws_ml, a.ws_scan, (const T *)nullptr,
                               (const T *)nullptr);
    } else {
        if (a.new_key) {
            const hipError_t e = launch_append_rows(
                a.new_key, a.new_value, (void *)a.key_cache, (void *)a.value_cache, a.block_tables,
                a.context_lens, a.num_seqs, a.num_kv_heads, D, B, a.max_blocks_per_seq,
                a.num_blocks, max_tokens(a), (int)sizeof(T), stream);
            if (e != hipSuccess) return e;
        }
        dim3 grid(a.num_partitions, a.num_kv_heads, a.num_seqs);
        hipLaunchKernelGGL((decode_partition_kernel<T, D, B, G, kDecodeWaves>), grid,
                           dim3(kDecodeWaves * 64), 0, stream, (T *)a.out, (const T *)a.query,
                           (const T *)a.key_cache, (const T *)a.value_cache, a.block_tables,
                           a.context_lens, a.num_q_heads, a.num_kv_heads, a.max_blocks_per_seq,
                           max_tokens(a), a.num_blocks, a.partition_size, a.num_partitions,
                           a.scale * kLog2e, a.ws_o, a.ws_ml);
    }
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
    if (a.num_seqs == 0) return hipSuccess;
    if (a.stream_waves == 0 && a.num_partitions == 0) return hipSuccess;
    return a.dtype == 1 ? by_dim<bf16_t>(a, stream) : by_dim<float>(a, stream);
}

template <typename T, int D>
static hipError_t launch_red(const DecodeArgs &a, hipStream_t stream,
                             const PrefixArgs *px = nullptr) {
    const unsigned blocks = (unsigned)cdiv((int)((int64_t)a.num_seqs * a.num_q_heads), 4);
    if (a.stream_waves > 0 && px) {
        hipLaunchKernelGGL((decode_stream_reduce_kernel<T, D, true>), dim3(blocks), dim3(256), 0,
                           stream, (T *)a.out, a.ws_scan, a.num_seqs, a.num_q_heads,
                           a.num_kv_heads, a.stream_waves, a.ws_o, a.ws_ml, px->x_o, px->x_ml,
                           px->ksplit);
    } else if (a.stream_waves > 0) {
        hipLaunchKernelGGL((decode_stream_reduce_kernel<T, D, false>), dim3(blocks), dim3(256), 0,
                           stream, (T *)a.out, a.ws_scan, a.num_seqs, a.num_q_heads,
                           a.num_kv_heads, a.stream_waves, a.ws_o, a.ws_ml, nullptr, nullptr, 0);
    } else {
        hipLaunchKernelGGL((decode_reduce_kernel<T, D>), dim3(blocks), dim3(256), 0, stream,
                           (T *)a.out, a.context_lens, a.num_seqs, a.num_q_heads, max_tokens(a),
                           a.partition_size, a.num_partitions, a.ws_o, a.ws_ml);
    }
    return hipGetLastError();
}

hipError_t launch_decode_reduce(const DecodeArgs &a, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    if (a.stream_waves > 0 && a.pairs) return hipSuccess;  // every pair finished by its wave
    if (a.dtype == 1)
        return a.head_dim == 64 ? launch_red<bf16_t, 64>(a, stream)
                                : launch_red<bf16_t, 128>(a, stream);
    return a.head_dim == 64 ? launch_red<float, 64>(a, stream) : launch_red<float, 128>(a, stream);
}


// ---- shared prefix --------------------------------------------------------

// Waves the prefix pass aims for: the splits of the prefix grow until the
// (kv head, column group) pairs times the splits reach one wave per SIMD.
// (Two or eight splits on the 128-sequence, 1,024-token prefix took longer.)
constexpr int kPrefixWaves = 1024;

static int64_t cdiv_i64(int64_t a, int64_t b) { return (a + b - 1) / b; }

int prefix_splits(int num_seqs, int num_q_heads, int num_kv_heads, int prefix_tokens) {
    const int G = num_q_heads / num_kv_heads;
    const int64_t ncg = cdiv(num_seqs, 16 / G);
    const int64_t units = cdiv(prefix_tokens, kUnitTokens);
    int64_t k = cdiv_i64(kPrefixWaves, (int64_t)num_kv_heads * ncg);
    if (k > kPrefixMaxSplits) k = kPrefixMaxSplits;
    if (k > units) k = units;
    return k < 1 ? 1 : (int)k;
}

template <int D, int B, int G>
static hipError_t launch_prefix_as(const DecodeArgs &a, const PrefixArgs &p, hipStream_t stream) {
    const int64_t waves = (int64_t)a.num_kv_heads * cdiv(a.num_seqs, 16 / G) * p.ksplit;
    if (a.kv_fp8) {
        hipLaunchKernelGGL((decode_prefix_fp8_kernel<D, B, G, kMmaWaves>),
                           dim3((unsigned)cdiv_i64(waves, kMmaWaves)), dim3(kMmaWaves * 64), 0,
                           stream, (const bf16_t *)a.query, (const uint8_t *)a.key_cache,
                           (const uint8_t *)a.value_cache, p.prefix_table, a.context_lens,
                           a.num_seqs, a.num_q_heads, a.num_kv_heads, a.num_blocks,
                           p.prefix_tokens, p.ksplit, a.scale * kLog2e * a.k_scale, a.v_scale,
                           p.x_o, p.x_ml);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((decode_prefix_mma_kernel<D, B, G, kMmaWaves>),
                       dim3((unsigned)cdiv_i64(waves, kMmaWaves)), dim3(kMmaWaves * 64), 0, stream,
                       (const bf16_t *)a.query, (const bf16_t *)a.key_cache,
                       (const bf16_t *)a.value_cache, p.prefix_table, a.context_lens, a.num_seqs,
                       a.num_q_heads, a.num_kv_heads, a.num_blocks, p.prefix_tokens, p.ksplit,
                       a.scale * kLog2e, p.x_o, p.x_ml);
    return hipGetLastError();
}

template <int D, int B>
static hipError_t prefix_by_group(const DecodeArgs &a, const PrefixArgs &p, hipStream_t stream) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_prefix_as<D, B, 1>(a, p, stream);
        case 2: return launch_prefix_as<D, B, 2>(a, p, stream);
        case 4: return launch_prefix_as<D, B, 4>(a, p, stream);
        case 8: return launch_prefix_as<D, B, 8>(a, p, stream);
    }
    return hipErrorNotSupported;
}

hipError_t launch_decode_prefix(const DecodeArgs &a, const PrefixArgs &p, hipStream_t stream) {
    if (a.num_seqs == 0 || p.prefix_tokens == 0) return hipSuccess;
    if (a.dtype != 1) return hipErrorNotSupported;
    if (a.head_dim == 64)
        return a.block_size == 16 ? prefix_by_group<64, 16>(a, p, stream)
                                  : prefix_by_group<64, 32>(a, p, stream);
    return a.block_size == 16 ? prefix_by_group<128, 16>(a, p, stream)
                              : prefix_by_group<128, 32>(a, p, stream);
}

template <int D, int B, int G>
static hipError_t launch_suffix_fp8(const DecodeArgs &a, int len_skip, hipStream_t stream) {
    launch_stream_fp8_as<D, B, G, false>(a, stream, len_skip, 1);
    return hipGetLastError();
}

template <int D, int B>
static hipError_t suffix_by_group(const DecodeArgs &a, int len_skip, hipStream_t stream) {
    if (a.kv_fp8) {
        switch (a.num_q_heads / a.num_kv_heads) {
            case 1: return launch_suffix_fp8<D, B, 1>(a, len_skip, stream);
            case 2: return launch_suffix_fp8<D, B, 2>(a, len_skip, stream);
            case 4: return launch_suffix_fp8<D, B, 4>(a, len_skip, stream);
            case 8: return launch_suffix_fp8<D, B, 8>(a, len_skip, stream);
        }
        return hipErrorNotSupported;
    }
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_stream_mma<D, B, 1>(a, stream, len_skip, 1);
        case 2: return launch_stream_mma<D, B, 2>(a, stream, len_skip, 1);
        case 4: return launch_stream_mma<D, B, 4>(a, stream, len_skip, 1);
        case 8: return launch_stream_mma<D, B, 8>(a, stream, len_skip, 1);
    }
    return hipErrorNotSupported;
}

hipError_t launch_decode_suffix(const DecodeArgs &a, int len_skip, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    if (a.dtype != 1 || a.stream_waves == 0 || a.new_key) return hipErrorNotSupported;
    if (a.head_dim == 64)
        return a.block_size == 16 ? suffix_by_group<64, 16>(a, len_skip, stream)
                                  : suffix_by_group<64, 32>(a, len_skip, stream);
    return a.block_size == 16 ? suffix_by_group<128, 16>(a, len_skip, stream)
                              : suffix_by_group<128, 32>(a, len_skip, stream);
}

hipError_t launch_decode_reduce_prefix(const DecodeArgs &a, const PrefixArgs &p,
                                       hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    if (a.dtype != 1 || a.stream_waves == 0) return hipErrorNotSupported;
    return a.head_dim == 64 ? launch_red<bf16_t, 64>(a, stream, &p)
                            : launch_red<bf16_t, 128>(a, stream, &p);
}

}  // namespace pa
