// Chunked-prefill attention over a paged KV cache on gfx950 matrix cores.
//
// A long prompt is processed in chunks (e.g. 512 tokens) that ride along with
// decode steps; each chunk's queries attend causally to everything already in
// the cache plus the chunk itself ("Configuring vLLM and PagedAttention for
// High Throughput Enterprise LLM Serving", section "High-Throughput Batching:
// Continuous Batching & Chunked Prefill").  Unlike decode this is a dense
// contraction with high arithmetic intensity (same page, section "Memory
// Bottlenecks in Autoregressive LLM Inference": prefill is compute-bound), so
// both products run on bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulate)
// and the softmax runs online in fp32 (tiled attention, Dao et al. 2022;
// online normaliser, Milakov & Gimelshein 2018).
//
// Tiling.  A workgroup of 4 waves owns one (chunk, kv head, tile of QT
// queries); its 128 rows are the QT queries x G = Hq / Hkv heads that share
// the kv head, so every K/V block brought into LDS serves all of them.  Each
// wave owns 32 rows.  Keys advance in blocks of 64 (four 16-token or two
// 32-token pages), gathered through the block table into LDS: K as [key][dim]
// (row padded by 16 bytes), V transposed to [dim][key] so that the PV operand
// of a lane is a run of consecutive keys.
//
// The products are computed transposed, S^T = K Q^T and O^T = V^T P^T: the
// fp32 S^T tile a lane holds (4 consecutive keys of one row) is, after
// conversion to bf16, exactly the P^T operand the next MFMA needs (the keys of
// the contraction are visited in a fixed permutation shared by both
// operands), so P never goes through LDS.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_v2 __attribute__((ext_vector_type(2)));
typedef float floatx4_v __attribute__((ext_vector_type(4)));
typedef float floatx2_v __attribute__((ext_vector_type(2)));

constexpr int kPfWaves = 4;
constexpr int kPfRows = 128;        // rows (query x head) per workgroup
constexpr int kKeyBlock = 64;       // keys per LDS block

__device__ __forceinline__ floatx4_v mfma16x16x32(const uint4 &a, const uint4 &b, floatx4_v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, a),
                                                   __builtin_bit_cast(bf16x8_v, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    floatx2_v f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_v2));
}

template <int D, int B, int G>
__global__ __launch_bounds__(kPfWaves * 64) void prefill_chunk_kernel(
    bf16_t *__restrict__ out, const bf16_t *__restrict__ query,
    const bf16_t *__restrict__ key_cache, const bf16_t *__restrict__ value_cache,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ cu_query_lens,
    const int32_t *__restrict__ context_lens, int num_q_heads, int num_kv_heads, int max_blocks,
    int64_t num_blocks, float scale_log2) {
    constexpr int QT = kPfRows / G;           // queries per tile
    constexpr int NCH = D * 2 / 16;           // 16-byte chunks per K/V row
    constexpr int KS = D / 32;                // k-steps of S^T = K Q^T
    constexpr int DT = D / 16;                // 16-dim tiles of O^T
    constexpr int KPAD = D + 8;               // K row stride in LDS (elements)
    constexpr int VPAD = kKeyBlock + 8;       // V^T row stride in LDS (elements)
    constexpr float NEG_INF = -__builtin_inff();

    __shared__ __attribute__((aligned(16))) bf16_t Ks[kKeyBlock * KPAD];
    __shared__ __attribute__((aligned(16))) bf16_t Vt[D * VPAD];

    const int tile = blockIdx.x, g = blockIdx.y, c = blockIdx.z;
    const int q_begin = cu_query_lens[c];
    const int n = cu_query_lens[c + 1] - q_begin;
    const int q0 = tile * QT;
    if (q0 >= n) return;
    const int max_tokens = max_blocks * B;
    int L = context_lens[c];
    L = L < 0 ? 0 : (L > max_tokens ? max_tokens : L);
    const int nq = min(QT, n - q0);                 // valid queries in this tile
    const int pos0 = L - n + q0;                    // position of the tile's first query
    const int kend = min(L, pos0 + nq);             // keys any row of the tile may see
    const int32_t *bt = block_tables + (int64_t)c * max_blocks;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;

    // ---- this lane's rows and their Q^T operands ----------------------------
    // Row r (0..127) of the tile = query r / G, head r % G of the group.
    int row_pos[2];
    bool row_ok[2];
    uint4 qf[2][KS];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int r = w * 32 + rt * 16 + l16;
        const int qi = r / G, hh = r - qi * G;
        row_ok[rt] = qi < nq;
        const int qc = row_ok[rt] ? qi : nq - 1;          // clamp reads of padding rows
        row_pos[rt] = pos0 + qc;
        const bf16_t *qrow = query + ((int64_t)(q_begin + q0 + qc) * num_q_heads + g * G + hh) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[rt][ks] = *(const uint4 *)(qrow + ks * 32 + lg * 8);
    }

    floatx4_v acc_o[DT][2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) acc_o[dt][rt] = floatx4_v{0.f, 0.f, 0.f, 0.f};
    float m_row[2] = {NEG_INF, NEG_INF};
    float l_part[2] = {0.f, 0.f};  // this lane's share of the row sum

    const int64_t head_elems = (int64_t)B * D;
    const int64_t block_elems = head_elems * num_kv_heads;
    const int nkb = cdiv(kend, kKeyBlock);

    for (int kb = 0; kb < nkb; ++kb) {
        const int key0 = kb * kKeyBlock;
        // ---- gather K and V of 64 keys into LDS ------------------------------
#pragma unroll
        for (int i = 0; i < kKeyBlock * NCH / (kPfWaves * 64); ++i) {
            const int ci = tid + i * kPfWaves * 64;
            const int kk = ci / NCH, ch = ci - kk * NCH;
            const int j = key0 + kk;
            uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
            if (j < kend) {
                const int phys = bt[j / B];
                if (phys >= 0 && (int64_t)phys < num_blocks) {
                    const int64_t off = (int64_t)phys * block_elems + g * head_elems +
                                        (j % B) * D + ch * 8;
                    kv = *(const uint4 *)(key_cache + off);
                    vv = *(const uint4 *)(value_cache + off);
                }
            }
            *(uint4 *)(&Ks[kk * KPAD + ch * 8]) = kv;
            const bf16_t *ve = (const bf16_t *)&vv;
#pragma unroll
            for (int e = 0; e < 8; ++e) Vt[(ch * 8 + e) * VPAD + kk] = ve[e];
        }
        __syncthreads();

        // ---- S^T = K Q^T for 64 keys x this wave's 32 rows -------------------
        floatx4_v s[4][2];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            uint4 kf[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kf[ks] = *(const uint4 *)(&Ks[(kt * 16 + l16) * KPAD + ks * 32 + lg * 8]);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                floatx4_v a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) a = mfma16x16x32(kf[ks], qf[rt][ks], a);
                s[kt][rt] = a;
            }
        }

        // ---- online softmax (base 2), causal mask on the key index -----------
        uint4 pf[2][2];  // P^T operands: [rt][32-key half]
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            float mx = NEG_INF;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int j = key0 + kt * 16 + lg * 4 + i;
                    float x = s[kt][rt][i] * scale_log2;
                    x = (j <= row_pos[rt]) ? x : NEG_INF;
                    s[kt][rt][i] = x;
                    mx = fmaxf(mx, x);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mn = fmaxf(m_row[rt], mx);
            const float alpha = (m_row[rt] == NEG_INF) ? 0.f : fast_exp2(m_row[rt] - mn);
            const float mref = (mn == NEG_INF) ? 0.f : mn;
            m_row[rt] = mn;
            float psum = 0.f;
            float p[4][4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[kt][i] = fast_exp2(s[kt][rt][i] - mref);
                    psum += p[kt][i];
                }
            l_part[rt] = l_part[rt] * alpha + psum;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc_o[dt][rt] *= alpha;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                pf[rt][h].x = pack_bf16x2(p[2 * h][0], p[2 * h][1]);
                pf[rt][h].y = pack_bf16x2(p[2 * h][2], p[2 * h][3]);
                pf[rt][h].z = pack_bf16x2(p[2 * h + 1][0], p[2 * h + 1][1]);
                pf[rt][h].w = pack_bf16x2(p[2 * h + 1][2], p[2 * h + 1][3]);
            }
        }

        // ---- O^T += V^T P^T --------------------------------------------------
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bf16_t *vrow = &Vt[(dt * 16 + l16) * VPAD + h * 32 + lg * 4];
                const uint2 lo = *(const uint2 *)(vrow);
                const uint2 hi = *(const uint2 *)(vrow + 16);
                const uint4 vf = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) acc_o[dt][rt] = mfma16x16x32(vf, pf[rt][h], acc_o[dt][rt]);
            }
        }
        __syncthreads();
    }

    // ---- normalise and store: lane holds O^T[4 dims][one row] per tile -------
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        float lsum = l_part[rt];
        lsum += __shfl_xor(lsum, 16);
        lsum += __shfl_xor(lsum, 32);
        if (!row_ok[rt]) continue;
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        const int r = w * 32 + rt * 16 + l16;
        const int qi = r / G, hh = r - qi * G;
        bf16_t *orow = out + ((int64_t)(q_begin + q0 + qi) * num_q_heads + g * G + hh) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            uint2 v;
            v.x = pack_bf16x2(acc_o[dt][rt][0] * inv, acc_o[dt][rt][1] * inv);
            v.y = pack_bf16x2(acc_o[dt][rt][2] * inv, acc_o[dt][rt][3] * inv);
            *(uint2 *)(orow + dt * 16 + lg * 4) = v;
        }
    }
}

template <int D, int B, int G>
static hipError_t launch(const PrefillArgs &a, hipStream_t stream) {
    constexpr int QT = kPfRows / G;
    dim3 grid(cdiv(a.max_query_len, QT), a.num_kv_heads, a.num_chunks);
    hipLaunchKernelGGL((prefill_chunk_kernel<D, B, G>), grid, dim3(kPfWaves * 64), 0, stream,
                       (bf16_t *)a.out, (const bf16_t *)a.query, (const bf16_t *)a.key_cache,
                       (const bf16_t *)a.value_cache, a.block_tables, a.cu_query_lens,
                       a.context_lens, a.num_q_heads, a.num_kv_heads, a.max_blocks_per_seq,
                       a.num_blocks, a.scale * kLog2e);
    return hipGetLastError();
}

template <int D, int B>
static hipError_t by_group(const PrefillArgs &a, hipStream_t stream) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch<D, B, 1>(a, stream);
        case 2: return launch<D, B, 2>(a, stream);
        case 4: return launch<D, B, 4>(a, stream);
        case 8: return launch<D, B, 8>(a, stream);
    }
    return hipErrorNotSupported;
}

template <int D>
static hipError_t by_block(const PrefillArgs &a, hipStream_t stream) {
    switch (a.block_size) {
        case 16: return by_group<D, 16>(a, stream);
        case 32: return by_group<D, 32>(a, stream);
    }
    return hipErrorNotSupported;
}

bool prefill_shape_supported(int head_dim, int block_size, int group) {
    return (head_dim == 64 || head_dim == 128) && (block_size == 16 || block_size == 32) &&
           (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_prefill_chunk(const PrefillArgs &a, hipStream_t stream) {
    switch (a.head_dim) {
        case 64: return by_block<64>(a, stream);
        case 128: return by_block<128>(a, stream);
    }
    return hipErrorNotSupported;
}

}  // namespace pa
