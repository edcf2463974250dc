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
// Tiling.  A workgroup of 8 waves owns one (chunk, kv head, tile of QT
// queries); its 128 rows are the QT queries x G = Hq / Hkv heads that share
// the kv head, so every K/V block brought into LDS serves all of them.  The
// waves form 4 row groups of 32 rows x 2 key parities: even and odd 64-key
// blocks sit in LDS together and each is read by the 4 waves of its parity
// (half the LDS traffic per matrix product of 8 waves sharing one block),
// while two waves per SIMD still overlap one another's softmax and loads.
// The two parities' partial softmax states are merged once at the end.  Keys advance in blocks of 64 (four 16-token or two
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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 8
#endif
constexpr int kPfWaves = PA_PREFILL_WAVES;  // waves per workgroup (2 per SIMD at 8)
constexpr int kPfRows = 128;        // rows (query x head) per workgroup
constexpr int kKeyBlock = 64;       // keys per LDS block
constexpr int kXcds = 8;            // MI355X: 8 accelerator complex dies, one L2 each
constexpr float kPfRescale = 8.0f;  // log2 units
constexpr int kBtCache = 2048;      // block-table entries a tile keeps in LDS

template <typename A, typename Bv>
__device__ __forceinline__ floatx4_v mfma16x16x32(const A &a, const Bv &b, floatx4_v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, a),
                                                   __builtin_bit_cast(bf16x8_v, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    floatx2_v f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_v2));
}

// Staging of one 64-key block from the paged pools into LDS.
//   K: each thread moves KPT 16-byte chunks; a wave covers whole 256-byte
//      rows, so the global reads are contiguous.
//   V: each thread moves one 16-byte chunk of two consecutive keys and
//      transposes them in registers (v_perm), so V^T is written one word (2
//      keys of one dim) at a time.
// The data are fetched into registers one block pair ahead of their use.
template <int D, int B>
struct KVStage {
    static constexpr int NCH = D * 2 / 16;
    static constexpr int KPT = kKeyBlock * NCH / (kPfWaves * 64);  // 1 or 2
    // V: keys per thread, so that the threads cover 64 keys x NCH chunks once
    static constexpr int VK = kKeyBlock * NCH / (kPfWaves * 64);     // 1 or 2
    static constexpr int KPAD = D + 8;
    static constexpr int VPAD = kKeyBlock + 4;
    static_assert(KPT == 1 || KPT == 2, "K chunks per thread");
    static_assert(VK == 1 || VK == 2, "V keys per thread");
    int k_lds0, k_lds1;        // LDS element offsets of this thread's K chunks
    int k_off0, k_off1;        // element offsets inside a page
    int k_pg0, k_pg1;          // page index inside the block
    int v_pg, v_off, v_lds;    // V: page in block, offset in page, LDS position
    int vkey;                  // first of this thread's two V keys in the block
    u32x4 k0, k1, v0, v1;      // native vectors: plain loads/stores, no memcpy

    __device__ __forceinline__ void init(int tid, int g) {
        const int ci0 = tid, ci1 = tid + kPfWaves * 64;
        const int kk0 = ci0 / NCH, ch0 = ci0 - kk0 * NCH;
        const int kk1 = ci1 / NCH, ch1 = ci1 - kk1 * NCH;
        k_lds0 = kk0 * KPAD + ch0 * 8;
        k_lds1 = kk1 * KPAD + ch1 * 8;
        k_pg0 = kk0 / B;
        k_pg1 = kk1 / B;
        k_off0 = g * B * D + (kk0 % B) * D + ch0 * 8;
        k_off1 = g * B * D + (kk1 % B) * D + ch1 * 8;
        // V: thread (vkg, vc) moves chunk vc of keys VK*vkg .. VK*vkg + VK-1
        const int vkg = tid % (kKeyBlock / VK), vc = tid / (kKeyBlock / VK);
        vkey = VK * vkg;
        v_pg = vkey / B;
        v_off = g * B * D + (vkey % B) * D + vc * 8;
        v_lds = vc * 8 * VPAD + vkey;
    }
    // Pages past the tile's keys and entries outside the pool (a caller error)
    // read block 0 harmlessly; keys past the end are masked and their values
    // zeroed in stash().
    static __device__ __forceinline__ int64_t page_base(int phys, int64_t num_blocks,
                                                        int64_t block_elems) {
        return (phys >= 0 && (int64_t)phys < num_blocks) ? (int64_t)phys * block_elems : 0;
    }
    // Block-table entries come from the tile's LDS window, which holds the
    // entries from page win_p0 on (index clamped to the tile's last page).
    static __device__ __forceinline__ int page(int idx, const int *bt_s, int win_p0, int nbt) {
        return bt_s[(idx < nbt ? idx : nbt - 1) - win_p0];
    }
    __device__ __forceinline__ void fetch(int key0, const int *bt_s, int win_p0, int nbt,
                                          const bf16_t *key_cache, const bf16_t *value_cache,
                                          int64_t block_elems, int64_t num_blocks) {
        const int pg0 = key0 / B;
        const int64_t kb0 = page_base(page(pg0 + k_pg0, bt_s, win_p0, nbt), num_blocks, block_elems);
        k0 = *(const u32x4 *)(key_cache + kb0 + k_off0);
        if (KPT > 1) {
            const int64_t kb1 =
                page_base(page(pg0 + k_pg1, bt_s, win_p0, nbt), num_blocks, block_elems);
            k1 = *(const u32x4 *)(key_cache + kb1 + k_off1);
        }
        const int64_t vb = page_base(page(pg0 + v_pg, bt_s, win_p0, nbt), num_blocks, block_elems);
        const u32x4 *vsrc = (const u32x4 *)(value_cache + vb + v_off);
        v0 = vsrc[0];
        if (VK > 1) v1 = vsrc[D / 8];
    }
    // K rows as they are; V transposed: the 8 dims of the two keys become 8
    // LDS words, each holding one dim of both keys (v_perm packs the halves).
    __device__ __forceinline__ void stash(bf16_t *Ks, bf16_t *Vt, int key0, int kend) {
        *(u32x4 *)(&Ks[k_lds0]) = k0;
        if (KPT > 1) *(u32x4 *)(&Ks[k_lds1]) = k1;
        if (key0 + kKeyBlock > kend) {  // last block: values past the end read as 0
            if (key0 + vkey >= kend) v0 = u32x4{0, 0, 0, 0};
            if (VK > 1 && key0 + vkey + 1 >= kend) v1 = u32x4{0, 0, 0, 0};
        }
        if (VK > 1) {
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
                *(uint32_t *)(&Vt[v_lds + 2 * w2 * VPAD]) =
                    __builtin_amdgcn_perm(v1[w2], v0[w2], 0x05040100u);
                *(uint32_t *)(&Vt[v_lds + (2 * w2 + 1) * VPAD]) =
                    __builtin_amdgcn_perm(v1[w2], v0[w2], 0x07060302u);
            }
        } else {
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
                Vt[v_lds + 2 * w2 * VPAD] = (bf16_t)(v0[w2] & 0xffffu);
                Vt[v_lds + (2 * w2 + 1) * VPAD] = (bf16_t)(v0[w2] >> 16);
            }
        }
    }
};

template <int D, int B, int G>
__global__ __launch_bounds__(kPfWaves * 64) void prefill_chunk_kernel(
    bf16_t *__restrict__ out, const bf16_t *__restrict__ query,
    const bf16_t *__restrict__ key_cache, const bf16_t *__restrict__ value_cache,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ cu_query_lens,
    const int32_t *__restrict__ context_lens, int num_q_heads, int num_kv_heads, int max_blocks,
    int64_t num_blocks, float scale_log2, int num_tiles, int total) {
    constexpr int QT = kPfRows / G;            // queries per tile
    constexpr int KS = D / 32;                 // k-steps of S^T = K Q^T
    constexpr int DT = D / 16;                 // 16-dim tiles of O^T
    constexpr int RT = 2;                      // 16-row tiles per wave (32 rows)
    constexpr int KPAD = KVStage<D, B>::KPAD;  // K row stride in LDS (elements, +16 bytes)
    constexpr int VPAD = KVStage<D, B>::VPAD;  // V^T row stride: 34 dwords, so 16 rows
                                               // read 8 bytes each hit 32 distinct banks
    constexpr int KS_ELEMS = kKeyBlock * KPAD, VT_ELEMS = D * VPAD;
    constexpr float NEG_INF = -__builtin_inff();
    static_assert(kPfWaves == 8 && kPfRows == 4 * RT * 16, "4 row groups x 2 key parities");

    // Two key blocks resident at once (even and odd); the same memory holds the
    // partial results of the odd waves for the final merge.
    constexpr int STAGE_BYTES = 2 * (KS_ELEMS + VT_ELEMS) * 2;
    constexpr int MERGE_BYTES = 4 * 64 * (DT * RT * 4 + 2 * RT) * 4;
    __shared__ __attribute__((aligned(16))) char smem[STAGE_BYTES > MERGE_BYTES ? STAGE_BYTES
                                                                                : MERGE_BYTES];
    bf16_t *const lds = (bf16_t *)smem;  // [K even][K odd][V^T even][V^T odd]

    // Workgroups are dispatched round-robin over the 8 XCDs (each with its own
    // L2).  Renumber them so that the tiles of one (chunk, kv head), which
    // read the same keys and values, run on the same XCD.
    const int bid = blockIdx.x;
    const int xcd = bid % kXcds, idx = bid / kXcds;
    const int q8 = total / kXcds, rem = total % kXcds;
    const int lin = xcd < rem ? xcd * (q8 + 1) + idx : rem * (q8 + 1) + (xcd - rem) * q8 + idx;
    const int pair = lin / num_tiles, tile = lin - pair * num_tiles;
    const int c = pair / num_kv_heads, g = pair - c * num_kv_heads;
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
    const int rg = w & 3, kp = w >> 2;  // row group, key parity

    // ---- this lane's rows and their Q^T operands ----------------------------
    // Row r (0..127) of the tile = query r / G, head r % G of the group.
    int row_pos[RT];
    bool row_ok[RT];
    u32x4 qf[RT][KS];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = (rg * RT + rt) * 16 + l16;
        const int qi = r / G, hh = r - qi * G;
        row_ok[rt] = qi < nq;
        const int qc = row_ok[rt] ? qi : nq - 1;          // clamp reads of padding rows
        row_pos[rt] = pos0 + qc;
        const bf16_t *qrow = query + ((int64_t)(q_begin + q0 + qc) * num_q_heads + g * G + hh) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[rt][ks] = *(const u32x4 *)(qrow + ks * 32 + lg * 8);
    }

    floatx4_v acc_o[DT][RT];
    floatx4_v acc_l[RT];  // row sums: element 0 of lanes 0..15 (row = lane)
    float m_row[RT];
    // A operand whose row 0 is all ones (bf16 1.0) and rows 1..15 zero.
    const u32x4 ones_row = l16 == 0 ? u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u}
                                    : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        m_row[rt] = NEG_INF;
        acc_l[rt] = floatx4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc_o[dt][rt] = floatx4_v{0.f, 0.f, 0.f, 0.f};
    }

    const int64_t head_elems = (int64_t)B * D;
    const int64_t block_elems = head_elems * num_kv_heads;
    const int nkb = cdiv(kend, kKeyBlock);
    const int nbt = cdiv(kend, B);  // pages the tile reads

    // One 64-key block of this wave's parity: S^T = K Q^T, online softmax,
    // O^T += V^T P^T.
    auto compute = [&](const bf16_t *Kb, const bf16_t *Vb, int key0) __attribute__((always_inline)) {
        floatx4_v s[4][RT];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            u32x4 kf[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kf[ks] = *(const u32x4 *)(&Kb[(kt * 16 + l16) * KPAD + ks * 32 + lg * 8]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                floatx4_v a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) a = mfma16x16x32(kf[ks], qf[rt][ks], a);
                s[kt][rt] = a;
            }
        }
        // Causal mask: only blocks that reach past the tile's first position
        // need it (a uniform branch).  Masked logits are -inf, never scaled.
        if (key0 + kKeyBlock - 1 > pos0) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (key0 + kt * 16 + lg * 4 + i > row_pos[rt]) s[kt][rt][i] = NEG_INF;
        }
        u32x4 pf[RT][2];  // P^T operands: [rt][32-key half]
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            // Row maximum over this block (lanes l, l+16, l+32, l+48 share a row).
            float mx = NEG_INF;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
                mx = fmaxf(mx, fmaxf(fmaxf(s[kt][rt][0], s[kt][rt][1]),
                                     fmaxf(s[kt][rt][2], s[kt][rt][3])));
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            // The reference maximum m_row (log2 units) is raised only when a
            // logit exceeds it by more than kPfRescale, so the rescale of the
            // accumulators is rare; weights stay below 2^kPfRescale.
            const float cand = mx * scale_log2;
            if (__builtin_amdgcn_ballot_w64(cand > m_row[rt] + kPfRescale)) {
                const float mn = fmaxf(m_row[rt], cand);
                const float alpha = (m_row[rt] == NEG_INF) ? 0.f : fast_exp2(m_row[rt] - mn);
                m_row[rt] = mn;
                acc_l[rt] *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc_o[dt][rt] *= alpha;
            }
            const float mneg = (m_row[rt] == NEG_INF) ? 0.f : -m_row[rt];
            float p[4][4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) p[kt][i] = fast_exp2(fmaf(s[kt][rt][i], scale_log2, mneg));
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                pf[rt][h][0] = pack_bf16x2(p[2 * h][0], p[2 * h][1]);
                pf[rt][h][1] = pack_bf16x2(p[2 * h][2], p[2 * h][3]);
                pf[rt][h][2] = pack_bf16x2(p[2 * h + 1][0], p[2 * h + 1][1]);
                pf[rt][h][3] = pack_bf16x2(p[2 * h + 1][2], p[2 * h + 1][3]);
            }
            // Row sums on the matrix core: a ones row against the same bf16
            // P^T the output uses, so numerator and denominator agree.
#pragma unroll
            for (int h = 0; h < 2; ++h) acc_l[rt] = mfma16x16x32(ones_row, pf[rt][h], acc_l[rt]);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bf16_t *vrow = &Vb[(dt * 16 + l16) * VPAD + h * 32 + lg * 4];
                const uint2 lo = *(const uint2 *)(vrow);
                const uint2 hi = *(const uint2 *)(vrow + 16);
                const u32x4 vf = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    acc_o[dt][rt] = mfma16x16x32(vf, pf[rt][h], acc_o[dt][rt]);
            }
        }
    };

    // Blocks go in pairs: stage 0 holds the even block, stage 1 the odd one.
    // Each stage's next block is fetched while the current pair is multiplied.
    KVStage<D, B> st0, st1;
    st0.init(tid, g);
    st1.init(tid, g);
    // Page lookups read an LDS window of the block table, so that they never
    // wait on global loads queued behind the K/V prefetch.  A window covers
    // kWinBlocks key blocks plus the two the pipeline fetches ahead; it is
    // refilled (rarely: every 32K keys at 16-token pages) at the top of an
    // iteration, where the stash waits for all loads anyway.
    constexpr int kWinBlocks = kBtCache * B / kKeyBlock - 2;
    static_assert(kWinBlocks > 0 && kWinBlocks % 2 == 0, "window steps by block pairs");
    __shared__ int bt_s[kBtCache];
    int win_p0 = 0, next_win = kWinBlocks;
    auto load_window = [&](int kb0) __attribute__((always_inline)) {
        win_p0 = kb0 * (kKeyBlock / B);
        const int n = min(nbt - win_p0, kBtCache);
        for (int i = tid; i < n; i += kPfWaves * 64) bt_s[i] = bt[win_p0 + i];
    };
    load_window(0);
    __syncthreads();
    if (nkb > 0)
        st0.fetch(0, bt_s, win_p0, nbt, key_cache, value_cache, block_elems, num_blocks);
    if (nkb > 1)
        st1.fetch(kKeyBlock, bt_s, win_p0, nbt, key_cache, value_cache, block_elems,
                  num_blocks);
    for (int kb = 0; kb < nkb; kb += 2) {
        const int key0 = kb * kKeyBlock;
        if (kb == next_win) {  // every thread's fetch from the old window is issued
            load_window(kb);
            next_win += kWinBlocks;
        }
        st0.stash(lds, lds + 2 * KS_ELEMS, key0, kend);
        if (kb + 1 < nkb)
            st1.stash(lds + KS_ELEMS, lds + 2 * KS_ELEMS + VT_ELEMS, key0 + kKeyBlock, kend);
        __syncthreads();
        if (kb + 2 < nkb)
            st0.fetch(key0 + 2 * kKeyBlock, bt_s, win_p0, nbt, key_cache, value_cache, block_elems,
                      num_blocks);
        if (kb + 3 < nkb)
            st1.fetch(key0 + 3 * kKeyBlock, bt_s, win_p0, nbt, key_cache, value_cache, block_elems,
                      num_blocks);
        if (kb + kp < nkb)
            compute(lds + kp * KS_ELEMS, lds + 2 * KS_ELEMS + kp * VT_ELEMS, key0 + kp * kKeyBlock);
        __syncthreads();
    }

    // ---- merge the two key parities, normalise, store ------------------------
    // Each lane of an odd wave hands its (max, sum, O^T fragment) to the lane
    // of the even wave with the same rows; both use the same lane layout.
    float *mo = (float *)smem + (size_t)rg * 64 * (DT * RT * 4 + 2 * RT);
    float *my = mo + lane * (DT * RT * 4 + 2 * RT);
    float lsum[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) lsum[rt] = __shfl(acc_l[rt][0], l16);  // row l16's sum
    if (kp == 1) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                *(floatx4_v *)(my + (rt * DT + dt) * 4) = acc_o[dt][rt];
            my[DT * RT * 4 + 2 * rt] = m_row[rt];
            my[DT * RT * 4 + 2 * rt + 1] = lsum[rt];
        }
    }
    __syncthreads();
    if (kp == 1) return;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const float m1 = my[DT * RT * 4 + 2 * rt], l1 = my[DT * RT * 4 + 2 * rt + 1];
        const float M = fmaxf(m_row[rt], m1);
        const float f0 = (m_row[rt] == NEG_INF) ? 0.f : fast_exp2(m_row[rt] - M);
        const float f1 = (m1 == NEG_INF) ? 0.f : fast_exp2(m1 - M);
        const float l = lsum[rt] * f0 + l1 * f1;
        if (!row_ok[rt]) continue;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int r = (rg * RT + rt) * 16 + l16;
        const int qi = r / G, hh = r - qi * G;
        bf16_t *orow = out + ((int64_t)(q_begin + q0 + qi) * num_q_heads + g * G + hh) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const floatx4_v o1 = *(const floatx4_v *)(my + (rt * DT + dt) * 4);
            const floatx4_v o = (acc_o[dt][rt] * f0 + o1 * f1) * inv;
            uint2 v;
            v.x = pack_bf16x2(o[0], o[1]);
            v.y = pack_bf16x2(o[2], o[3]);
            *(uint2 *)(orow + dt * 16 + lg * 4) = v;
        }
    }
}

template <int D, int B, int G>
static hipError_t launch(const PrefillArgs &a, hipStream_t stream) {
    constexpr int QT = kPfRows / G;
    const int tiles = cdiv(a.max_query_len, QT);
    const int64_t total = (int64_t)tiles * a.num_kv_heads * a.num_chunks;
    if (total > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prefill_chunk_kernel<D, B, G>), dim3((unsigned)total), dim3(kPfWaves * 64),
                       0, stream, (bf16_t *)a.out, (const bf16_t *)a.query,
                       (const bf16_t *)a.key_cache, (const bf16_t *)a.value_cache, a.block_tables,
                       a.cu_query_lens, a.context_lens, a.num_q_heads, a.num_kv_heads,
                       a.max_blocks_per_seq, a.num_blocks, a.scale * kLog2e, tiles, (int)total);
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
